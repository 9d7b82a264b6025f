// k_mfma.hip -- bf16 x bf16 -> fp32 join + sum aggregation on the gfx950
// matrix cores (v_mfma_f32_32x32x16_bf16).
//
// Page "EinDecomp：基于爱因斯坦求和与张量关系代数的自动张量并行分解算法",
// section 2.2: when the join is a product and the aggregate a sum, joining a
// key-matched pair of sub-tensors is a small matrix product and the
// aggregation over the contracted keys is a sum of such products.  One
// workgroup owns one output tile of one output sub-tensor group and folds
// every contracted partition into the same fp32 accumulators, contracted keys
// in ascending order, so the per-pair partial products are never written out.
// (The 2.5D SUMMA of the page "ColossalAI 2.5D 张量并行深度解析" is this with
// X cut into (depth*q) x q blocks and A into q x q blocks: each block of Y is
// a sum over q block products, folded here in registers.)
//
// Operands are read in place from their relation layout through per-
// sub-dimension strides.  An operand stored contiguously along the
// contracted labels ("K-major") is staged in LDS as [row][k] and fed to the
// matrix cores with 16-byte LDS reads; one stored contiguously along its
// output labels ("MN-major") is staged as [k][row] and gathered with 16-bit
// LDS reads.
#include <hip/hip_runtime.h>

#include "device_common.h"
#include "plan.h"

namespace tra {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx16_t __attribute__((ext_vector_type(16)));
typedef short shortx8_t __attribute__((ext_vector_type(8)));

struct MfmaCfg {
    int bm, bn, bk, wm, wn;
};
// variant 0: 256x256 tile, 8 waves (2 x 4), wave tile 128x64
// variant 1: 128x128 tile, 4 waves (2 x 2), wave tile 64x64
// variant 2: 64x64 tile, 4 waves (2 x 2), wave tile 32x32
__host__ __device__ constexpr MfmaCfg mfma_cfg(int v)
{
    return v == 0 ? MfmaCfg{256, 256, 64, 2, 4} : v == 1 ? MfmaCfg{128, 128, 64, 2, 2} : MfmaCfg{64, 64, 64, 2, 2};
}

TileShape mfma_tile_shape(int variant)
{
    if (variant < 0 || variant > 2) return {0, 0, 0};
    MfmaCfg c = mfma_cfg(variant);
    return {c.bm, c.bn, c.bk};
}

__device__ __forceinline__ void mfma_tile_of(uint32_t nb, uint32_t tiles_n, uint32_t &tm, uint32_t &tn)
{
    uint32_t b = blockIdx.x;
    if (nb % 8 == 0) b = (b % 8) * (nb / 8) + b / 8;
    const uint32_t G = 4;
    uint32_t tiles_m = nb / tiles_n;
    uint32_t per = G * tiles_n;
    uint32_t g = b / per, first = g * G;
    uint32_t gs = min(tiles_m - first, G);
    uint32_t r = b % per;
    tm = first + r % gs;
    tn = r / gs;
}

template <int V>
constexpr int lds_elems(bool kmajor, bool is_a)
{
    constexpr MfmaCfg c = mfma_cfg(V);
    int rows = is_a ? c.bm : c.bn;
    return kmajor ? rows * (c.bk + 8) : c.bk * (rows + 8);
}

template <int V, bool AK, bool BKM>
constexpr size_t mfma_lds_bytes()
{
    return 2 * (size_t)(lds_elems<V>(AK, true) + lds_elems<V>(BKM, false)) * 2;
}

// Loader for one operand tile (rows x BK) into LDS.
//   KM: operand contiguous along k.  Vectors of 8 bf16 (16 bytes).
template <int ROWS, int BK, int NT, bool KM, int T>
struct TileLoader {
    static constexpr int NV = ROWS * BK / 8 / NT;   // vectors per thread
    static constexpr int LD = KM ? BK + 8 : ROWS + 8;
    int32_t row_off[NV];  // KM: offset of each row; !KM: offset of the 8-row group
    int col[NV];          // KM: k within tile; !KM: k row within tile
    int row[NV];          // KM: row within tile; !KM: first row of the group
    uint4 reg[NV];

    __device__ __forceinline__ void init(const Pow2Group &g_rows, uint32_t r0, int32_t base, int tid)
    {
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            int q = tid + NT * i;
            if constexpr (KM) {
                col[i] = (q % (BK / 8)) * 8;
                row[i] = q / (BK / 8);
            } else {
                row[i] = (q % (ROWS / 8)) * 8;
                col[i] = q / (ROWS / 8);
            }
            row_off[i] = p2off<0>(g_rows, r0 + row[i]) + base;
        }
    }
    __device__ __forceinline__ void load(const uint16_t *__restrict__ p, const Pow2Group &gk, uint32_t k0)
    {
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            int32_t o = row_off[i] + p2off<T>(gk, k0 + col[i]);
            reg[i] = *(const uint4 *)(p + o);
        }
    }
    __device__ __forceinline__ void store(uint16_t *lds)
    {
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            if constexpr (KM) *(uint4 *)&lds[row[i] * LD + col[i]] = reg[i];
            else *(uint4 *)&lds[col[i] * LD + row[i]] = reg[i];
        }
    }
};

// 8 consecutive k of one row r of a staged operand, as an MFMA operand.
template <bool KM, int LD>
__device__ __forceinline__ bf16x8_t frag(const uint16_t *lds, int r, int k)
{
    if constexpr (KM) {
        uint4 u = *(const uint4 *)&lds[r * LD + k];
        return __builtin_bit_cast(bf16x8_t, u);
    } else {
        shortx8_t s;
#pragma unroll
        for (int e = 0; e < 8; ++e) s[e] = (short)lds[(k + e) * LD + r];
        return __builtin_bit_cast(bf16x8_t, s);
    }
}

template <int V, bool AK, bool BKM, typename TO>
__global__ __launch_bounds__(mfma_cfg(V).wm *mfma_cfg(V).wn * 64) void k_mfma_bf16(
    GemmView v, const uint16_t *__restrict__ x, const uint16_t *__restrict__ y, TO *__restrict__ z,
    float *__restrict__ ws)
{
    constexpr MfmaCfg C = mfma_cfg(V);
    constexpr int BM = C.bm, BN = C.bn, BK = C.bk, WM = C.wm, WN = C.wn;
    constexpr int NT = WM * WN * 64;
    constexpr int TM = BM / WM / 32, TN = BN / WN / 32;
    constexpr int A_EL = lds_elems<V>(AK, true), B_EL = lds_elems<V>(BKM, false);
    constexpr int LDA = AK ? BK + 8 : BM + 8, LDB = BKM ? BK + 8 : BN + 8;
    extern __shared__ __attribute__((aligned(16))) uint16_t smem[];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave / WN, wn = wave % WN;
    const uint32_t tiles_n = v.gn.total / BN;
    const uint32_t nb = (v.gm.total / BM) * tiles_n;
    uint32_t tm, tn;
    mfma_tile_of(nb, tiles_n, tm, tn);
    const uint32_t m0 = tm * BM, n0 = tn * BN;
    const uint32_t bidx = blockIdx.y;
    const int32_t bx = p2off<0>(v.gb, bidx), by = p2off<1>(v.gb, bidx), bz = p2off<2>(v.gb, bidx);
    const uint32_t kbeg = blockIdx.z * (uint32_t)v.k_per_split;
    const uint32_t kend = kbeg + (uint32_t)v.k_per_split;

    TileLoader<BM, BK, NT, AK, 0> la;
    TileLoader<BN, BK, NT, BKM, 1> lb;
    la.init(v.gm, m0, bx, tid);
    lb.init(v.gn, n0, by, tid);

    floatx16_t acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

    // stage s: A at s * (A_EL + B_EL), B right after it
    constexpr int STAGE = A_EL + B_EL;

    la.load(x, v.gk, kbeg);
    lb.load(y, v.gk, kbeg);
    la.store(smem);
    lb.store(smem + A_EL);
    __syncthreads();

    const int r_lane = lane & 31, k_lane = (lane >> 5) * 8;
    int stage = 0;
    for (uint32_t k0 = kbeg; k0 < kend; k0 += BK) {
        const bool more = k0 + BK < kend;
        if (more) {
            la.load(x, v.gk, k0 + BK);
            lb.load(y, v.gk, k0 + BK);
        }
        const uint16_t *a_s = smem + stage * STAGE, *b_s = a_s + A_EL;
#pragma unroll
        for (int ks = 0; ks < BK; ks += 16) {
            bf16x8_t af[TM], bf[TN];
#pragma unroll
            for (int i = 0; i < TM; ++i) af[i] = frag<AK, LDA>(a_s, wm * (BM / WM) + i * 32 + r_lane, ks + k_lane);
#pragma unroll
            for (int j = 0; j < TN; ++j) bf[j] = frag<BKM, LDB>(b_s, wn * (BN / WN) + j * 32 + r_lane, ks + k_lane);
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bf[j], acc[i][j], 0, 0, 0);
        }
        if (more) {
            la.store(smem + (stage ^ 1) * STAGE);
            lb.store(smem + (stage ^ 1) * STAGE + A_EL);
        }
        __syncthreads();
        stage ^= 1;
    }

    // Epilogue.  Accumulator element e of lane l holds row
    // 8*(e/4) + 4*(l/32) + e%4 and column l%32 of its 32x32 block.
    const bool split = v.split > 1;
    float *wsp = split ? ws + (int64_t)blockIdx.z * v.z_elems : nullptr;
#pragma unroll
    for (int j = 0; j < TN; ++j) {
        const uint32_t n = n0 + wn * (BN / WN) + j * 32 + r_lane;
        const int32_t on = p2off<1>(v.gn, n) + bz;
#pragma unroll
        for (int i = 0; i < TM; ++i) {
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const uint32_t m = m0 + wm * (BM / WM) + i * 32 + 8 * (e / 4) + 4 * (lane >> 5) + (e % 4);
                const int32_t o = p2off<1>(v.gm, m) + on;
                if (split) wsp[o] = acc[i][j][e];
                else Scalar<TO>::store(z, o, acc[i][j][e] * v.post_scale);
            }
        }
    }
}

int launch_split_fold(const tra_plan_s &p, const void *ws, void *z, void *stream);

template <int V, bool AK, bool BKM, typename TO>
static int launch_v(const tra_plan_s &p, const void *x, const void *y, void *z, void *ws, hipStream_t s)
{
    constexpr MfmaCfg C = mfma_cfg(V);
    constexpr size_t lds = mfma_lds_bytes<V, AK, BKM>();
    static bool attr_set = false;
    if (!attr_set) {
        hipError_t e = hipFuncSetAttribute((const void *)k_mfma_bf16<V, AK, BKM, TO>,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return (int)e;
        attr_set = true;
    }
    const GemmView &v = p.gv;
    dim3 grid((v.gm.total / C.bm) * (v.gn.total / C.bn), v.gb.total, v.split);
    hipLaunchKernelGGL((k_mfma_bf16<V, AK, BKM, TO>), grid, dim3(C.wm * C.wn * 64), lds, s, v,
                       (const uint16_t *)x, (const uint16_t *)y, (TO *)z, (float *)ws);
    return (int)hipGetLastError();
}

template <int V, typename TO>
static int launch_layout(const tra_plan_s &p, const void *x, const void *y, void *z, void *ws, hipStream_t s)
{
    if (p.b_kmajor) return launch_v<V, true, true, TO>(p, x, y, z, ws, s);
    return launch_v<V, true, false, TO>(p, x, y, z, ws, s);
}

template <typename TO>
static int launch_tile(const tra_plan_s &p, const void *x, const void *y, void *z, void *ws, hipStream_t s)
{
    switch (p.tile) {
    case 0: return launch_layout<0, TO>(p, x, y, z, ws, s);
    case 1: return launch_layout<1, TO>(p, x, y, z, ws, s);
    default: return launch_layout<2, TO>(p, x, y, z, ws, s);
    }
}

int launch_mfma_bf16(const tra_plan_s &p, const void *x, const void *y, void *z, void *ws, void *stream)
{
    hipStream_t s = (hipStream_t)stream;
    int err;
    if (p.gv.split > 1 || p.out_dtype == D_F32) err = launch_tile<float>(p, x, y, z, ws, s);
    else err = launch_tile<bf16_t>(p, x, y, z, ws, s);
    if (err || p.gv.split == 1) return err;
    return launch_split_fold(p, ws, z, stream);
}

}  // namespace tra
