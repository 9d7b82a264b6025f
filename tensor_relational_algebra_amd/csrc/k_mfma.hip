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
// output labels ("MN-major") is staged as [k][row] exactly as it arrives and
// transposed on the way to the matrix cores by gfx950's ds_read_b64_tr_b16.
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

// LDS staging.  K-major operand: [rows][BK + 8] (16-byte fragment reads,
// conflict-free with the 144-byte row pitch).  MN-major operand: [BK][rows +
// 32]: rows are written as they arrive from HBM and transposed on the way out
// by ds_read_b64_tr_b16 (the 64-element pad spreads the four k-rows one read
// touches over distinct banks).
template <int V>
constexpr int lds_elems(bool kmajor, bool is_a)
{
    constexpr MfmaCfg c = mfma_cfg(V);
    int rows = is_a ? c.bm : c.bn;
    return kmajor ? rows * (c.bk + 8) : c.bk * (rows + 32);
}

template <int V, bool BKM>
constexpr size_t mfma_lds_bytes()
{
    return 2 * (size_t)(lds_elems<V>(true, true) + lds_elems<V>(BKM, false)) * 2;
}

typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef short shortx4_t __attribute__((ext_vector_type(4)));

// Power-of-two digit layouts split cleanly at aligned boundaries: for r0 a
// multiple of 2^b and d < 2^b, off(r0 + d) = off(r0) + off(d).  So every
// per-thread offset below is computed once, and each k-tile only adds the
// uniform term off(k0).

// Loader for one operand tile (rows x BK) into LDS, 16-byte vectors.
//   KM: operand contiguous along k -> LDS [row][k]; else along rows -> LDS [k][row].
template <int ROWS, int BK, int NT, bool KM, int T>
struct TileLoader {
    static constexpr int NV = ROWS * BK / 8 / NT;   // vectors per thread
    static constexpr int LD = KM ? BK + 8 : ROWS + 32;
    int32_t off[NV];      // row part + in-tile k part of each vector's source offset
    int32_t lds_off[NV];  // destination element offset in the stage
    uint4 reg[NV];

    __device__ __forceinline__ void init(const Pow2Group &g_rows, const Pow2Group &gk, uint32_t r0, int32_t base,
                                         int tid)
    {
        const int32_t rbase = p2off<0>(g_rows, r0) + base;
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            int q = tid + NT * i;
            int row, col;
            if constexpr (KM) {
                col = (q % (BK / 8)) * 8;
                row = q / (BK / 8);
                lds_off[i] = row * LD + col;
            } else {
                row = (q % (ROWS / 8)) * 8;
                col = q / (ROWS / 8);
                lds_off[i] = col * LD + row;
            }
            off[i] = rbase + p2off<0>(g_rows, row) + p2off<T>(gk, col);
        }
    }
    __device__ __forceinline__ void load(const uint16_t *__restrict__ p, int32_t koff)
    {
#pragma unroll
        for (int i = 0; i < NV; ++i) reg[i] = *(const uint4 *)(p + off[i] + koff);
    }
    __device__ __forceinline__ void store(uint16_t *lds)
    {
#pragma unroll
        for (int i = 0; i < NV; ++i) *(uint4 *)&lds[lds_off[i]] = reg[i];
    }
};

// A fragment (K-major staging): 8 consecutive k of row r.
template <int LD>
__device__ __forceinline__ bf16x8_t frag_k(const uint16_t *lds, int r, int k)
{
    uint4 u = *(const uint4 *)&lds[r * LD + k];
    return __builtin_bit_cast(bf16x8_t, u);
}

// B fragment from [k][n] staging via two transposing reads.  Lane l (group
// g = l/16, s = l%16) addresses row kb + s/4, columns nb + 4*(s%4)..+3 with
// kb = k + 8*(g/2), nb = n + 16*(g%2); lane l then holds B[k + 8*(l/32) + e][n + l%32].
template <int LD>
__device__ __forceinline__ bf16x8_t frag_tr(const uint16_t *lds, int n, int k, int lane)
{
    const int g = lane >> 4, sl = lane & 15;
    const int kb = k + 8 * (g >> 1) + (sl >> 2), nb = n + 16 * (g & 1) + 4 * (sl & 3);
    typedef __attribute__((address_space(3))) bf16x4_t lds_v4;
    const uint16_t *p0 = lds + kb * LD + nb;
    bf16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_v4 *)(p0));
    bf16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_v4 *)(p0 + 4 * LD));
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

template <int V, bool BKM, typename TO>
__global__ __launch_bounds__(mfma_cfg(V).wm *mfma_cfg(V).wn * 64) void k_mfma_bf16(
    GemmView v, const uint16_t *__restrict__ x, const uint16_t *__restrict__ y, TO *__restrict__ z,
    float *__restrict__ ws)
{
    constexpr MfmaCfg C = mfma_cfg(V);
    constexpr int BM = C.bm, BN = C.bn, BK = C.bk, WM = C.wm, WN = C.wn;
    constexpr int NT = WM * WN * 64;
    constexpr int TM = BM / WM / 32, TN = BN / WN / 32;
    constexpr int A_EL = lds_elems<V>(true, true), B_EL = lds_elems<V>(BKM, false);
    constexpr int LDA = BK + 8, LDB = BKM ? BK + 8 : BN + 32;
    constexpr int STAGE = A_EL + B_EL;
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

    TileLoader<BM, BK, NT, true, 0> la;
    TileLoader<BN, BK, NT, BKM, 1> lb;
    la.init(v.gm, v.gk, m0, bx, tid);
    lb.init(v.gn, v.gk, n0, by, tid);

    floatx16_t acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

    la.load(x, p2off<0>(v.gk, kbeg));
    lb.load(y, p2off<1>(v.gk, kbeg));
    la.store(smem);
    lb.store(smem + A_EL);
    __syncthreads();

    const int r_lane = lane & 31, k_lane = (lane >> 5) * 8;
    const int a_row0 = wm * (BM / WM) + r_lane;
    const int b_col0 = wn * (BN / WN);
    int stage = 0;
    for (uint32_t k0 = kbeg; k0 < kend; k0 += BK) {
        const bool more = k0 + BK < kend;
        if (more) {
            la.load(x, p2off<0>(v.gk, k0 + BK));
            lb.load(y, p2off<1>(v.gk, k0 + BK));
        }
        const uint16_t *a_s = smem + stage * STAGE, *b_s = a_s + A_EL;
        bf16x8_t af[2][TM], bf[2][TN];
#pragma unroll
        for (int i = 0; i < TM; ++i) af[0][i] = frag_k<LDA>(a_s, a_row0 + i * 32, k_lane);
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            if constexpr (BKM) bf[0][j] = frag_k<LDB>(b_s, b_col0 + j * 32 + r_lane, k_lane);
            else bf[0][j] = frag_tr<LDB>(b_s, b_col0 + j * 32, 0, lane);
        }
#pragma unroll
        for (int ks = 0; ks < BK / 16; ++ks) {
            const int cur = ks & 1, nxt = cur ^ 1;
            if (ks + 1 < BK / 16) {
#pragma unroll
                for (int i = 0; i < TM; ++i) af[nxt][i] = frag_k<LDA>(a_s, a_row0 + i * 32, (ks + 1) * 16 + k_lane);
#pragma unroll
                for (int j = 0; j < TN; ++j) {
                    if constexpr (BKM) bf[nxt][j] = frag_k<LDB>(b_s, b_col0 + j * 32 + r_lane, (ks + 1) * 16 + k_lane);
                    else bf[nxt][j] = frag_tr<LDB>(b_s, b_col0 + j * 32, (ks + 1) * 16, lane);
                }
            }
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[cur][i], bf[cur][j], acc[i][j], 0, 0, 0);
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
    // row = (wave row + 32 i + 8 (e/4)) + (4 (l/32) + e%4): a multiple of 8 plus
    // a part below 8, so its offset splits into a wave-uniform and a lane part.
    const int32_t zm0 = p2off<1>(v.gm, m0) + bz, zn0 = p2off<1>(v.gn, n0);
    int32_t lo[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) lo[r] = p2off<1>(v.gm, 4 * (lane >> 5) + r);
#pragma unroll
    for (int i = 0; i < TM; ++i) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int32_t hi = zm0 + p2off<1>(v.gm, wm * (BM / WM) + i * 32 + 8 * q);
#pragma unroll
            for (int j = 0; j < TN; ++j) {
                const int32_t on = zn0 + p2off<1>(v.gn, b_col0 + j * 32 + r_lane);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int32_t o = hi + lo[r] + on;
                    const float val = acc[i][j][4 * q + r];
                    if (split) wsp[o] = val;
                    else Scalar<TO>::store(z, o, val * v.post_scale);
                }
            }
        }
    }
}

int launch_split_fold(const tra_plan_s &p, const void *ws, void *z, void *stream);

template <int V, bool BKM, typename TO>
static int launch_v(const tra_plan_s &p, const void *x, const void *y, void *z, void *ws, hipStream_t s)
{
    constexpr MfmaCfg C = mfma_cfg(V);
    constexpr size_t lds = mfma_lds_bytes<V, BKM>();
    static bool attr_set = false;
    if (!attr_set) {
        hipError_t e = hipFuncSetAttribute((const void *)k_mfma_bf16<V, BKM, TO>,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return (int)e;
        attr_set = true;
    }
    const GemmView &v = p.gv;
    dim3 grid((v.gm.total / C.bm) * (v.gn.total / C.bn), v.gb.total, v.split);
    hipLaunchKernelGGL((k_mfma_bf16<V, BKM, TO>), grid, dim3(C.wm * C.wn * 64), lds, s, v,
                       (const uint16_t *)x, (const uint16_t *)y, (TO *)z, (float *)ws);
    return (int)hipGetLastError();
}

template <int V, typename TO>
static int launch_layout(const tra_plan_s &p, const void *x, const void *y, void *z, void *ws, hipStream_t s)
{
    if (p.b_kmajor) return launch_v<V, true, TO>(p, x, y, z, ws, s);
    return launch_v<V, false, TO>(p, x, y, z, ws, s);
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
