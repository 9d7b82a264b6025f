// k_valu_tile.hip -- register-blocked join + aggregation on the vector ALUs.
//
// Page "EinDecomp：基于爱因斯坦求和与张量关系代数的自动张量并行分解算法",
// section 2.1: the join may be any binary scalar function, e.g. (x-y)^2, and
// the aggregate any associative-commutative reduction, e.g. max.  Such joins
// are not products, so they do not map to the matrix cores: each thread owns
// an 8x8 block of one output sub-tensor, keeps its 64 running aggregates in
// registers, and walks the contracted range (contracted keys ascending, then
// the in-block index) through an LDS-staged tile of both operands.
//
// Operands are addressed through the relation layout's per-sub-dimension
// strides (power-of-two groups), so any partition vector d is read in place.
#include <hip/hip_runtime.h>

#include "device_common.h"
#include "plan.h"

namespace tra {

constexpr int VT_BM = 128, VT_BN = 128, VT_BK = 32, VT_PAD = 4, VT_THREADS = 256;

TileShape valu_tile_shape(int variant)
{
    if (variant == 0) return {VT_BM, VT_BN, VT_BK};
    return {0, 0, 0};
}

// Map the linear workgroup id to an output tile.  Consecutive ids land on
// different XCDs (round-robin dispatch); regroup them so each XCD owns a
// contiguous run of tiles, then sweep tile columns within groups of 8 rows so
// that neighbouring workgroups share operand panels in that XCD's L2.
__device__ __forceinline__ void tile_of(uint32_t nb, uint32_t tiles_n, uint32_t &tm, uint32_t &tn)
{
    uint32_t b = blockIdx.x;
    if (nb % 8 == 0) b = (b % 8) * (nb / 8) + b / 8;
    const uint32_t G = 8;
    uint32_t tiles_m = nb / tiles_n;
    uint32_t per = G * tiles_n;
    uint32_t g = b / per, first = g * G;
    uint32_t gs = min(tiles_m - first, G);
    uint32_t r = b % per;
    tm = first + r % gs;
    tn = r / gs;
}

template <int JOIN, typename A>
__device__ __forceinline__ A vjoin(A a, A b)
{
    if constexpr (std::is_same<A, float>::value) {
        if constexpr (JOIN == J_MUL) return a * b;
        else if constexpr (JOIN == J_SQDIFF) { float t = a - b; return t * t; }
        else return a + b;
    } else {
        if constexpr (JOIN == J_MUL) return wmul(a, b);
        else if constexpr (JOIN == J_SQDIFF) { int32_t t = wsub(a, b); return wmul(t, t); }
        else return wadd(a, b);
    }
}

template <int AGG, typename A>
__device__ __forceinline__ A vfold(A acc, A v)
{
    if constexpr (AGG == A_SUM) {
        if constexpr (std::is_same<A, float>::value) return acc + v;
        else return wadd(acc, v);
    } else if constexpr (AGG == A_MAX) {
        if constexpr (std::is_same<A, float>::value) return fmaxf(acc, v);
        else return max(acc, v);
    } else {
        if constexpr (std::is_same<A, float>::value) return fminf(acc, v);
        else return min(acc, v);
    }
}

// Two contracted steps folded at once (lets max / min use a 3-input op).
template <int JOIN, int AGG, typename A>
__device__ __forceinline__ A vstep2(A acc, A a0, A b0, A a1, A b1)
{
    if constexpr (AGG == A_SUM && JOIN == J_SQDIFF && std::is_same<A, float>::value) {
        float t0 = a0 - b0, t1 = a1 - b1;
        return fmaf(t1, t1, fmaf(t0, t0, acc));
    } else if constexpr (AGG == A_SUM && JOIN == J_MUL && std::is_same<A, float>::value) {
        return fmaf(a1, b1, fmaf(a0, b0, acc));
    } else if constexpr (AGG == A_SUM) {
        return vfold<AGG>(vfold<AGG>(acc, vjoin<JOIN>(a0, b0)), vjoin<JOIN>(a1, b1));
    } else if constexpr (std::is_same<A, int32_t>::value) {
        // one 3-input max / min per two terms, written as the instruction so
        // that the compiler cannot re-associate the chain into 2-input ones
        // (which costs 3 half-rate instructions per 4 terms instead of 2)
        if constexpr (JOIN == J_ADD) {
            // the two sums and their fold as one block: the sums never wait
            // in registers for a later fold
            int32_t t0, t1;
            if constexpr (AGG == A_MAX)
                asm("v_add_u32 %1, %3, %4\n\tv_add_u32 %2, %5, %6\n\tv_max3_i32 %0, %0, %1, %2"
                    : "+v"(acc), "=&v"(t0), "=&v"(t1) : "v"(a0), "v"(b0), "v"(a1), "v"(b1));
            else
                asm("v_add_u32 %1, %3, %4\n\tv_add_u32 %2, %5, %6\n\tv_min3_i32 %0, %0, %1, %2"
                    : "+v"(acc), "=&v"(t0), "=&v"(t1) : "v"(a0), "v"(b0), "v"(a1), "v"(b1));
            return acc;
        }
        const int32_t t0 = vjoin<JOIN>(a0, b0), t1 = vjoin<JOIN>(a1, b1);
        int32_t r;
        if constexpr (AGG == A_MAX) asm("v_max3_i32 %0, %1, %2, %3" : "=v"(r) : "v"(acc), "v"(t0), "v"(t1));
        else asm("v_min3_i32 %0, %1, %2, %3" : "=v"(r) : "v"(acc), "v"(t0), "v"(t1));
        return r;
    } else {
        return vfold<AGG>(acc, vfold<AGG>(vjoin<JOIN>(a0, b0), vjoin<JOIN>(a1, b1)));
    }
}

template <int AGG, typename A>
__device__ __forceinline__ A vinit()
{
    if constexpr (AGG == A_SUM) return A(0);
    else if constexpr (AGG == A_MAX) {
        if constexpr (std::is_same<A, float>::value) return -INFINITY;
        else return INT32_MIN;
    } else {
        if constexpr (std::is_same<A, float>::value) return INFINITY;
        else return INT32_MAX;
    }
}

// Offset of row / column idx of a ragged group in tensor slot t (mixed radix,
// last sub-dimension fastest).
__device__ __forceinline__ int32_t rad_off(const Radix &r, int t, uint32_t idx)
{
    int64_t o = 0;
    for (int i = r.n - 1; i >= 0; --i) {
        const uint32_t e = r.ext[i], q = idx / e;
        o += (int64_t)(idx - q * e) * r.st[t][i];
        idx = q;
    }
    return (int32_t)o;
}

// ---- int32 max-plus / min-plus on packed 16-bit halves -------------------
//
// Every integer of magnitude at most 2048 is exact in IEEE binary16 (11-bit
// significand), so when all inputs lie in [-SI_LIM, SI_LIM] (SI_LIM = 1024)
// each sum x + y and each max / min of such sums is computed exactly in f16:
// the result is the int32 result, bit for bit.  gfx950 then forms two sums per
// instruction (v_pk_add_f16) and folds two sums into each of two running
// aggregates per instruction (v_pk_maximum3_f16 / v_pk_minimum3_f16), 1.5
// instruction slots per term where the 32-bit path needs 2 (measured issue
// rates: about 55 packed lanes/clk/CU against 94 for v_add_u32).
//
// A call runs three kernels on its stream: the range check writes one flag
// word per workgroup into the workspace; the packed kernel runs when every
// flag is clear, the 32-bit kernel when one is set (each reads all flags at
// entry and the other returns at once).  The choice is made on the device,
// per call, with no host synchronisation.
constexpr int SI_LIM = 1024;
constexpr int SI_FLAGS = 256;   // range-check workgroups = flag words
static_assert(SI_FLAGS == VT_THREADS, "one flag word per tile-kernel thread");
static_assert(SI_FLAGS * 4 == SMALL_INT_FLAG_BYTES, "flag words in the plan's workspace");

template <int JOIN, int AGG, typename T>
__host__ __device__ constexpr bool small_int_join()
{
    return JOIN == J_ADD && (AGG == A_MAX || AGG == A_MIN) && std::is_same<T, int32_t>::value;
}

// true when the flags say this kernel runs: packed = every flag clear.
__device__ __forceinline__ bool gate_open(const uint32_t *__restrict__ gate, bool packed)
{
    const int any = __syncthreads_or(gate[threadIdx.x] != 0);
    return packed ? !any : any != 0;
}

__device__ __forceinline__ uint32_t si_out_of_range(int32_t a) { return (uint32_t)a + SI_LIM > 2u * SI_LIM; }

// One flag word per workgroup: 1 if any element of X or Y lies outside
// [-SI_LIM, SI_LIM].  SI_CHECK_THREADS threads per workgroup, each with four
// 16-byte loads in flight per round.
constexpr int SI_CHECK_THREADS = 1024;
__global__ __launch_bounds__(SI_CHECK_THREADS) void k_small_int_check(const int32_t *__restrict__ x, int64_t nx,
                                                                      const int32_t *__restrict__ y, int64_t ny,
                                                                      uint32_t *__restrict__ flags)
{
    typedef int32_t I4 __attribute__((ext_vector_type(4)));
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    const int64_t t0 = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    uint32_t bad = 0;
    auto test4 = [&](I4 q) {
        bad |= si_out_of_range(q.x) | si_out_of_range(q.y) | si_out_of_range(q.z) | si_out_of_range(q.w);
    };
    auto scan = [&](const int32_t *__restrict__ p, int64_t n) {
        const int64_t nv = ((uintptr_t)p & 15) == 0 ? n / 4 : 0;
        const I4 *p4 = (const I4 *)p;
        int64_t i = t0;
        for (; i + 3 * stride < nv; i += 4 * stride) {
            const I4 q0 = p4[i], q1 = p4[i + stride], q2 = p4[i + 2 * stride], q3 = p4[i + 3 * stride];
            test4(q0);
            test4(q1);
            test4(q2);
            test4(q3);
        }
        for (; i < nv; i += stride) test4(p4[i]);
        for (int64_t j = nv * 4 + t0; j < n; j += stride) bad |= si_out_of_range(p[j]);
    };
    scan(x, nx);
    scan(y, ny);
    bad = __syncthreads_or(bad);
    if (threadIdx.x == 0) flags[blockIdx.x] = bad;
}

// Store a thread's 8x8 block of aggregates: to the output through its
// relation layout, or (split aggregation) to this split's fp32 / int32 slice of
// the workspace, which the fold kernel combines.
// Rows ty*4+{0..3}, 64+ty*4+{0..3}; columns tx*4+{0..3}, 64+tx*4+{0..3}.
template <typename A, typename TO, bool RAG = false>
__device__ __forceinline__ void vt_store(const GemmView &v, A (&acc)[8][8], TO *__restrict__ z, A *__restrict__ ws,
                                         uint32_t m0, uint32_t n0, int32_t bz, int tx, int ty,
                                         const RaggedMN *rag = nullptr)
{
    typedef A V4 __attribute__((ext_vector_type(4)));
    const bool split = v.split > 1;
    A *wsp = split ? ws + (int64_t)blockIdx.z * v.z_elems : nullptr;
    const int32_t zm0 = RAG ? bz : p2off<1>(v.gm, m0) + bz, zn0 = RAG ? 0 : p2off<1>(v.gn, n0);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const uint32_t m = i < 4 ? ty * 4 + i : 64 + ty * 4 + (i - 4);
        // ragged edge: rows past the extent hold values of clamped loads
        if (RAG && m0 + m >= rag->M) continue;
        const int32_t om = zm0 + (RAG ? rad_off(rag->m, 1, m0 + m) : p2off<1>(v.gm, m));
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const uint32_t nbase = h * 64 + tx * 4;
            int32_t on[4];
            bool ok[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                ok[j] = !RAG || n0 + nbase + j < rag->N;
                on[j] = RAG ? (ok[j] ? rad_off(rag->n, 1, n0 + nbase + j) : 0) : zn0 + p2off<1>(v.gn, nbase + j);
            }
            const bool vec = ok[3] && on[1] == on[0] + 1 && on[2] == on[0] + 2 && on[3] == on[0] + 3 &&
                             ((om + on[0]) & 3) == 0;
            A r4[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) r4[j] = acc[i][h * 4 + j];
            if (split) {
                if (vec) *(V4 *)&wsp[om + on[0]] = V4{r4[0], r4[1], r4[2], r4[3]};
                else
                    for (int j = 0; j < 4; ++j)
                        if (ok[j]) wsp[om + on[j]] = r4[j];
            } else {
                if constexpr (std::is_same<A, float>::value) {
#pragma unroll
                    for (int j = 0; j < 4; ++j) r4[j] *= v.post_scale;
                }
                if constexpr (std::is_same<TO, float>::value || std::is_same<TO, int32_t>::value) {
                    if (vec) *(V4 *)&z[om + on[0]] = V4{r4[0], r4[1], r4[2], r4[3]};
                    else
                        for (int j = 0; j < 4; ++j)
                            if (ok[j]) z[om + on[j]] = r4[j];
                } else {
                    for (int j = 0; j < 4; ++j)
                        if (ok[j]) Scalar<TO>::store(z, om + on[j], (float)r4[j]);
                }
            }
        }
    }
}

// Loader assignment: 4 vectors of 4 elements per thread for each operand.
// K-major operand: vector along k; 8 vectors per row of BK.
// MN-major operand: vector along m/n; BM/4 vectors per k-row.
// Offsets split at the tile boundary (power-of-two digits): off(r0 + d) =
// off(r0) + off(d), so the per-thread parts are computed once and every
// k-tile adds only the uniform off(k0).
template <bool AK, bool BKM>
struct VtLoad {
    int32_t a_off[4], b_off[4];
    int a_row[4], a_col[4], b_row[4], b_col[4];

    // RAG: rows and columns past the extents are clamped to the last valid
    // one (the last valid vector of 4 for an MN-major operand, whose fastest
    // extent is a multiple of 4), so every load stays inside the operand; the
    // store drops what they produce.
    template <bool RAG = false>
    __device__ __forceinline__ void init(const GemmView &v, uint32_t m0, uint32_t n0, int32_t bx, int32_t by,
                                         int tid, const RaggedMN *rag = nullptr)
    {
        constexpr int BM = VT_BM, BN = VT_BN, BK = VT_BK;
        const int32_t am0 = RAG ? bx : p2off<0>(v.gm, m0) + bx, bn0 = RAG ? by : p2off<0>(v.gn, n0) + by;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            int q = tid + VT_THREADS * r;
            if constexpr (AK) {
                a_col[r] = (q % (BK / 4)) * 4;  // k
                a_row[r] = q / (BK / 4);        // m
            } else {
                a_row[r] = (q % (BM / 4)) * 4;  // m
                a_col[r] = q / (BM / 4);        // k
            }
            if constexpr (RAG) {
                const uint32_t m = min(m0 + (uint32_t)a_row[r], rag->M - (AK ? 1u : 4u));
                a_off[r] = am0 + rad_off(rag->m, 0, m) + p2off<0>(v.gk, a_col[r]);
            } else {
                a_off[r] = am0 + p2off<0>(v.gm, a_row[r]) + p2off<0>(v.gk, a_col[r]);
            }
            if constexpr (BKM) {
                b_col[r] = (q % (BK / 4)) * 4;
                b_row[r] = q / (BK / 4);
            } else {
                b_row[r] = (q % (BN / 4)) * 4;
                b_col[r] = q / (BN / 4);
            }
            if constexpr (RAG) {
                const uint32_t n = min(n0 + (uint32_t)b_row[r], rag->N - (BKM ? 1u : 4u));
                b_off[r] = bn0 + rad_off(rag->n, 0, n) + p2off<1>(v.gk, b_col[r]);
            } else {
                b_off[r] = bn0 + p2off<0>(v.gn, b_row[r]) + p2off<1>(v.gk, b_col[r]);
            }
        }
    }
};

template <int JOIN, int AGG, typename T, typename TO, bool AK, bool BKM, bool RAG>
__global__ __launch_bounds__(VT_THREADS) void k_valu_tile(GemmView v, const T *__restrict__ x,
                                                         const T *__restrict__ y, TO *__restrict__ z,
                                                         T *__restrict__ ws, const uint32_t *__restrict__ gate,
                                                         RaggedMN rag)
{
    using A = T;
    // int32 max-plus / min-plus runs after the packed 16-bit kernel, and only
    // where the range check found an input it cannot represent (ragged plans
    // have no packed path)
    if constexpr (small_int_join<JOIN, AGG, T>() && !RAG) {
        if (!gate_open(gate, false)) return;
    }
    constexpr int BM = VT_BM, BN = VT_BN, BK = VT_BK;
    constexpr int LDA = BM + VT_PAD, LDB = BN + VT_PAD;
    __shared__ __attribute__((aligned(16))) A As[BK * LDA];
    __shared__ __attribute__((aligned(16))) A Bs[BK * LDB];

    const int tid = threadIdx.x;
    const uint32_t tiles_n = v.gn.total / BN;
    const uint32_t nb = (v.gm.total / BM) * tiles_n;
    uint32_t tm, tn;
    tile_of(nb, tiles_n, tm, tn);
    const uint32_t m0 = tm * BM, n0 = tn * BN;
    const uint32_t bidx = blockIdx.y;
    const int32_t bx = p2off<0>(v.gb, bidx), by = p2off<1>(v.gb, bidx), bz = p2off<2>(v.gb, bidx);
    const uint32_t kbeg = blockIdx.z * (uint32_t)v.k_per_split;
    const uint32_t kend = kbeg + (uint32_t)v.k_per_split;

    VtLoad<AK, BKM> ld;
    ld.template init<RAG>(v, m0, n0, bx, by, tid, &rag);
    const int32_t *a_off = ld.a_off, *b_off = ld.b_off;
    const int *a_row = ld.a_row, *a_col = ld.a_col, *b_row = ld.b_row, *b_col = ld.b_col;

    A acc[8][8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[i][j] = vinit<AGG, A>();

    const int tx = tid % 16, ty = tid / 16;
    // Native 4-vectors (not HIP's union-based float4/int4): those stop the
    // compiler from keeping the prefetch registers out of scratch memory.
    typedef A V4 __attribute__((ext_vector_type(4)));
    V4 ra[4], rb[4];

    auto gload = [&](uint32_t k0) {
        const int32_t kx = p2off<0>(v.gk, k0), ky = p2off<1>(v.gk, k0);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            ra[r] = *(const V4 *)(x + a_off[r] + kx);
            rb[r] = *(const V4 *)(y + b_off[r] + ky);
        }
    };
    auto lstore = [&]() {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            if constexpr (AK) {
                As[(a_col[r] + 0) * LDA + a_row[r]] = ra[r].x;
                As[(a_col[r] + 1) * LDA + a_row[r]] = ra[r].y;
                As[(a_col[r] + 2) * LDA + a_row[r]] = ra[r].z;
                As[(a_col[r] + 3) * LDA + a_row[r]] = ra[r].w;
            } else {
                *(V4 *)&As[a_col[r] * LDA + a_row[r]] = ra[r];
            }
            if constexpr (BKM) {
                Bs[(b_col[r] + 0) * LDB + b_row[r]] = rb[r].x;
                Bs[(b_col[r] + 1) * LDB + b_row[r]] = rb[r].y;
                Bs[(b_col[r] + 2) * LDB + b_row[r]] = rb[r].z;
                Bs[(b_col[r] + 3) * LDB + b_row[r]] = rb[r].w;
            } else {
                *(V4 *)&Bs[b_col[r] * LDB + b_row[r]] = rb[r];
            }
        }
    };

    gload(kbeg);
    for (uint32_t k0 = kbeg; k0 < kend; k0 += BK) {
        __syncthreads();
        lstore();
        __syncthreads();
        if (k0 + BK < kend) gload(k0 + BK);
#pragma unroll 4
        for (int kk = 0; kk < BK; kk += 2) {
            V4 a0l = *(const V4 *)&As[kk * LDA + ty * 4], a0h = *(const V4 *)&As[kk * LDA + 64 + ty * 4];
            V4 b0l = *(const V4 *)&Bs[kk * LDB + tx * 4], b0h = *(const V4 *)&Bs[kk * LDB + 64 + tx * 4];
            V4 a1l = *(const V4 *)&As[(kk + 1) * LDA + ty * 4], a1h = *(const V4 *)&As[(kk + 1) * LDA + 64 + ty * 4];
            V4 b1l = *(const V4 *)&Bs[(kk + 1) * LDB + tx * 4], b1h = *(const V4 *)&Bs[(kk + 1) * LDB + 64 + tx * 4];
            A a0[8] = {a0l.x, a0l.y, a0l.z, a0l.w, a0h.x, a0h.y, a0h.z, a0h.w};
            A b0[8] = {b0l.x, b0l.y, b0l.z, b0l.w, b0h.x, b0h.y, b0h.z, b0h.w};
            A a1[8] = {a1l.x, a1l.y, a1l.z, a1l.w, a1h.x, a1h.y, a1h.z, a1h.w};
            A b1[8] = {b1l.x, b1l.y, b1l.z, b1l.w, b1h.x, b1h.y, b1h.z, b1h.w};
#pragma unroll
            for (int i = 0; i < 8; ++i)
#pragma unroll
                for (int j = 0; j < 8; ++j) acc[i][j] = vstep2<JOIN, AGG>(acc[i][j], a0[i], b0[j], a1[i], b1[j]);
        }
    }

    vt_store<A, TO, RAG>(v, acc, z, ws, m0, n0, bz, tx, ty, &rag);
}

// Packed 16-bit int32 max-plus / min-plus (see above).  The same 128x128 tile,
// loaders and epilogue as k_valu_tile; operands are converted to f16 on their
// way into LDS, where
//   Xh[k/2][m]          holds (x[m][k], x[m][k+1])            (k even)
//   Yh[k/2][n/2][k&1]   holds (y[k][n], y[k][n+1])            (n even)
// so that a thread's 8 rows and 8 columns of one k-pair are four 16-byte reads.
// Accumulator word c of row i holds the aggregates of columns 2c and 2c+1 of
// the thread's columns; per k-pair and word, the x of row i (low half for k,
// high half for k+1, broadcast by op_sel) is added to the column pair of k and
// of k+1 and both sums are folded by one 3-input op.
// One row's four accumulator words per block: the eight sums first, then the
// four folds, so that no instruction overwrites a register that one of the
// two before it still reads (packed instructions take two passes; such a
// write costs a wait state).
#define TRA_H16_ROW(FOLD)                                                                                   \
    asm("v_pk_add_f16 %4, %12, %13 op_sel_hi:[0,1]\n\t"                                                      \
        "v_pk_add_f16 %5, %12, %14 op_sel:[1,0] op_sel_hi:[1,1]\n\t"                                         \
        "v_pk_add_f16 %6, %12, %15 op_sel_hi:[0,1]\n\t"                                                      \
        "v_pk_add_f16 %7, %12, %16 op_sel:[1,0] op_sel_hi:[1,1]\n\t"                                         \
        "v_pk_add_f16 %8, %12, %17 op_sel_hi:[0,1]\n\t"                                                      \
        "v_pk_add_f16 %9, %12, %18 op_sel:[1,0] op_sel_hi:[1,1]\n\t"                                         \
        "v_pk_add_f16 %10, %12, %19 op_sel_hi:[0,1]\n\t"                                                     \
        "v_pk_add_f16 %11, %12, %20 op_sel:[1,0] op_sel_hi:[1,1]\n\t" FOLD " %0, %0, %4, %5\n\t" FOLD        \
        " %1, %1, %6, %7\n\t" FOLD " %2, %2, %8, %9\n\t" FOLD " %3, %3, %10, %11"                            \
        : "+v"(acc[0]), "+v"(acc[1]), "+v"(acc[2]), "+v"(acc[3]), "=&v"(t[0]), "=&v"(t[1]), "=&v"(t[2]),      \
          "=&v"(t[3]), "=&v"(t[4]), "=&v"(t[5]), "=&v"(t[6]), "=&v"(t[7])                                  \
        : "v"(xw), "v"(y0[0]), "v"(y1[0]), "v"(y0[1]), "v"(y1[1]), "v"(y0[2]), "v"(y1[2]), "v"(y0[3]),       \
          "v"(y1[3]))
template <int AGG>
__device__ __forceinline__ void h16_row(uint32_t (&acc)[4], uint32_t xw, const uint32_t (&y0)[4],
                                        const uint32_t (&y1)[4])
{
    uint32_t t[8];
    if constexpr (AGG == A_MAX) TRA_H16_ROW("v_pk_maximum3_f16");
    else TRA_H16_ROW("v_pk_minimum3_f16");
}
#undef TRA_H16_ROW

// int32 -> f16 bits, exact for |a| <= 2048
__device__ __forceinline__ uint16_t h16_of(int32_t a) { return __builtin_bit_cast(uint16_t, (_Float16)(float)a); }
__device__ __forceinline__ uint32_t h16_pack(int32_t a, int32_t b)
{
    return (uint32_t)h16_of(a) | ((uint32_t)h16_of(b) << 16);
}
__device__ __forceinline__ int32_t h16_to_int(uint32_t w) { return (int32_t)(float)__builtin_bit_cast(_Float16, (uint16_t)w); }

template <int AGG, bool AK, bool BKM>
__global__ __launch_bounds__(VT_THREADS) void k_valu_tile_h16(GemmView v, const int32_t *__restrict__ x,
                                                             const int32_t *__restrict__ y, int32_t *__restrict__ z,
                                                             int32_t *__restrict__ ws,
                                                             const uint32_t *__restrict__ gate)
{
    if (!gate_open(gate, true)) return;
    constexpr int BM = VT_BM, BN = VT_BN, BK = VT_BK;
    constexpr int LXW = BM + 4;   // words per k-pair row of Xh
    constexpr int LYW = BN + 4;   // words per k-pair row of Yh (BN/2 column pairs x 2 k)
    __shared__ __attribute__((aligned(16))) uint32_t Xh[BK / 2 * LXW];
    __shared__ __attribute__((aligned(16))) uint32_t Yh[BK / 2 * LYW];
    uint16_t *const Xs = (uint16_t *)Xh, *const Ys = (uint16_t *)Yh;

    const int tid = threadIdx.x;
    const uint32_t tiles_n = v.gn.total / BN;
    const uint32_t nb = (v.gm.total / BM) * tiles_n;
    uint32_t tm, tn;
    tile_of(nb, tiles_n, tm, tn);
    const uint32_t m0 = tm * BM, n0 = tn * BN;
    const uint32_t bidx = blockIdx.y;
    const int32_t bx = p2off<0>(v.gb, bidx), by = p2off<1>(v.gb, bidx), bz = p2off<2>(v.gb, bidx);
    const uint32_t kbeg = blockIdx.z * (uint32_t)v.k_per_split;
    const uint32_t kend = kbeg + (uint32_t)v.k_per_split;

    VtLoad<AK, BKM> ld;
    ld.init(v, m0, n0, bx, by, tid);

    // -inf / +inf in both halves: the identity of max / min
    constexpr uint32_t init = AGG == A_MAX ? 0xFC00FC00u : 0x7C007C00u;
    uint32_t acc[8][4];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int c = 0; c < 4; ++c) acc[i][c] = init;

    const int tx = tid % 16, ty = tid / 16;
    typedef int32_t V4 __attribute__((ext_vector_type(4)));
    typedef uint32_t W4 __attribute__((ext_vector_type(4)));
    V4 ra[4], rb[4];

    auto gload = [&](uint32_t k0) {
        const int32_t kx = p2off<0>(v.gk, k0), ky = p2off<1>(v.gk, k0);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            ra[r] = *(const V4 *)(x + ld.a_off[r] + kx);
            rb[r] = *(const V4 *)(y + ld.b_off[r] + ky);
        }
    };
    auto lstore = [&]() {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int ar = ld.a_row[r], ac = ld.a_col[r], br = ld.b_row[r], bc = ld.b_col[r];
            if constexpr (AK) {
                // 4 consecutive k of row ar (ac even): two k-pair words
                Xh[(ac / 2) * LXW + ar] = h16_pack(ra[r].x, ra[r].y);
                Xh[(ac / 2 + 1) * LXW + ar] = h16_pack(ra[r].z, ra[r].w);
            } else {
                // 4 consecutive rows at one k: four halves
                const int w = (ac / 2) * LXW + ar, hk = ac & 1;
                Xs[2 * (w + 0) + hk] = h16_of(ra[r].x);
                Xs[2 * (w + 1) + hk] = h16_of(ra[r].y);
                Xs[2 * (w + 2) + hk] = h16_of(ra[r].z);
                Xs[2 * (w + 3) + hk] = h16_of(ra[r].w);
            }
            if constexpr (BKM) {
                // 4 consecutive k of column br: four halves
                const int hn = br & 1, wn = (br / 2) * 2;
                Ys[2 * (((bc + 0) / 2) * LYW + wn + ((bc + 0) & 1)) + hn] = h16_of(rb[r].x);
                Ys[2 * (((bc + 1) / 2) * LYW + wn + ((bc + 1) & 1)) + hn] = h16_of(rb[r].y);
                Ys[2 * (((bc + 2) / 2) * LYW + wn + ((bc + 2) & 1)) + hn] = h16_of(rb[r].z);
                Ys[2 * (((bc + 3) / 2) * LYW + wn + ((bc + 3) & 1)) + hn] = h16_of(rb[r].w);
            } else {
                // 4 consecutive columns (br even) at one k: two column-pair words
                const int w = (bc / 2) * LYW + br + (bc & 1);
                Yh[w] = h16_pack(rb[r].x, rb[r].y);
                Yh[w + 2] = h16_pack(rb[r].z, rb[r].w);
            }
        }
    };

    gload(kbeg);
    for (uint32_t k0 = kbeg; k0 < kend; k0 += BK) {
        __syncthreads();
        lstore();
        __syncthreads();
        if (k0 + BK < kend) gload(k0 + BK);
#pragma unroll 4
        for (int kp = 0; kp < BK / 2; ++kp) {
            const W4 xl = *(const W4 *)&Xh[kp * LXW + ty * 4], xh = *(const W4 *)&Xh[kp * LXW + 64 + ty * 4];
            const W4 yl = *(const W4 *)&Yh[kp * LYW + tx * 4], yh = *(const W4 *)&Yh[kp * LYW + 64 + tx * 4];
            const uint32_t xa[8] = {xl.x, xl.y, xl.z, xl.w, xh.x, xh.y, xh.z, xh.w};
            // column pairs 2tx, 2tx+1, 32+2tx, 32+2tx+1 at k (y0) and k+1 (y1)
            const uint32_t y0[4] = {yl.x, yl.z, yh.x, yh.z}, y1[4] = {yl.y, yl.w, yh.y, yh.w};
#pragma unroll
            for (int i = 0; i < 8; ++i) h16_row<AGG>(acc[i], xa[i], y0, y1);
        }
    }

    int32_t r[8][8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            r[i][2 * c] = h16_to_int(acc[i][c]);
            r[i][2 * c + 1] = h16_to_int(acc[i][c] >> 16);
        }
    vt_store<int32_t, int32_t>(v, r, z, ws, m0, n0, bz, tx, ty);
}

int launch_split_fold(const tra_plan_s &p, const void *ws, void *z, void *stream);

template <int JOIN, int AGG, typename T, typename TO>
static int launch_vt(const tra_plan_s &p, const void *x, const void *y, void *z, void *ws, void *stream)
{
    hipStream_t s = (hipStream_t)stream;
    const GemmView &v = p.gv;
    dim3 grid((v.gm.total / VT_BM) * (v.gn.total / VT_BN), v.gb.total, v.split);
    const uint32_t *gate = nullptr;
    if constexpr (small_int_join<JOIN, AGG, T>()) {
        if (!p.ragged) {
            uint32_t *flags = (uint32_t *)((char *)ws + small_int_flags_offset(v.split, p.info.z_elems));
            hipLaunchKernelGGL(k_small_int_check, dim3(SI_FLAGS), dim3(SI_CHECK_THREADS), 0, s, (const int32_t *)x,
                               p.info.x_elems, (const int32_t *)y, p.info.y_elems, flags);
#define TRA_H16(AK, BKM)                                                                                 \
    hipLaunchKernelGGL((k_valu_tile_h16<AGG, AK, BKM>), grid, dim3(VT_THREADS), 0, s, v, (const int32_t *)x, \
                       (const int32_t *)y, (int32_t *)z, (int32_t *)ws, (const uint32_t *)flags)
            if (p.a_kmajor && p.b_kmajor) TRA_H16(true, true);
            else if (p.a_kmajor) TRA_H16(true, false);
            else if (p.b_kmajor) TRA_H16(false, true);
            else TRA_H16(false, false);
#undef TRA_H16
            gate = flags;
        }
    }
#define TRA_VT(AK, BKM, RAG)                                                                             \
    hipLaunchKernelGGL((k_valu_tile<JOIN, AGG, T, TO, AK, BKM, RAG>), grid, dim3(VT_THREADS), 0, s, v,  \
                       (const T *)x, (const T *)y, (TO *)z, (T *)ws, gate, p.rag)
    if (p.ragged) {
        if (p.a_kmajor && p.b_kmajor) TRA_VT(true, true, true);
        else if (p.a_kmajor) TRA_VT(true, false, true);
        else if (p.b_kmajor) TRA_VT(false, true, true);
        else TRA_VT(false, false, true);
    } else {
        if (p.a_kmajor && p.b_kmajor) TRA_VT(true, true, false);
        else if (p.a_kmajor) TRA_VT(true, false, false);
        else if (p.b_kmajor) TRA_VT(false, true, false);
        else TRA_VT(false, false, false);
    }
#undef TRA_VT
    int err = (int)hipGetLastError();
    if (err || v.split == 1) return err;
    return launch_split_fold(p, ws, z, stream);
}

template <typename T, typename TO>
static int launch_vt_ops(const tra_plan_s &p, const void *x, const void *y, void *z, void *ws, void *stream)
{
#define TRA_OPS(J, AG) if (p.join == J && p.agg == AG) return launch_vt<J, AG, T, TO>(p, x, y, z, ws, stream)
    TRA_OPS(J_MUL, A_SUM);
    TRA_OPS(J_SQDIFF, A_SUM);
    TRA_OPS(J_ADD, A_MAX);
    TRA_OPS(J_ADD, A_MIN);
#undef TRA_OPS
    return (int)hipErrorInvalidValue;
}

int launch_valu_tile(const tra_plan_s &p, const void *x, const void *y, void *z, void *ws, void *stream)
{
    if (p.in_dtype == D_I32) return launch_vt_ops<int32_t, int32_t>(p, x, y, z, ws, stream);
    if (p.out_dtype == D_BF16) return launch_vt_ops<float, bf16_t>(p, x, y, z, ws, stream);
    return launch_vt_ops<float, float>(p, x, y, z, ws, stream);
}

}  // namespace tra
