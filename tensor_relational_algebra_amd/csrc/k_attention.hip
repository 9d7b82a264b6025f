// k_attention.hip -- the attention chain of an EinGraph (scores join, softmax
// as a logsumexp aggregate, weighted-sum join) as one kernel.
//
// Page "EinDecomp：基于爱因斯坦求和与张量关系代数的自动张量并行分解算法":
//  * section 2.1: multi-head attention as EinSums: S[h,s,t] = sum_d Q[s,h,d]
//    K[t,h,d] (scaled), softmax over t, O[s,h,d] = sum_t A[h,s,t] V[t,h,d];
//    softmax is an EinSum whose aggregate is associative (here: logsumexp);
//  * its closing remarks on fusing operators into one "super-operator".
// The aggregation over the t partitions is the logsumexp monoid carried as a
// running (max m, sum l) pair, folded in ascending t order, with the weighted
// sum rescaled whenever m grows: the same fold that the unfused softmax node
// performs over its t blocks, except that neither S nor A is ever written.
//
// Work decomposition: one workgroup per (head, 128 query rows); four waves,
// each owning 32 query rows.  Per 64-row tile of keys/values:
//   S^T = K Q^T           (32 x 32 x 16 bf16 matrix-core steps; K from LDS,
//                          Q^T fragments held in registers for the whole run)
//   online logsumexp      (each lane owns one query column of S^T, so the
//                          running (m, l) live in the lane; the two 32-lane
//                          halves that share a column exchange one value)
//   O^T += V^T P^T        (P^T taken straight from the S^T accumulators: the
//                          16-wide k step of this product enumerates t in the
//                          order in which a lane holds it, and V^T is read in
//                          the same order with gfx950's transposing LDS read)
// Key/value tiles are copied from HBM straight into a two-stage LDS ring
// (global_load_lds_dwordx4), with 16-byte granules XOR-permuted by row so
// that the fragment reads hit distinct banks.  Every operand is read in place
// from its relation layout through per-sub-dimension strides (power-of-two
// digits), so the blockings the chooser picked for the producers are used as
// they are.
#include <hip/hip_runtime.h>

#include <utility>

#include "device_common.h"
#include "plan.h"

namespace tra {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float floatx16_t __attribute__((ext_vector_type(16)));
typedef float float2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void lds_void_t;

constexpr int AT_BM = 128;   // query rows per workgroup
constexpr int AT_BT = 64;    // key/value rows per tile
constexpr int AT_THREADS = 256;

static __device__ __forceinline__ uint32_t at_lds_addr(const void *p)
{
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void *)p;
}
// LDS reads with a compile-time byte offset in the instruction: a lane's
// fragment addresses then differ only in that offset, so few address
// registers stay live across the loop.
template <int OFF>
static __device__ __forceinline__ u32x4_t at_ds_read16(uint32_t addr)
{
    static_assert(OFF >= 0 && OFF < 65536, "LDS offset field is 16 bits");
    u32x4_t v;
    asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(v) : "v"(addr), "i"(OFF));
    return v;
}
template <int OFF>
static __device__ __forceinline__ u32x2_t at_ds_read8_tr(uint32_t addr)
{
    static_assert(OFF >= 0 && OFF < 65536, "LDS offset field is 16 bits");
    u32x2_t v;
    asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(v) : "v"(addr), "i"(OFF));
    return v;
}
// f(integral_constant<int, i>) for i = 0 .. N-1, unrolled at compile time.
template <typename F, int... I>
static __device__ __forceinline__ void at_static_for(F &&f, std::integer_sequence<int, I...>)
{
    (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
static __device__ __forceinline__ void at_static_for(F &&f)
{
    at_static_for(f, std::make_integer_sequence<int, N>{});
}
// One 16-byte copy from global memory straight into LDS (lane l lands at
// the wave-uniform LDS base + 16 l).
static __device__ __forceinline__ void at_copy16(const uint16_t *g, uint16_t *lds)
{
    __builtin_amdgcn_global_load_lds(g, (lds_void_t *)lds, 16, 0, 0);
}
static __device__ __forceinline__ void at_lds_wait() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }
template <typename T>
static __device__ __forceinline__ void at_ready(T &v)
{
    asm volatile("" : "+v"(v));
}

// 16-byte granule permutations (G granules per row of D bf16).
template <int G>
static __device__ __forceinline__ int swz_key(int t) { return t & (G - 1); }
template <int G>
static __device__ __forceinline__ int swz_val(int t) { return ((t & 7) << 2) & (G - 1); }

template <int D, typename TO>
__global__ __launch_bounds__(AT_THREADS) __attribute__((amdgpu_waves_per_eu(2))) void k_attention(
    AttnDesc a, const uint16_t *__restrict__ q,
                                                          const uint16_t *__restrict__ k,
                                                          const uint16_t *__restrict__ v, TO *__restrict__ o)
{
    constexpr int G = D / 8;                         // granules per row
    constexpr int KS = D / 16;                       // 16-wide k steps of S^T
    constexpr int DB = D / 32;                       // 32-row blocks of O^T
    constexpr int NCP = AT_BT * G / AT_THREADS;      // copies per thread per tile and operand
    __shared__ __attribute__((aligned(16))) uint16_t ks0[AT_BT * D], ks1[AT_BT * D];
    __shared__ __attribute__((aligned(16))) uint16_t vs0[AT_BT * D], vs1[AT_BT * D];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    // Workgroups of one head run on one XCD (consecutive ids go round-robin
    // over the 8 XCDs), so that head's keys and values are read into a single L2.
    const uint32_t n_s = a.S / AT_BM, nb = n_s * a.H;
    uint32_t b = blockIdx.x;
    if (nb % 8 == 0) b = (b % 8) * (nb / 8) + b / 8;
    const uint32_t h = b / n_s, s0 = (b % n_s) * AT_BM;

    const int32_t qh = p2off<0>(a.gh, h), kh = p2off<1>(a.gh, h), vh = p2off<2>(a.gh, h);
    const int32_t oh = p2off<0>(a.gho, h);

    // Q^T fragments (B operand of S^T): lane l holds Q[s][8 (l/32) + 16 ks + e].
    const int col = lane & 31, half = lane >> 5;
    const uint32_t s_mine = s0 + wave * 32 + col;
    u32x4_t qf[KS];
    {
        const int32_t qs = p2off<0>(a.gs, s_mine) + qh;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            qf[ks] = *(const u32x4_t *)(q + qs + p2off<0>(a.gd, 16 * ks + 8 * half));
    }

    // Copy plan: granule p = i * 256 + tid of a tile is row p / G, physical
    // granule p % G; the logical granule (d / 8) is un-permuted here so that
    // the source address carries the permutation.
    int32_t ksrc[NCP], vsrc[NCP];
#pragma unroll
    for (int i = 0; i < NCP; ++i) {
        const int p = i * AT_THREADS + tid, row = p / G, pg = p % G;
        ksrc[i] = p2off<0>(a.gt, row) + kh + p2off<1>(a.gd, 8 * (pg ^ swz_key<G>(row)));
        vsrc[i] = p2off<1>(a.gt, row) + vh + p2off<2>(a.gd, 8 * (pg ^ swz_val<G>(row)));
    }
    auto issue = [&](uint16_t *kst, uint16_t *vst, uint32_t t0) {
        const int32_t kt = p2off<0>(a.gt, t0), vt = p2off<1>(a.gt, t0);
#pragma unroll
        for (int i = 0; i < NCP; ++i) at_copy16(k + ksrc[i] + kt, kst + (i * AT_THREADS + wave * 64) * 8);
#pragma unroll
        for (int i = 0; i < NCP; ++i) at_copy16(v + vsrc[i] + vt, vst + (i * AT_THREADS + wave * 64) * 8);
    };

    floatx16_t acc_o[DB];
#pragma unroll
    for (int j = 0; j < DB; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc_o[j][e] = 0.f;
    float m_run = -INFINITY, l_part = 0.f;
    const float c = a.scale_log2;

    // Per-lane LDS byte offsets of the fragments (the parts that vary with the
    // lane; what varies with the k step, block or key row is an immediate).
    //  K (A operand of S^T): row t = 32 bb + col, granule (2 ks + half) ^ swz(t);
    //    swz(t) depends on col only, so one register per k step.
    //  V (A operand of O^T, transposing read): source lane 4 se + sq of its
    //    16-lane group g reads key row 16 kk + 8 hi + 4 (g/2) + se, columns
    //    32 j + 16 (g%2) + 4 sq .. +3; the row permutation depends on the lane
    //    only, so one register per 32-column block j.
    uint32_t koff[KS], voff[DB];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) koff[ks] = (col * D + 8 * ((2 * ks + half) ^ swz_key<G>(col))) * 2;
    {
        const int g = (lane >> 4) & 3, si = lane & 15, se = si >> 2, sq = si & 3;
        const int t0 = 4 * (g >> 1) + se;
#pragma unroll
        for (int j = 0; j < DB; ++j) {
            const int dcol = 32 * j + 16 * (g & 1) + 4 * sq;
            voff[j] = (t0 * D + 8 * ((dcol >> 3) ^ swz_val<G>(t0)) + (dcol & 7)) * 2;
        }
    }

    auto tile = [&](const uint16_t *kst, const uint16_t *vst) {
        const uint32_t kb = at_lds_addr(kst), vb = at_lds_addr(vst);
        // S^T = K Q^T for the two 32-row blocks of the key tile; the two
        // blocks' accumulation chains are interleaved so that consecutive
        // matrix-core instructions are independent.
        floatx16_t sc[2];
        constexpr int KC = KS < 4 ? KS : 4;   // k steps whose fragments are read together
#pragma unroll
        for (int bb = 0; bb < 2; ++bb)
#pragma unroll
            for (int e = 0; e < 16; ++e) sc[bb][e] = 0.f;
        at_static_for<KS / KC>([&](auto k0c) {
            constexpr int k0 = decltype(k0c)::value * KC;
            u32x4_t kf[2][KC];
            at_static_for<KC>([&](auto ic) {
                constexpr int i = decltype(ic)::value;
                kf[0][i] = at_ds_read16<0>(kb + koff[k0 + i]);
                kf[1][i] = at_ds_read16<32 * D * 2>(kb + koff[k0 + i]);
            });
            at_lds_wait();
#pragma unroll
            for (int i = 0; i < KC; ++i) {
                at_ready(kf[0][i]);
                at_ready(kf[1][i]);
            }
#pragma unroll
            for (int i = 0; i < KC; ++i)
#pragma unroll
                for (int bb = 0; bb < 2; ++bb)
                    sc[bb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, kf[bb][i]),
                                                                     __builtin_bit_cast(bf16x8_t, qf[k0 + i]), sc[bb],
                                                                     0, 0, 0);
        });
        // Online logsumexp over this tile's 64 keys of the lane's query column.
        // The running maximum m used in the exponents moves only when a key
        // exceeds it by more than 2^8 (log2 domain), and then for the whole
        // wave at once: exp2(x - m) stays below 2^8, the sum l and the
        // weighted sum use the same m, so O = (sum p v) / l is unchanged,
        // and most tiles skip rescaling the weighted-sum accumulators.
        float tmax = sc[0][0];
#pragma unroll
        for (int bb = 0; bb < 2; ++bb)
#pragma unroll
            for (int e = 0; e < 16; ++e) tmax = fmaxf(tmax, sc[bb][e]);
        tmax = fmaxf(tmax, __shfl_xor(tmax, 32)) * c;
        if (__builtin_amdgcn_ballot_w64(tmax > m_run + 8.f)) {
            const float m_new = fmaxf(m_run, tmax);
            const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
            m_run = m_new;
            l_part *= alpha;
#pragma unroll
            for (int j = 0; j < DB; ++j)
#pragma unroll
                for (int e = 0; e < 16; ++e) acc_o[j][e] *= alpha;
        }
        const float m_new = m_run;
        float psum = 0.f;
        u32x4_t pf[4];   // P^T fragments: k step 2 bb + hh holds elements 8 hh .. 8 hh + 7 of block bb
#pragma unroll
        for (int bb = 0; bb < 2; ++bb)
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                uint32_t w[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    float2_t pv;
                    pv[0] = __builtin_amdgcn_exp2f(fmaf(sc[bb][8 * hh + 2 * j], c, -m_new));
                    pv[1] = __builtin_amdgcn_exp2f(fmaf(sc[bb][8 * hh + 2 * j + 1], c, -m_new));
                    psum += pv[0] + pv[1];
                    w[j] = __builtin_bit_cast(uint32_t, __builtin_convertvector(pv, bf16x2_t));
                }
                pf[2 * bb + hh] = u32x4_t{w[0], w[1], w[2], w[3]};
            }
        l_part += psum;
        // O^T += V^T P^T.  k step kk covers keys 16 kk .. 16 kk + 15 in the order
        // t = 16 kk + 8 (e'/4) + 4 (l/32) + e'%4 for lane l's element e'.  Per
        // k step, the DB output blocks are independent accumulation chains.
        at_static_for<4>([&](auto kkc) {
            constexpr int kk = decltype(kkc)::value;
            u32x2_t lo[DB], hi[DB];
#pragma unroll
            for (int j = 0; j < DB; ++j) {
                lo[j] = at_ds_read8_tr<16 * kk * D * 2>(vb + voff[j]);
                hi[j] = at_ds_read8_tr<(16 * kk + 8) * D * 2>(vb + voff[j]);
            }
            at_lds_wait();
#pragma unroll
            for (int j = 0; j < DB; ++j) {
                at_ready(lo[j]);
                at_ready(hi[j]);
            }
#pragma unroll
            for (int j = 0; j < DB; ++j) {
                const u32x4_t af = {lo[j][0], lo[j][1], hi[j][0], hi[j][1]};
                acc_o[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, af),
                                                                   __builtin_bit_cast(bf16x8_t, pf[kk]), acc_o[j],
                                                                   0, 0, 0);
            }
        });
    };
    auto barrier = [&]() {
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
    };

    // Two-stage ring: wait for this thread's copies of tile j, make every
    // thread's copies visible (the barrier also ends every wave's reads of
    // tile j-1, whose stage then takes tile j+1), then compute on tile j.
    // One loop body with the stage chosen at run time: the per-lane fragment
    // addresses are then held once, not once per stage.
    const uint32_t nt = a.T / AT_BT;
    issue(ks0, vs0, 0);
    for (uint32_t j = 0; j < nt; ++j) {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        barrier();
        const bool odd = j & 1;
        if (j + 1 < nt) issue(odd ? ks0 : ks1, odd ? vs0 : vs1, (j + 1) * AT_BT);
        tile(odd ? ks1 : ks0, odd ? vs1 : vs0);
    }

    // O = O^T / l: lane l holds O[s][32 j + 8 (e/4) + 4 (l/32) + e%4].
    const float l_tot = l_part + __shfl_xor(l_part, 32);
    const float inv = 1.f / l_tot;
    const int32_t os = p2off<1>(a.gs, s_mine) + oh;
#pragma unroll
    for (int jj = 0; jj < DB; ++jj)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int d0 = 32 * jj + 8 * r + 4 * half;
            const int32_t off = os + p2off<0>(a.gdo, d0);
            if constexpr (std::is_same<TO, bf16_t>::value) {
                if (a.o_vec4) {
                    float2_t p0 = {acc_o[jj][4 * r] * inv, acc_o[jj][4 * r + 1] * inv};
                    float2_t p1 = {acc_o[jj][4 * r + 2] * inv, acc_o[jj][4 * r + 3] * inv};
                    const u32x2_t w = {__builtin_bit_cast(uint32_t, __builtin_convertvector(p0, bf16x2_t)),
                                       __builtin_bit_cast(uint32_t, __builtin_convertvector(p1, bf16x2_t))};
                    *(u32x2_t *)(o + off) = w;
                    continue;
                }
            } else {
                if (a.o_vec4) {
                    *(float4 *)(o + off) = make_float4(acc_o[jj][4 * r] * inv, acc_o[jj][4 * r + 1] * inv,
                                                       acc_o[jj][4 * r + 2] * inv, acc_o[jj][4 * r + 3] * inv);
                    continue;
                }
            }
#pragma unroll
            for (int e = 0; e < 4; ++e)
                Scalar<TO>::store(o, os + p2off<0>(a.gdo, d0 + e), acc_o[jj][4 * r + e] * inv);
        }
}

#define TRA_ATT_INST(D, TO)                                                                                 \
    template __global__ void k_attention<D, TO>(AttnDesc, const uint16_t *, const uint16_t *, const uint16_t *, \
                                                TO *);
TRA_ATT_INST(32, bf16_t)
TRA_ATT_INST(64, bf16_t)
TRA_ATT_INST(128, bf16_t)
TRA_ATT_INST(32, float)
TRA_ATT_INST(64, float)
TRA_ATT_INST(128, float)
#undef TRA_ATT_INST

template <int D, typename TO>
static int launch_att(const AttnDesc &a, const void *q, const void *k, const void *v, void *o, hipStream_t s)
{
    hipLaunchKernelGGL((k_attention<D, TO>), dim3((a.S / AT_BM) * a.H), dim3(AT_THREADS), 0, s, a,
                       (const uint16_t *)q, (const uint16_t *)k, (const uint16_t *)v, (TO *)o);
    return (int)hipGetLastError();
}

int launch_attention(const AttnDesc &a, int out_dtype, const void *q, const void *k, const void *v, void *o,
                     void *stream)
{
    hipStream_t s = (hipStream_t)stream;
    const bool bf = out_dtype == D_BF16;
    switch (a.D) {
    case 32: return bf ? launch_att<32, bf16_t>(a, q, k, v, o, s) : launch_att<32, float>(a, q, k, v, o, s);
    case 64: return bf ? launch_att<64, bf16_t>(a, q, k, v, o, s) : launch_att<64, float>(a, q, k, v, o, s);
    case 128: return bf ? launch_att<128, bf16_t>(a, q, k, v, o, s) : launch_att<128, float>(a, q, k, v, o, s);
    default: return (int)hipErrorInvalidValue;
    }
}

}  // namespace tra
