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
// sub-dimension strides, copied straight from HBM into a four-stage LDS ring
// (global_load_lds_dwordx4: no register staging, three k-tiles in flight).
// An operand stored contiguously along the contracted labels ("K-major") is
// staged as [row][k] and fed to the matrix cores with 16-byte LDS reads; one
// stored contiguously along its output labels ("MN-major") is staged as
// [k][row] exactly as it arrives and transposed on the way to the matrix
// cores by gfx950's ds_read_b64_tr_b16.  Either operand may be either: a
// product with a transposed operand (X^T Y, X Y^T, the backward products of
// a matmul) runs on the same kernel.
#include <hip/hip_runtime.h>

#include <cstdlib>
#include <type_traits>
#include <utility>

// k-tiles the four-wave tile keeps in its LDS ring (32 KiB each)
#ifndef TRA_MFMA4_STAGES
#define TRA_MFMA4_STAGES 4
#endif

#include "mfma_common.h"

namespace tra {

TileShape mfma_tile_shape(int variant)
{
    if (variant == 4) return {256, 256, 64};
    if (variant == 5) return {256, 128, 64};   // the 64-deep tile, 128 columns
    if (variant == 3) return {256, 256, MF_BK};
    if (variant < 0 || variant > 2) return {0, 0, 0};
    MfmaCfg c = mfma_cfg(variant);
    return {c.bm, c.bn, MF_BK};
}

// The tile kernel's body.  TC is void for a plain product; otherwise the
// epilogue applies the two elementwise steps of a ChainEpi to each element
// (TC = their intermediate dtype) instead of storing the product.
template <int V, bool AKM, bool BKM, typename TO, typename TC, int CH = 0>
__device__ __forceinline__ void mfma_body(const GemmView &v, const uint16_t *__restrict__ x,
                                          const uint16_t *__restrict__ y, TO *__restrict__ z,
                                          float *__restrict__ ws, const ChainEpi &ce)
{
    constexpr MfmaCfg C = mfma_cfg(V);
    constexpr int BM = C.bm, BN = C.bn, BK = MF_BK, WM = C.wm, WN = C.wn;
    constexpr int NT = WM * WN * 64;
    constexpr int TM = BM / WM / 32, TN = BN / WN / 32;
    // one array per stage: the compiler can then see that a load into one
    // stage does not touch the stage being read
    __shared__ __attribute__((aligned(16))) uint16_t sa0[BM * BK], sa1[BM * BK], sa2[BM * BK], sa3[BM * BK];
    __shared__ __attribute__((aligned(16))) uint16_t sb0[BN * BK], sb1[BN * BK], sb2[BN * BK], sb3[BN * BK];
    // stage index -> array (always called with a constant, so it folds away)
    auto SA = [&](int G) -> uint16_t * { return G == 0 ? sa0 : G == 1 ? sa1 : G == 2 ? sa2 : sa3; };
    auto SB = [&](int G) -> uint16_t * { return G == 0 ? sb0 : G == 1 ? sb1 : G == 2 ? sb2 : sb3; };

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / WN, wn = wave % WN;
    const uint32_t tiles_n = v.gn.total / BN;
    const uint32_t nb = (v.gm.total / BM) * tiles_n;
    uint32_t tm, tn, bidx;
    mfma_tile_of(nb, tiles_n, v.gb.total, bidx, tm, tn);
    const uint32_t m0 = tm * BM, n0 = tn * BN;
    const int32_t bx = p2off<0>(v.gb, bidx), by = p2off<1>(v.gb, bidx), bz = p2off<2>(v.gb, bidx);
    const uint32_t kbeg = blockIdx.z * (uint32_t)v.k_per_split;
    const uint32_t nk = (uint32_t)v.k_per_split / BK;

    DmaPlan<BM, NT, AKM, 0> da;
    DmaPlan<BN, NT, BKM, 1> db;
    da.init(v.gm, v.gk, m0, bx, tid);
    db.init(v.gn, v.gk, n0, by, tid);
    constexpr int L = DmaPlan<BM, NT, AKM, 0>::N + DmaPlan<BN, NT, BKM, 1>::N;

    floatx16_t acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

    const int r_lane = lane & 31, k_lane = (lane >> 5) * 8;
    const int a_row0 = wm * (BM / WM) + r_lane;
    const int b_col0 = wn * (BN / WN);

    auto issue = [&](int stg, uint32_t t) {
        const uint32_t k0 = kbeg + t * BK;
        da.issue(x, p2off<0>(v.gk, k0), SA(stg), wave);
        db.issue(y, p2off<1>(v.gk, k0), SB(stg), wave);
    };
    // Both k-steps of a stage: all fragment reads first, one wait, then the
    // matrix-core work.
    auto compute = [&](int stg) {
        const uint32_t a_b = lds_addr(SA(stg)), b_b = lds_addr(SB(stg));
        u32x4_t af[2][TM];
        u32x2_t at[2][TM][2];
        u32x4_t bk[2][TN];
        u32x2_t bt[2][TN][2];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
            for (int i = 0; i < TM; ++i) {
                if constexpr (AKM) {
                    const int r = a_row0 + i * 32, c = ((ks * 16 + k_lane) >> 3) ^ swz_k(r);
                    af[ks][i] = ds_read16(a_b + (r * MF_BK + c * 8) * 2);
                } else {
                    // [k][row] stage: the transposing read hands lane l the
                    // eight k of row l%32 (rows play the part the columns
                    // play for an MN-major Y)
                    const int g = lane >> 4, sl = lane & 15;
                    const int kb = ks * 16 + 8 * (g >> 1) + (sl >> 2);
                    const int mb = wm * (BM / WM) + i * 32 + 16 * (g & 1) + 4 * (sl & 3);
                    const uint32_t e0 = kb * BM + (((mb >> 3) ^ swz_n<BM>(kb)) << 3) + (mb & 7);
                    at[ks][i][0] = ds_read8_tr(a_b + e0 * 2);
                    at[ks][i][1] = ds_read8_tr(a_b + (e0 + 4 * BM) * 2);
                }
            }
#pragma unroll
            for (int j = 0; j < TN; ++j) {
                if constexpr (BKM) {
                    const int r = b_col0 + j * 32 + r_lane, c = ((ks * 16 + k_lane) >> 3) ^ swz_k(r);
                    bk[ks][j] = ds_read16(b_b + (r * MF_BK + c * 8) * 2);
                } else {
                    const int g = lane >> 4, sl = lane & 15;
                    const int kb = ks * 16 + 8 * (g >> 1) + (sl >> 2);
                    const int nb = b_col0 + j * 32 + 16 * (g & 1) + 4 * (sl & 3);
                    const uint32_t e0 = kb * BN + (((nb >> 3) ^ swz_n<BN>(kb)) << 3) + (nb & 7);
                    bt[ks][j][0] = ds_read8_tr(b_b + e0 * 2);
                    bt[ks][j][1] = ds_read8_tr(b_b + (e0 + 4 * BN) * 2);
                }
            }
        }
        lds_wait_all();
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
            for (int i = 0; i < TM; ++i) {
                if constexpr (AKM) {
                    lds_ready(af[ks][i]);
                } else {
                    lds_ready(at[ks][i][0]);
                    lds_ready(at[ks][i][1]);
                }
            }
#pragma unroll
            for (int j = 0; j < TN; ++j) {
                if constexpr (BKM) {
                    lds_ready(bk[ks][j]);
                } else {
                    lds_ready(bt[ks][j][0]);
                    lds_ready(bt[ks][j][1]);
                }
            }
        }
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j) {
                    bf16x8_t a;
                    if constexpr (AKM) {
                        a = __builtin_bit_cast(bf16x8_t, af[ks][i]);
                    } else {
                        u32x4_t w = {at[ks][i][0][0], at[ks][i][0][1], at[ks][i][1][0], at[ks][i][1][1]};
                        a = __builtin_bit_cast(bf16x8_t, w);
                    }
                    bf16x8_t b;
                    if constexpr (BKM) {
                        b = __builtin_bit_cast(bf16x8_t, bk[ks][j]);
                    } else {
                        u32x4_t w = {bt[ks][j][0][0], bt[ks][j][0][1], bt[ks][j][1][0], bt[ks][j][1][1]};
                        b = __builtin_bit_cast(bf16x8_t, w);
                    }
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[i][j], 0, 0, 0);
                }
    };
    // The copy is issued unconditionally: past the last k-tile it re-reads that
    // tile into the free stage (never consumed), which keeps the number of
    // copies in flight, and so the wait below, the same at every step.
    auto step = [&](int G, uint32_t t) {
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * L));
        // the barrier intrinsic does not order memory for the optimiser: keep
        // every LDS access on its side of it
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        issue((G + 3) % MF_STAGES, min(t + 3, nk - 1));
        compute(G);
    };
    issue(0, 0);
    issue(1, min(1u, nk - 1));
    issue(2, min(2u, nk - 1));
    uint32_t t = 0;
    for (; t + MF_STAGES <= nk; t += MF_STAGES) {
        step(0, t);
        step(1, t + 1);
        step(2, t + 2);
        step(3, t + 3);
    }
    if (t < nk) step(0, t);
    if (t + 1 < nk) step(1, t + 1);
    if (t + 2 < nk) step(2, t + 2);

    // Epilogue.  Accumulator element e of lane l holds row
    // 8*(e/4) + 4*(l/32) + e%4 and column l%32 of its 32x32 block.
    // row = (wave row + 32 i + 8 (e/4)) + (4 (l/32) + e%4): a multiple of 8 plus
    // a part below 8, so its offset splits into a wave-uniform and a lane part
    // (likewise the column into the block's and the lane's).  The loops are
    // unrolled at compile time: an accumulator indexed at run time would live
    // in scratch memory.
    const bool split = v.split > 1;
    float *wsp = split ? ws + (int64_t)blockIdx.z * v.z_elems : nullptr;
    const int32_t zm0 = p2off<1>(v.gm, m0) + bz, zn0 = p2off<1>(v.gn, n0);
    int32_t lo[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) lo[r] = p2off<1>(v.gm, 4 * (lane >> 5) + r);
    if constexpr (std::is_void<TC>::value) {
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
    } else {
        // The product as the fp32 output it would be stored as, then the two
        // elementwise steps exactly as the chained elementwise kernel computes
        // them.  The row operand's offset splits like the output's.  CH = 1
        // is the pair (x - y, then x * y) with the joins fixed at compile time
        // (the softmax Jacobian of the attention backward); CH = 0 takes any
        // pair, branching on the joins per element.
        const int32_t rm0 = p2off<0>(ce.rb, bidx) + p2off<0>(ce.rm, m0) + p2off<0>(ce.rn, n0);
        int32_t rlo[4], ron[TN], zon[TN];
#pragma unroll
        for (int r = 0; r < 4; ++r) rlo[r] = p2off<0>(ce.rm, 4 * (lane >> 5) + r);
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            ron[j] = p2off<0>(ce.rn, b_col0 + j * 32 + r_lane);
            zon[j] = zn0 + p2off<1>(v.gn, b_col0 + j * 32 + r_lane);
        }
        const float *__restrict__ ya = (const float *)ce.ya;
        const TC *__restrict__ xb = (const TC *)ce.xb;
        // Rows are done in groups of TN * 4 elements (one (i, q) pair).  The
        // two operands of group g + 1 are loaded before group g is computed
        // and stored, so each group's loads are in flight together and under
        // the previous group's work instead of one element at a time (a load
        // cannot be moved above a store the compiler cannot prove disjoint).
        constexpr int GE = TN * 4;
        float yv[2][GE], xv[2][GE];
        auto load_group = [&](auto IQ, int buf) {
            constexpr int i = decltype(IQ)::value / 4, q = decltype(IQ)::value % 4;
            const int32_t row = wm * (BM / WM) + i * 32 + 8 * q;
            const int32_t hi = zm0 + p2off<1>(v.gm, row), rhi = rm0 + p2off<0>(ce.rm, row);
            sfor<GE>([&](auto JR) {
                constexpr int j = decltype(JR)::value / 4, r = decltype(JR)::value % 4;
                yv[buf][decltype(JR)::value] = ya[rhi + rlo[r] + ron[j]];
                xv[buf][decltype(JR)::value] = Scalar<TC>::load(xb, hi + lo[r] + zon[j]);
            });
        };
        load_group(std::integral_constant<int, 0>{}, 0);
        sfor<TM * 4>([&](auto IQ) {
            constexpr int g = decltype(IQ)::value, i = g / 4, q = g % 4, buf = g % 2;
            if constexpr (g + 1 < TM * 4) load_group(std::integral_constant<int, g + 1>{}, 1 - buf);
            const int32_t hi = zm0 + p2off<1>(v.gm, wm * (BM / WM) + i * 32 + 8 * q);
            sfor<GE>([&](auto JR) {
                constexpr int e = decltype(JR)::value, j = e / 4, r = e % 4;
                const float av = acc[i][j][4 * q + r] * v.post_scale;
                float t;
                if constexpr (CH == 1) t = (av - yv[buf][e]) * ce.scale_a;
                else t = join_any(ce.join_a, av, yv[buf][e]) * ce.scale_a;
                if constexpr (std::is_same<TC, bf16_t>::value) t = bf16_to_f32(f32_to_bf16(t));
                float o;
                if constexpr (CH == 1) o = xv[buf][e] * t;
                else o = join_any(ce.join_b, xv[buf][e], t);
                Scalar<TO>::store(z, hi + lo[r] + zon[j], o * ce.scale_b);
            });
        });
    }
}

// EPI: 0 the direct epilogue, 1 the staged one, 2 the staged chained one
// (CH, YROW as for mfma4_chain_staged; ce used only then).
template <bool AKM, bool BKM, typename TO, int STAGES, int EPI, int CH = 0, bool YROW = false>
__device__ __forceinline__ void mfma4_body(const GemmView &v, const uint16_t *__restrict__ x,
                                           const uint16_t *__restrict__ y, TO *__restrict__ z,
                                           float *__restrict__ ws, const ChainEpi &ce)
{
    using namespace mf4;
    // the operand stages (the epilogue reuses them as a staging tile)
    __shared__ __attribute__((aligned(16))) uint16_t sa[STAGES * BM * BK];
    __shared__ __attribute__((aligned(16))) uint16_t sb[STAGES * BN * BK];
    static_assert(STAGES * BM * BK * 2 >= 64 * BN * 4 && STAGES * BN * BK * 2 >= 64 * BN * 4,
                  "each operand's stages hold 64 staged rows");

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / WN, wn = wave % WN;
    const uint32_t tiles_n = v.gn.total / BN;
    const uint32_t nb = (v.gm.total / BM) * tiles_n;
    uint32_t tm, tn, bidx;
    mfma_tile_of(nb, tiles_n, v.gb.total, bidx, tm, tn);
    const uint32_t m0 = tm * BM, n0 = tn * BN;
    const int32_t bx = p2off<0>(v.gb, bidx), by = p2off<1>(v.gb, bidx), bz = p2off<2>(v.gb, bidx);
    const uint32_t kbeg = blockIdx.z * (uint32_t)v.k_per_split;
    const uint32_t nk = (uint32_t)v.k_per_split / BK;

    DmaPlan<BM, NT, AKM, 0> da;
    DmaPlan<BN, NT, BKM, 1> db;
    da.init(v.gm, v.gk, m0, bx, tid);
    db.init(v.gn, v.gk, n0, by, tid);
    constexpr int L = DmaPlan<BM, NT, AKM, 0>::N + DmaPlan<BN, NT, BKM, 1>::N;

    FragAddr4<AKM, BM, WM, STAGES> fa;
    FragAddr4<BKM, BN, WN, STAGES> fb;
    fa.init(lds_addr(sa), wm, lane);
    fb.init(lds_addr(sb), wn, lane);

    floatx16_t acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

    auto issue = [&](int stg, uint32_t t) {
        const uint32_t k0 = kbeg + t * BK;
        da.issue(x, p2off<0>(v.gk, k0), sa + stg * BM * BK, wave);
        db.issue(y, p2off<1>(v.gk, k0), sb + stg * BN * BK, wave);
    };
    auto mma = [&](const Frag4<AKM, TM> &A, const Frag4<BKM, TN> &B) {
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A.op(i), B.op(j), acc[i][j], 0, 0, 0);
    };
    // Two fragment sets: F0 holds k-step 0 of a stage, F1 k-step 1.
    Frag4<AKM, TM> A0, A1;
    Frag4<BKM, TN> B0, B1;
    constexpr int NA = Frag4<AKM, TM>::reads;

    // Step of stage G (k-tile t): k-step 0 computes from A0/B0 while k-step 1
    // is read into A1/B1; then the next stage is published (its copies
    // waited for, a barrier) and the copy of k-tile t + STAGES - 1 issued into
    // the stage freed by k-tile t - 1; then k-step 1 computes while k-step 0
    // of the next stage is read.  Each "wait for the older reads" leaves only
    // the newest NA reads (the next A fragments) in flight.
    auto publish = [&](int G, uint32_t t) {
        __builtin_amdgcn_s_waitcnt(vmcnt_imm((STAGES - 3) * L));
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        issue((G + STAGES - 1) % STAGES, min(t + STAGES - 1, nk - 1));
    };
    constexpr int NB_ = Frag4<BKM, TN>::reads;
    constexpr int LA = DmaPlan<BM, NT, AKM, 0>::N, LB = DmaPlan<BN, NT, BKM, 1>::N;
    static_assert(NA + NB_ <= TM * TN && LA + LB <= TM * TN, "one read and one copy per product slot");
    // One k-step of the loop body: the 16 products on (Ac, Bc), one per slot;
    // in the slots, in this order, the reads of the next k-step (stage GR,
    // k-step KR) into (An, Bn); when COPY, the copies into stage GC from the
    // operand offsets (ka, kb); when !COPY, one digit per slot of the offsets
    // (ka, kb) of k-tile `tc` (scalar work that then runs under the
    // products instead of delaying the barrier).  The scheduler may not move
    // anything across a slot boundary, so the reads run under the products
    // instead of ahead of their wait.  Every read of (Ac, Bc) was issued
    // during the previous k-step.
    auto kstep = [&](auto GR, auto KR, auto COPY, auto GC, const Frag4<AKM, TM> &Ac, const Frag4<BKM, TN> &Bc,
                     Frag4<AKM, TM> &An, Frag4<BKM, TN> &Bn, uint32_t tc, int32_t &ka, int32_t &kb) {
        constexpr int gr = decltype(GR)::value, kr = decltype(KR)::value, gc = decltype(GC)::value;
        constexpr bool copy = decltype(COPY)::value;
        const uint32_t k0 = kbeg + tc * BK;
        if constexpr (!copy) {
            ka = 0;
            kb = 0;
        }
        __builtin_amdgcn_sched_barrier(0);
        sfor<TM * TN>([&](auto MC) {
            constexpr int m = decltype(MC)::value, i = m / TN, j = m % TN;
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(Ac.op(i), Bc.op(j), acc[i][j], 0, 0, 0);
            if constexpr (m < NA) fa.template read_one<gr, kr, m>(An);
            else if constexpr (m < NA + NB_) fb.template read_one<gr, kr, m - NA>(Bn);
            if constexpr (copy && m < LA) da.issue_one(m, x, ka, sa + gc * BM * BK, wave);
            else if constexpr (copy && m < LA + LB) db.issue_one(m - LA, y, kb, sb + gc * BN * BK, wave);
            if constexpr (!copy && m < kP2Max) {
                ka += (int32_t)((k0 >> v.gk.sh[m]) & v.gk.mask[m]) * v.gk.st[0][m];
                kb += (int32_t)((k0 >> v.gk.sh[m]) & v.gk.mask[m]) * v.gk.st[1][m];
            }
            __builtin_amdgcn_sched_barrier(0);
        });
    };
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using NoCopy = std::integral_constant<bool, false>;
    using Copy = std::integral_constant<bool, true>;
    // Step of stage G (k-tile t) in the loop body: k-step 0 computes from
    // A0/B0 while k-step 1 is read into A1/B1 (and the operand offsets of
    // k-tile t + STAGES - 1 are formed); then the next stage is published (its
    // copies waited for, a barrier); then k-step 1 computes while k-step 0 of
    // the next stage is read and the copy of k-tile t + STAGES - 1 goes into
    // the stage freed by k-tile t - 1.
    auto step = [&](auto GC, uint32_t t) {
        constexpr int G = decltype(GC)::value;
        constexpr int GN = (G + 1) % STAGES, GF = (G + STAGES - 1) % STAGES;
        int32_t ka, kb;
        lds_wait<0>();
        A0.ready();
        B0.ready();
        kstep(GC, I1{}, NoCopy{}, I0{}, A0, B0, A1, B1, min(t + STAGES - 1, nk - 1), ka, kb);
        __builtin_amdgcn_s_waitcnt(vmcnt_imm((STAGES - 3) * L));
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        lds_wait<0>();
        A1.ready();
        B1.ready();
        kstep(std::integral_constant<int, GN>{}, I0{}, Copy{}, std::integral_constant<int, GF>{}, A1, B1, A0, B0,
              0u, ka, kb);
    };
    // Step of the tail (fewer than STAGES k-tiles left): the same work, but
    // every read is waited for within the step, so that no read is in flight
    // across the branch that skips the steps past the last k-tile.  A0/B0
    // arrive ready.
    auto tail_step = [&](auto GC, uint32_t t) {
        constexpr int G = decltype(GC)::value;
        fa.template read<G, 1>(A1);
        fb.template read<G, 1>(B1);
        mma(A0, B0);
        lds_wait<0>();
        A1.ready();
        B1.ready();
        publish(G, t);
        mma(A1, B1);
        if (t + 1 < nk) {
            fa.template read<G + 1, 0>(A0);
            fb.template read<G + 1, 0>(B0);
            lds_wait<0>();
            A0.ready();
            B0.ready();
        }
    };

    // prologue: STAGES - 1 k-tiles in flight, the first stage's first k-step read
#pragma unroll
    for (int s = 0; s < STAGES - 1; ++s) issue(s, min((uint32_t)s, nk - 1));
    __builtin_amdgcn_s_waitcnt(vmcnt_imm((STAGES - 2) * L));
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    fa.template read<0, 0>(A0);
    fb.template read<0, 0>(B0);
    lds_wait<0>();
    A0.ready();
    B0.ready();

    // The loop body runs STAGES k-tiles; every fragment read it issues is
    // waited for inside it, except those of the next body's first k-step,
    // which are waited for (and handed on through lds_ready) before the
    // back-edge, so that no read is in flight at a branch or merge and no
    // register copy can take one in flight.
    uint32_t t = 0;
    for (; t + STAGES <= nk; t += STAGES) {
        sfor<STAGES>([&](auto GC) { step(GC, t + decltype(GC)::value); });
        lds_wait<0>();
        A0.ready();
        B0.ready();
    }
    sfor<STAGES - 1>([&](auto GC) {
        constexpr int G = decltype(GC)::value;
        if (t + G < nk) tail_step(GC, t + G);
    });
    // nothing may stay in flight past the k-loop
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    lds_wait<0>();

    // Epilogue.  Accumulator element e of lane l holds row
    // 8*(e/4) + 4*(l/32) + e%4 and column l%32 of its 32x32 block.
    const bool split = v.split > 1;
    float *wsp = split ? ws + (int64_t)blockIdx.z * v.z_elems : nullptr;
    if constexpr (EPI == 2) {
        lds_barrier();   // every wave past its last read of the operand stages
        mfma4_chain_staged<TO, CH, YROW>(v, z, ce, acc, lds_addr(sa), lds_addr(sb), m0, n0, bidx, bz, wave, lane);
        return;
    } else if constexpr (EPI == 1) {
        lds_barrier();
        if (split) mfma4_store_staged<float, false>(v, wsp, acc, lds_addr(sa), lds_addr(sb), m0, n0, bz, wave, lane);
        else mfma4_store_staged<TO, true>(v, z, acc, lds_addr(sa), lds_addr(sb), m0, n0, bz, wave, lane);
        return;
    }
    mfma4_store_direct<TO>(v, z, wsp, split, acc, m0, n0, bz, wave);
}

// VEC: the staged epilogue (the output's four consecutive columns form one
// aligned vector, and z / the workspace are 16-byte aligned)
template <bool AKM, bool BKM, typename TO, bool VEC>
__global__ __launch_bounds__(mf4::NT) void k_mfma4_bf16(GemmView v, const uint16_t *__restrict__ x,
                                                        const uint16_t *__restrict__ y, TO *__restrict__ z,
                                                        float *__restrict__ ws)
{
    mfma4_body<AKM, BKM, TO, TRA_MFMA4_STAGES, VEC ? 1 : 0>(v, x, y, z, ws, ChainEpi{});
}

// The product with a chain of two elementwise steps in its staged epilogue
// (tra_execute_contract_chain on the four-wave tile)
template <bool AKM, bool BKM, typename TO, int CH, bool YROW>
__global__ __launch_bounds__(mf4::NT) void k_mfma4_chain(GemmView v, const uint16_t *__restrict__ x,
                                                         const uint16_t *__restrict__ y, TO *__restrict__ z,
                                                         ChainEpi ce)
{
    mfma4_body<AKM, BKM, TO, TRA_MFMA4_STAGES, 2, CH, YROW>(v, x, y, z, nullptr, ce);
}

template <int V, bool AKM, bool BKM, typename TO>
__global__ __launch_bounds__(mfma_cfg(V).wm *mfma_cfg(V).wn * 64) void k_mfma_bf16(
    GemmView v, const uint16_t *__restrict__ x, const uint16_t *__restrict__ y, TO *__restrict__ z,
    float *__restrict__ ws)
{
    mfma_body<V, AKM, BKM, TO, void>(v, x, y, z, ws, ChainEpi{});
}

template <int V, bool AKM, bool BKM, typename TO, int CH>
__global__ __launch_bounds__(mfma_cfg(V).wm *mfma_cfg(V).wn * 64) void k_mfma_chain(
    GemmView v, const uint16_t *__restrict__ x, const uint16_t *__restrict__ y, TO *__restrict__ z, ChainEpi ce)
{
    mfma_body<V, AKM, BKM, TO, TO, CH>(v, x, y, z, nullptr, ce);
}

// Every (tile, operand layout, output dtype) combination the launcher can
// pick, instantiated explicitly (the host pass otherwise emits only some).
#define TRA_MFMA_INST(V, AKM, BKM, TO)                                                                         \
    template __global__ void k_mfma_bf16<V, AKM, BKM, TO>(GemmView, const uint16_t *, const uint16_t *, TO *,    \
                                                          float *);
#define TRA_MFMA_INST4(V, TO)                                                                                  \
    TRA_MFMA_INST(V, true, true, TO)                                                                           \
    TRA_MFMA_INST(V, true, false, TO)                                                                          \
    TRA_MFMA_INST(V, false, true, TO)                                                                          \
    TRA_MFMA_INST(V, false, false, TO)
TRA_MFMA_INST4(0, float)
TRA_MFMA_INST4(0, bf16_t)
TRA_MFMA_INST4(1, float)
TRA_MFMA_INST4(1, bf16_t)
TRA_MFMA_INST4(2, float)
TRA_MFMA_INST4(2, bf16_t)
#undef TRA_MFMA_INST4
#undef TRA_MFMA_INST
#define TRA_MFMA4_INST(AKM, BKM, TO)                                                                          \
    template __global__ void k_mfma4_bf16<AKM, BKM, TO, false>(GemmView, const uint16_t *, const uint16_t *, TO *,  \
                                                               float *);                                           \
    template __global__ void k_mfma4_bf16<AKM, BKM, TO, true>(GemmView, const uint16_t *, const uint16_t *, TO *,   \
                                                              float *);
TRA_MFMA4_INST(true, true, float)
TRA_MFMA4_INST(true, false, float)
TRA_MFMA4_INST(false, true, float)
TRA_MFMA4_INST(false, false, float)
TRA_MFMA4_INST(true, true, bf16_t)
TRA_MFMA4_INST(true, false, bf16_t)
TRA_MFMA4_INST(false, true, bf16_t)
TRA_MFMA4_INST(false, false, bf16_t)
#undef TRA_MFMA4_INST
#define TRA_MFMA4C_INST(TO, CH, YROW)                                                                       \
    template __global__ void k_mfma4_chain<true, true, TO, CH, YROW>(GemmView, const uint16_t *,            \
                                                                     const uint16_t *, TO *, ChainEpi);       \
    template __global__ void k_mfma4_chain<true, false, TO, CH, YROW>(GemmView, const uint16_t *,           \
                                                                      const uint16_t *, TO *, ChainEpi);      \
    template __global__ void k_mfma4_chain<false, true, TO, CH, YROW>(GemmView, const uint16_t *,           \
                                                                      const uint16_t *, TO *, ChainEpi);      \
    template __global__ void k_mfma4_chain<false, false, TO, CH, YROW>(GemmView, const uint16_t *,          \
                                                                       const uint16_t *, TO *, ChainEpi);
TRA_MFMA4C_INST(float, 0, false)
TRA_MFMA4C_INST(float, 1, false)
TRA_MFMA4C_INST(float, 1, true)
TRA_MFMA4C_INST(bf16_t, 0, false)
TRA_MFMA4C_INST(bf16_t, 1, false)
TRA_MFMA4C_INST(bf16_t, 1, true)
#undef TRA_MFMA4C_INST


int launch_split_fold(const tra_plan_s &p, const void *ws, void *z, void *stream);

template <int V, bool AKM, bool BKM, typename TO>
static int launch_v(const tra_plan_s &p, const void *x, const void *y, void *z, void *ws, hipStream_t s)
{
    constexpr MfmaCfg C = mfma_cfg(V);
    const GemmView &v = p.gv;
    dim3 grid((v.gm.total / C.bm) * (v.gn.total / C.bn), v.gb.total, v.split);
    // naming the kernel through a pointer makes the host pass emit its launch
    // stub for every instantiation
    void (*kern)(GemmView, const uint16_t *, const uint16_t *, TO *, float *) = k_mfma_bf16<V, AKM, BKM, TO>;
    hipLaunchKernelGGL(kern, grid, dim3(C.wm * C.wn * 64), 0, s, v, (const uint16_t *)x, (const uint16_t *)y,
                       (TO *)z, (float *)ws);
    return (int)hipGetLastError();
}

// TRA_MFMA4_CHAIN=0 keeps the product chain on the eight-wave tile (for A/B runs)
static bool chain4_enabled()
{
    static const bool on = [] {
        const char *e = getenv("TRA_MFMA4_CHAIN");
        return !(e && e[0] == '0');
    }();
    return on;
}

// TRA_MFMA4_VEC_EPILOGUE=0 keeps the direct epilogue everywhere (for A/B runs)
static bool vec_epilogue_enabled()
{
    static const bool on = [] {
        const char *e = getenv("TRA_MFMA4_VEC_EPILOGUE");
        return !(e && e[0] == '0');
    }();
    return on;
}

template <bool AKM, bool BKM, typename TO>
static int launch4(const tra_plan_s &p, const void *x, const void *y, void *z, void *ws, hipStream_t s)
{
    const GemmView &v = p.gv;
    dim3 grid((v.gm.total / mf4::BM) * (v.gn.total / mf4::BN), v.gb.total, v.split);
    // the staged epilogue when the output's column vectors are aligned in
    // memory (z for a plain product, the workspace for a split)
    const void *out = v.split > 1 ? ws : z;
    const bool vec = v.z_vec4 && ((uintptr_t)out % 16) == 0 && vec_epilogue_enabled();
    void (*kern)(GemmView, const uint16_t *, const uint16_t *, TO *, float *) =
        vec ? k_mfma4_bf16<AKM, BKM, TO, true> : k_mfma4_bf16<AKM, BKM, TO, false>;
    hipLaunchKernelGGL(kern, grid, dim3(mf4::NT), 0, s, v, (const uint16_t *)x, (const uint16_t *)y, (TO *)z,
                       (float *)ws);
    return (int)hipGetLastError();
}

template <int V, typename TO>
static int launch_layout(const tra_plan_s &p, const void *x, const void *y, void *z, void *ws, hipStream_t s)
{
    if constexpr (V == 3) {
        if (p.a_kmajor) {
            if (p.b_kmajor) return launch4<true, true, TO>(p, x, y, z, ws, s);
            return launch4<true, false, TO>(p, x, y, z, ws, s);
        }
        if (p.b_kmajor) return launch4<false, true, TO>(p, x, y, z, ws, s);
        return launch4<false, false, TO>(p, x, y, z, ws, s);
    } else {
        if (p.a_kmajor) {
            if (p.b_kmajor) return launch_v<V, true, true, TO>(p, x, y, z, ws, s);
            return launch_v<V, true, false, TO>(p, x, y, z, ws, s);
        }
        if (p.b_kmajor) return launch_v<V, false, true, TO>(p, x, y, z, ws, s);
        return launch_v<V, false, false, TO>(p, x, y, z, ws, s);
    }
}

template <typename TO>
static int launch_tile(const tra_plan_s &p, const void *x, const void *y, void *z, void *ws, hipStream_t s)
{
    switch (p.tile) {
    case 0: return launch_layout<0, TO>(p, x, y, z, ws, s);
    case 1: return launch_layout<1, TO>(p, x, y, z, ws, s);
    case 3: return launch_layout<3, TO>(p, x, y, z, ws, s);
    case 4:
    case 5: return launch_mfma4k(p, x, y, z, ws, s, std::is_same<TO, float>::value, vec_epilogue_enabled());
    default: return launch_layout<2, TO>(p, x, y, z, ws, s);
    }
}

template <int V, typename TO>
static int launch_chain_v(const tra_plan_s &p, const void *x, const void *y, void *z, const ChainEpi &ce,
                          hipStream_t s)
{
    constexpr MfmaCfg C = mfma_cfg(V);
    const GemmView &v = p.gv;
    dim3 grid((v.gm.total / C.bm) * (v.gn.total / C.bn), v.gb.total, 1);
    void (*k)(GemmView, const uint16_t *, const uint16_t *, TO *, ChainEpi);
    if (ce.join_a == J_SUB && ce.join_b == J_MUL) {
        if (p.a_kmajor) k = p.b_kmajor ? k_mfma_chain<V, true, true, TO, 1> : k_mfma_chain<V, true, false, TO, 1>;
        else k = p.b_kmajor ? k_mfma_chain<V, false, true, TO, 1> : k_mfma_chain<V, false, false, TO, 1>;
    } else {
        if (p.a_kmajor) k = p.b_kmajor ? k_mfma_chain<V, true, true, TO, 0> : k_mfma_chain<V, true, false, TO, 0>;
        else k = p.b_kmajor ? k_mfma_chain<V, false, true, TO, 0> : k_mfma_chain<V, false, false, TO, 0>;
    }
    hipLaunchKernelGGL(k, grid, dim3(C.wm * C.wn * 64), 0, s, v, (const uint16_t *)x, (const uint16_t *)y, (TO *)z,
                       ce);
    return (int)hipGetLastError();
}

// The four-wave chain: output and xb in the output's layout with aligned
// four-column vectors; YROW when ya is constant along the output's columns.
template <typename TO>
static int launch_chain4(const tra_plan_s &p, const void *x, const void *y, void *z, const ChainEpi &ce,
                         hipStream_t s)
{
    const GemmView &v = p.gv;
    dim3 grid((v.gm.total / mf4::BM) * (v.gn.total / mf4::BN), v.gb.total, 1);
    bool yrow = true;
    for (int i = 0; i < kP2Max; ++i)
        if (ce.rn.mask[i] && ce.rn.st[0][i]) yrow = false;
    void (*k)(GemmView, const uint16_t *, const uint16_t *, TO *, ChainEpi);
    const bool ch = ce.join_a == J_SUB && ce.join_b == J_MUL;
#define TRA_PICK(AK, BK)                                                                                  \
    k = !ch ? k_mfma4_chain<AK, BK, TO, 0, false>                                                         \
            : (yrow ? k_mfma4_chain<AK, BK, TO, 1, true> : k_mfma4_chain<AK, BK, TO, 1, false>)
    if (p.a_kmajor) {
        if (p.b_kmajor) TRA_PICK(true, true);
        else TRA_PICK(true, false);
    } else {
        if (p.b_kmajor) TRA_PICK(false, true);
        else TRA_PICK(false, false);
    }
#undef TRA_PICK
    hipLaunchKernelGGL(k, grid, dim3(mf4::NT), 0, s, v, (const uint16_t *)x, (const uint16_t *)y, (TO *)z, ce);
    return (int)hipGetLastError();
}

template <typename TO>
static int launch_chain_t(const tra_plan_s &p, const void *x, const void *y, void *z, const ChainEpi &ce,
                          hipStream_t s)
{
    const bool vec = p.gv.z_vec4 && (uintptr_t)z % 16 == 0 && (uintptr_t)ce.xb % 16 == 0 && chain4_enabled();
    if (p.tile == 4 && vec) return launch_mfma4k_chain(p, ce, std::is_same<TO, float>::value, x, y, z, s);
    if (p.tile == 3 && vec) return launch_chain4<TO>(p, x, y, z, ce, s);
    switch (p.tile) {
    case 0:
    case 3:
    case 4: return launch_chain_v<0, TO>(p, x, y, z, ce, s);   // the same 256 x 256 tile on eight waves
    case 1:
    case 5: return launch_chain_v<1, TO>(p, x, y, z, ce, s);   // 128 x 128 divides the narrow tile's 256 x 128
    default: return launch_chain_v<2, TO>(p, x, y, z, ce, s);
    }
}

int launch_mfma_chain(const tra_plan_s &p, const ChainEpi &ce, bool out_f32, const void *x, const void *y, void *z,
                      void *stream)
{
    if (p.gv.split != 1) return TRA_E_OP;
    hipStream_t s = (hipStream_t)stream;
    return out_f32 ? launch_chain_t<float>(p, x, y, z, ce, s) : launch_chain_t<bf16_t>(p, x, y, z, ce, s);
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
