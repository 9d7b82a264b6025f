// k_mfma4k.hip -- bf16 x bf16 -> fp32 join + sum aggregation on the four-wave
// 256 x 256 matrix-core tile with 64-deep stages (tile variant 4), for
// products whose operands are each stored contiguously along the contracted
// labels ("K-major") or along their output labels ("MN-major").
//
// Page "EinDecomp：基于爱因斯坦求和与张量关系代数的自动张量并行分解算法",
// section 2.2: the join of a key-matched pair of sub-tensors is a small
// matrix product when the join is a product and the aggregate a sum, and the
// aggregation over the contracted keys is a sum of such products.  As in the
// 32-deep tiles, one workgroup owns one output tile of one output group and
// folds every contracted partition into the same fp32 accumulators, the
// contracted keys in ascending order.
//
// Why 64-deep stages.  A K-major operand staged 32 deep is copied in 64-byte
// pieces of each row: half a cache line per row and stage, which the load
// path moves at about half the bytes per clock of whole lines.  Here each
// stage holds 64 k of every row, 128 contiguous bytes, so each copy
// instruction moves 8 whole lines.  LDS holds two such stages per operand
// (2 x 2 x 32 KiB): the matrix cores consume one while the next is copied.
//
// Per 64-deep k-tile and wave: 4 k-steps of 16 products (32x32x16), 32
// fragment reads of 16 bytes (no transposing reads: both operands are
// K-major), 16 direct global -> LDS copies.  Fragments are read two k-steps
// ahead, so each stage is free after its second k-step and the copies of
// the k-tile two ahead spread over the last two k-steps (issued in one
// k-step, 64 KiB per CU backed up the load path and stalled the waves'
// in-order issue).  Each wave owns a 128 x 128 block
// of the tile (4 x 4 products of 32 x 32, the 256 accumulators of a lane in
// the accumulator registers), its 32-row blocks interleaved with the other
// waves' as in the 32-deep four-wave tile, so the epilogues are shared.

#include "mfma_common.h"

namespace tra {

namespace mf4k {
constexpr int BM = 256, BN = 256, BK = 64, WM = 2, WN = 2, NT = WM * WN * 64, TM = 4, TN = 4;
constexpr int STAGE_ELEMS = 256 * BK;           // one operand's stage (32 KiB)
constexpr int STAGE_BYTES = STAGE_ELEMS * 2;
constexpr int COPIES = STAGE_ELEMS / 8 / NT;    // 16-byte copies per thread per operand and stage
}  // namespace mf4k

// 64-deep K-major stage, [row][64 k]: 8 granules of 16 bytes per row, granule
// c of row r stored at c ^ swz_k8(r).  A fragment read takes one granule
// column of 16 consecutive rows per 16 lanes (16x16x32) or of 32 per 32 lanes
// (32x32x16).  The permutation, a linear map of row bits 0-4, spreads those
// rows over distinct banks under each lane grouping the LDS could use for a
// 16-byte read (8 or 16 consecutive lanes, 8 + 8 lanes 32 apart, 32
// consecutive lanes).  Bits 0-4 of a fragment's row are the lane's and the
// wave's, so the permutation depends on them alone.  (The LDS bank-conflict
// counter reads the same for this map and for a simpler one of bits 0-3,
// about four cycles per read, and near zero with the fragment reads taken
// out: it counts something in how the LDS serves these 16-byte reads that
// neither permutation changes, and the kernel's cycles did not move with it.)
__device__ __forceinline__ int swz_k8(int r)
{
    return (((r >> 1) ^ (r >> 4)) & 1) | ((((r) ^ (r >> 1) ^ (r >> 3)) & 1) << 1) | (((r >> 2) & 1) << 2);
}

// Per-thread plan of one operand's copies into a stage: copy i of thread tid
// moves LDS granule p = i * NT + tid, i.e. row p / 8, slot p % 8, which holds
// granule (p % 8) ^ swz_k8(row) of that row.  A wave's 64 copies fill 1 KiB
// of consecutive LDS (8 rows) from 8 whole 128-byte row segments.  T selects
// the operand's stride slot of the contracted digits (0 = X, 1 = Y); ROWS is
// the stage's rows (256, or 128 for the narrow tile's second operand).
template <int T, int ROWS = 256>
struct DmaPlan8 {
    static constexpr int N = ROWS * mf4k::BK / 8 / mf4k::NT;
    int32_t src[N];   // source offset minus the k-tile term

    __device__ __forceinline__ void init(const Pow2Group &g_rows, const Pow2Group &gk, uint32_t r0, int32_t base,
                                         int tid)
    {
        const int32_t rbase = p2off<0>(g_rows, r0) + base;
#pragma unroll
        for (int i = 0; i < N; ++i) {
            const int p = i * mf4k::NT + tid;
            const int row = p >> 3, c = (p & 7) ^ swz_k8(p >> 3);
            src[i] = rbase + p2off<0>(g_rows, row) + p2off<T>(gk, c * 8);
        }
    }
    // copy i alone (i a compile-time constant at every call)
    __device__ __forceinline__ void issue_one(int i, const uint16_t *__restrict__ g, int32_t koff, uint16_t *stage,
                                              int wave)
    {
        dma_copy16(g, koff, (uint32_t)src[i], stage + (i * mf4k::NT + wave * 64) * 8);
    }
};

// Per-lane LDS bases of one operand's fragment reads, one per k-step of a
// stage: block i of k-step ks reads row (i * 2 + w) * 32 + l % 32, granule
// 2 ks + l / 32.  The permutation depends only on the lane and the wave (not
// on i), so block i and stage G add the constant i * 8 KiB + G * 32 KiB.
struct FragAddr8 {
    uint32_t base[4];

    __device__ __forceinline__ void init(uint32_t lds, int w, int lane)
    {
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            const int r = w * 32 + (lane & 31);
            const int c = (2 * ks + (lane >> 5)) ^ swz_k8(r);
            base[ks] = lds + (uint32_t)(r * mf4k::BK + c * 8) * 2;
        }
    }
    // issue read R (block R) of k-step KS of stage G into f
    template <int G, int KS, int R, int T>
    __device__ __forceinline__ void read_one(Frag4<true, T> &f) const
    {
        constexpr int off = G * mf4k::STAGE_BYTES + R * 64 * mf4k::BK * 2;
        f.k[R] = ds_read16_at<off>(base[KS]);
    }
    template <int G, int KS, int T>
    __device__ __forceinline__ void read(Frag4<true, T> &f) const
    {
        sfor<T>([&](auto I) { read_one<G, KS, decltype(I)::value>(f); });
    }
};

// EPI: 0 the direct epilogue, 1 the staged one, 2 the staged chained one
// (CH, YROW as for mfma4_chain_staged; ce used only then).
template <typename TO, int EPI, int CH = 0, bool YROW = false>
__device__ __forceinline__ void mfma4k_body(const GemmView &v, const uint16_t *__restrict__ x,
                                            const uint16_t *__restrict__ y, TO *__restrict__ z,
                                            float *__restrict__ ws, const ChainEpi &ce)
{
    using namespace mf4k;
    // two stages per operand (the epilogue reuses them as a staging tile)
    __shared__ __attribute__((aligned(16))) uint16_t sa[2 * STAGE_ELEMS];
    __shared__ __attribute__((aligned(16))) uint16_t sb[2 * STAGE_ELEMS];
    static_assert(2 * STAGE_BYTES >= 64 * BN * 4, "each operand's stages hold 64 staged rows");
    static_assert(BM == mf4::BM && BN == mf4::BN && WM == mf4::WM && WN == mf4::WN && TM == mf4::TM &&
                      TN == mf4::TN,
                  "the epilogues assume the 32-deep four-wave tile's wave layout");

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

    DmaPlan8<0> da;
    DmaPlan8<1> db;
    da.init(v.gm, v.gk, m0, bx, tid);
    db.init(v.gn, v.gk, n0, by, tid);
    FragAddr8 fa, fb;
    fa.init(lds_addr(sa), wm, lane);
    fb.init(lds_addr(sb), wn, lane);

    floatx16_t acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

    // Four fragment sets, one per k-step of a stage: Fq = (Aq, Bq) holds
    // k-step q.  Fragments are read two k-steps ahead, so a wave is done
    // with a stage's LDS after its k-step 1; the stage's copies for two
    // k-tiles later then spread over its k-steps 2 and 3.
    Frag4<true, TM> A0, A1, A2, A3;
    Frag4<true, TN> B0, B1, B2, B3;
    using FA = Frag4<true, TM>;
    using FB = Frag4<true, TN>;

    // One 16-deep k-step: the 16 products on (Ac, Bc), one per slot, and in
    // the slots, in this order:
    //  * RD: the reads of k-step KR of stage GR into (An, Bn), A in slots 0-3,
    //    B in slots 4-7;
    //  * CP: one operand's copies of a k-tile into stage GC (CP = 1: X's from
    //    offset ka, CP = 2: Y's from offset kb), in the even slots (spread
    //    over the k-step: bunched into 8 consecutive slots they cost 6% more
    //    cycles);
    //  * DG: one digit per slot of the operand offsets (ka, kb) of k-tile tc
    //    (scalar work that runs under the products).
    // The scheduler may not move anything across a slot boundary, so the
    // reads and copies run under the products instead of ahead of their wait.
    auto kstep = [&](auto RD, auto GR, auto KR, auto CP, auto GC, auto DG, const FA &Ac, const FB &Bc, FA &An,
                     FB &Bn, uint32_t tc, int32_t &ka, int32_t &kb) {
        constexpr bool rd = decltype(RD)::value, dg = decltype(DG)::value;
        constexpr int cp = decltype(CP)::value, gr = decltype(GR)::value, kr = decltype(KR)::value,
                      gc = decltype(GC)::value;
        const uint32_t k0 = kbeg + tc * BK;
        if constexpr (dg) {
            ka = 0;
            kb = 0;
        }
        __builtin_amdgcn_sched_barrier(0);
        sfor<TM * TN>([&](auto MC) {
            constexpr int m = decltype(MC)::value, i = m / TN, j = m % TN;
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(Ac.op(i), Bc.op(j), acc[i][j], 0, 0, 0);
            if constexpr (rd && m < TM) fa.template read_one<gr, kr, m>(An);
            else if constexpr (rd && m < TM + TN) fb.template read_one<gr, kr, m - TM>(Bn);
            if constexpr (cp == 1 && m % 2 == 0) da.issue_one(m / 2, x, ka, sa + gc * STAGE_ELEMS, wave);
            if constexpr (cp == 2 && m % 2 == 0) db.issue_one(m / 2, y, kb, sb + gc * STAGE_ELEMS, wave);
            if constexpr (dg && m < kP2Max) {
                ka += (int32_t)((k0 >> v.gk.sh[m]) & v.gk.mask[m]) * v.gk.st[0][m];
                kb += (int32_t)((k0 >> v.gk.sh[m]) & v.gk.mask[m]) * v.gk.st[1][m];
            }
            __builtin_amdgcn_sched_barrier(0);
        });
    };
    static_assert(2 * COPIES <= TM * TN && TM + TN <= TM * TN, "one copy and one read per product slot");
    using T_ = std::true_type;
    using F_ = std::false_type;
    using C0 = std::integral_constant<int, 0>;
    using CX = std::integral_constant<int, 1>;
    using CY = std::integral_constant<int, 2>;
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;
    using I3 = std::integral_constant<int, 3>;

    // k-tile t in stage G.  On entry k-steps 0 and 1 are read (F0, F1; the
    // reads may be in flight).  k-steps 0 and 1 read k-steps 2 and 3; then
    // the wave has all its fragments of stage G (waited for), and the copies
    // of k-tile t + 1 into the other stage have landed: a barrier publishes
    // that stage and frees stage G.  k-steps 2 and 3 read k-steps 0 and 1 of
    // the other stage and copy k-tile t + 2 into stage G, X's half in k-step
    // 2 and Y's in k-step 3.  (Near the end that copy re-reads the last
    // k-tile: every copy stays in bounds, and the count of copies per step
    // stays fixed.)
    auto step = [&](auto GC, uint32_t t) {
        using GO = std::integral_constant<int, 1 - decltype(GC)::value>;
        int32_t ka = 0, kb = 0;
        lds_wait<TM + TN>();   // F0 landed (F1 may be in flight)
        A0.ready();
        B0.ready();
        kstep(T_{}, GC, I2{}, C0{}, GC, T_{}, A0, B0, A2, B2, min(t + 2, nk - 1), ka, kb);
        lds_wait<TM + TN>();   // F1 landed (F2 may be in flight)
        A1.ready();
        B1.ready();
        kstep(T_{}, GC, I3{}, C0{}, GC, F_{}, A1, B1, A3, B3, 0u, ka, kb);
        lds_wait<0>();   // this wave's reads of stage G are done
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        A2.ready();
        B2.ready();
        A3.ready();
        B3.ready();
        kstep(T_{}, GO{}, I0{}, CX{}, GC, F_{}, A2, B2, A0, B0, 0u, ka, kb);
        kstep(T_{}, GO{}, I1{}, CY{}, GC, F_{}, A3, B3, A1, B1, 0u, ka, kb);
    };
    // The last k-tile when the count is odd (stage 0): no copies and no reads
    // past it.
    auto tail_step = [&](uint32_t) {
        int32_t ka = 0, kb = 0;
        lds_wait<TM + TN>();
        A0.ready();
        B0.ready();
        kstep(T_{}, I0{}, I2{}, C0{}, I0{}, F_{}, A0, B0, A2, B2, 0u, ka, kb);
        lds_wait<TM + TN>();
        A1.ready();
        B1.ready();
        kstep(T_{}, I0{}, I3{}, C0{}, I0{}, F_{}, A1, B1, A3, B3, 0u, ka, kb);
        lds_wait<TM + TN>();
        A2.ready();
        B2.ready();
        kstep(F_{}, I0{}, I0{}, C0{}, I0{}, F_{}, A2, B2, A0, B0, 0u, ka, kb);
        lds_wait<0>();
        A3.ready();
        B3.ready();
        kstep(F_{}, I0{}, I0{}, C0{}, I0{}, F_{}, A3, B3, A1, B1, 0u, ka, kb);
    };

    // prologue: k-tiles 0 and 1 in flight, k-steps 0 and 1 of the first read
    {
        const uint32_t k1 = min(1u, nk - 1);
        const int32_t a0 = p2off<0>(v.gk, kbeg), b0 = p2off<1>(v.gk, kbeg);
        const int32_t a1 = p2off<0>(v.gk, kbeg + k1 * BK), b1 = p2off<1>(v.gk, kbeg + k1 * BK);
        sfor<COPIES>([&](auto I) { da.issue_one(decltype(I)::value, x, a0, sa, wave); });
        sfor<COPIES>([&](auto I) { db.issue_one(decltype(I)::value, y, b0, sb, wave); });
        sfor<COPIES>([&](auto I) { da.issue_one(decltype(I)::value, x, a1, sa + STAGE_ELEMS, wave); });
        sfor<COPIES>([&](auto I) { db.issue_one(decltype(I)::value, y, b1, sb + STAGE_ELEMS, wave); });
    }
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * COPIES));
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    fa.template read<0, 0>(A0);
    fb.template read<0, 0>(B0);
    fa.template read<0, 1>(A1);
    fb.template read<0, 1>(B1);
    lds_wait<0>();
    A0.ready();
    B0.ready();
    A1.ready();
    B1.ready();

    // The loop body runs two k-tiles (stages 0 and 1); every fragment read it
    // issues is waited for inside it, except those of the next body's first
    // two k-steps, which are waited for (and handed on through lds_ready)
    // before the back-edge, so that no read is in flight at a branch or merge.
    uint32_t t = 0;
    for (; t + 2 <= nk; t += 2) {
        step(I0{}, t);
        step(I1{}, t + 1);
        lds_wait<0>();
        A0.ready();
        B0.ready();
        A1.ready();
        B1.ready();
    }
    if (t < nk) tail_step(t);
    // nothing may stay in flight past the k-loop
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    lds_wait<0>();

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

// ---------------------------------------------------------------------------
// The same tile on 16x16x32 products.  Under sustained load the chip is held
// to its power budget, and a 16x16x32 product moves half the accumulator
// bytes per flop through the register file of a 32x32x16 one: a loop of
// products with random operands sustains about 7% more of them at the same
// budget.  Each wave's 128 x 128 block is 8 x 8 blocks of 16 x 16 (row blocks
// (2i + wm)*16, column blocks (2j + wn)*16), its 256 accumulators in the
// accumulator registers.  A k-step is 32 deep (two per stage): 64 products,
// 16 fragment reads of 16 bytes (lane l: row or column l % 16 of its block,
// k 8(l/16) .. +7).  Fragments are read one k-step ahead, so a wave is done
// with a stage after its first k-step; the stage's copies for two k-tiles
// later spread over its second.
//
// The products are issued by inline asm with the accumulators bound to the
// accumulator registers: with the compiler's own product the 64 four-element
// accumulators were moved around the register file in every iteration.
// Being asm, their register hazards are handled here: the accumulators are
// zeroed and then separated from the first product by wait states, each
// accumulator is next read by a product 64 products later, fragments come
// straight from LDS reads (waited for) with no vector-ALU write between, and
// after the last product wait states precede every read of an accumulator.
__device__ __forceinline__ void mfma16x16x32(floatx4_t &acc, const u32x4_t &a, const u32x4_t &b)
{
    asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}

// Binds every accumulator to the accumulator registers at one point of the
// instruction stream (an asm that reads and writes each of them).
template <int NJ>
__device__ __forceinline__ void acc16_bind(floatx4_t (&acc)[2 * mf4::TM][NJ])
{
#pragma unroll
    for (int i = 0; i < 2 * mf4::TM; ++i) {
        if constexpr (NJ == 8)
            asm volatile(""
                         : "+a"(acc[i][0]), "+a"(acc[i][1]), "+a"(acc[i][2]), "+a"(acc[i][3]), "+a"(acc[i][4]),
                           "+a"(acc[i][5]), "+a"(acc[i][6]), "+a"(acc[i][7]));
        else
            asm volatile("" : "+a"(acc[i][0]), "+a"(acc[i][1]), "+a"(acc[i][2]), "+a"(acc[i][3]));
    }
}
// Wait states between every write of the accumulators before it and every
// read after it (the two binds fix the order: volatile asm keeps its order).
template <int NJ>
__device__ __forceinline__ void acc16_fence(floatx4_t (&acc)[2 * mf4::TM][NJ])
{
    static_assert(NJ == 8 || NJ == 4, "eight or four 16-column blocks per wave");
    acc16_bind(acc);
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7");
    acc16_bind(acc);
}

// One operand's fragments of one 32-deep k-step: N blocks of 16 rows.
template <int N = 8>
struct Frag16 {
    u32x4_t k[N];
    __device__ __forceinline__ void ready()
    {
#pragma unroll
        for (int i = 0; i < N; ++i) lds_ready(k[i]);
    }
};

// Per-lane LDS bases of one operand's 16-row fragment reads, one per k-step
// of a stage: block i of k-step ks reads row (2i + w)*16 + l % 16, granule
// 4 ks + l / 16 (permuted by row bits 0-4: the lane's and the wave's); block
// i and stage G add i * 4 KiB + G * 32 KiB.
template <int SB = mf4k::STAGE_BYTES>   // bytes of one stage of the operand
struct FragAddr16 {
    uint32_t base[2];
    __device__ __forceinline__ void init(uint32_t lds, int w, int lane)
    {
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            const int r = w * 16 + (lane & 15);
            const int c = (4 * ks + (lane >> 4)) ^ swz_k8(r);
            base[ks] = lds + (uint32_t)(r * mf4k::BK + c * 8) * 2;
        }
    }
    template <int G, int KS, int R, typename F>
    __device__ __forceinline__ void read_one(F &f) const
    {
        constexpr int off = G * SB + R * 32 * mf4k::BK * 2;
        f.k[R] = ds_read16_at<off>(base[KS]);
    }
    // the same from the stage at byte offset soff (a runtime ring slot)
    template <int KS, int R, typename F>
    __device__ __forceinline__ void read_rt(F &f, uint32_t soff) const
    {
        constexpr int off = R * 32 * mf4k::BK * 2;
        f.k[R] = ds_read16_at<off>(base[KS] + soff);
    }
};

// 64-deep MN-major stage, [64 k][256 columns]: 32 granules of 16 bytes per
// k-row, granule c of k-row k stored at c ^ swz_n8(k).  A transposing
// fragment read of one 16-lane group covers 4 consecutive k-rows x 32 bytes,
// and the next group the same columns 8 k-rows further: k % 4 moves the 4
// rows' 32-byte pieces to distinct offsets within 128 bytes, and k-row bit 3
// moves the odd group's to the other 128 bytes, so each 32-lane half of a
// read covers the 64 banks once.  (With k % 4 alone the two groups collide:
// the bank-conflict counter of the blocked GEMM halved when bit 3 was added.)
// It depends on the lane only.
__device__ __forceinline__ int swz_n8(int k) { return ((k & 3) << 1) | (((k >> 3) & 1) << 3); }

// Per-thread copies of an MN-major operand into a stage: copy i of thread
// tid moves LDS granule p = i * NT + tid, k-row p / 32, slot p % 32, which
// holds granule (p % 32) ^ swz_n8(k) of that k-row (a wave's 64 copies: two
// whole 512-byte k-rows).
template <int T, int COLS = 256>   // COLS: the stage's columns (256, or 128)
struct DmaPlanN8 {
    static constexpr int GPR = COLS / 8;   // granules per k-row
    static constexpr int N = COLS * mf4k::BK / 8 / mf4k::NT;
    int32_t src[N];

    __device__ __forceinline__ void init(const Pow2Group &g_cols, const Pow2Group &gk, uint32_t c0, int32_t base,
                                         int tid)
    {
        const int32_t cbase = p2off<0>(g_cols, c0) + base;
#pragma unroll
        for (int i = 0; i < N; ++i) {
            const int p = i * mf4k::NT + tid;
            const int k = p / GPR, gl = (p % GPR) ^ swz_n8(p / GPR);
            src[i] = cbase + p2off<0>(g_cols, gl * 8) + p2off<T>(gk, k);
        }
    }
    __device__ __forceinline__ void issue_one(int i, const uint16_t *__restrict__ g, int32_t koff, uint16_t *stage,
                                              int wave)
    {
        dma_copy16(g, koff, (uint32_t)src[i], stage + (i * mf4k::NT + wave * 64) * 8);
    }
};

// One operand's fragments of one 32-deep k-step for an MN-major operand:
// per 16-column block two transposing 8-byte reads (k 8(l/16) .. +3 and
// +4 .. +7 of column l % 16).
template <int N = 8>
struct Frag16N {
    u32x2_t t[N][2];
    __device__ __forceinline__ void ready()
    {
#pragma unroll
        for (int j = 0; j < N; ++j) {
            lds_ready(t[j][0]);
            lds_ready(t[j][1]);
        }
    }
    __device__ __forceinline__ u32x4_t op(int j) const
    {
        return u32x4_t{t[j][0][0], t[j][0][1], t[j][1][0], t[j][1][1]};
    }
};

// Transposing reads of an MN-major stage (gfx950's ds_read_b64_tr_b16: in each
// 16-lane group, output lane i element e is element i % 4 of source lane
// 4e + i / 4).  Lane l = 16 g + s reads 4 columns 4(s % 4) .. +3 of its
// block at k-row 8g + 4r + s / 4 (read r), so output lane s holds column s,
// k 8g + 4r .. +3.  Block j covers columns (2j + wn)*16 .. +15, granules
// 4j + 2wn + (s % 4)/2; the permutation touches granule bits 1-3 (wn and j
// bits 0-1), so there is one base per j % 4, and j / 4, the read, the k-step
// and the stage add constants.
template <int COLS = 256>   // the stage's columns (256, or 128: then j < 4, one base each)
struct FragAddrN16 {
    uint32_t base[4];
    __device__ __forceinline__ void init(uint32_t lds, int w, int lane)
    {
        const int g = lane >> 4, sl = lane & 15;
        const int k = 8 * g + (sl >> 2);
#pragma unroll
        for (int jl = 0; jl < 4; ++jl) {
            const int gran = (4 * jl + 2 * w + ((sl & 3) >> 1)) ^ swz_n8(k);
            base[jl] = lds + (uint32_t)(k * COLS + gran * 8 + 4 * (sl & 1)) * 2;
        }
    }
    // read R of k-step KS of stage G: block R / 2, half R % 2
    template <int G, int KS, int R, typename F>
    __device__ __forceinline__ void read_one(F &f) const
    {
        constexpr int j = R / 2, h = R % 2, jl = j % 4, jh = j / 4;
        constexpr int off = G * COLS * mf4k::BK * 2 + (KS * 32 + 4 * h) * COLS * 2 + jh * 16 * 16;
        f.t[j][h] = ds_read8_tr_at<off>(base[jl]);
    }
    template <int KS, int R, typename F>
    __device__ __forceinline__ void read_rt(F &f, uint32_t soff) const
    {
        constexpr int j = R / 2, h = R % 2, jl = j % 4, jh = j / 4;
        constexpr int off = (KS * 32 + 4 * h) * COLS * 2 + jh * 16 * 16;
        f.t[j][h] = ds_read8_tr_at<off>(base[jl] + soff);
    }
};

// One piece of digit q of operand T's k-tile offset: PH 0 extracts the
// digit of k0, PH 1 adds its term to koff.  The empty asm statements pin each
// piece to its product slot: without them the compiler gathered all digits
// of a k-step into one run of ~50 scalar instructions between two products,
// which the wave issues one at a time while the matrix core idles.
template <int PH, int T>
__device__ __forceinline__ void digit_piece(uint32_t k0, int q, const Pow2Group &g, uint32_t &dig, int32_t &koff)
{
    if constexpr (PH == 0) {
        uint32_t kk = k0;
        asm volatile("" : "+s"(kk));
        dig = (kk >> g.sh[q]) & g.mask[q];
        asm volatile("" : "+s"(dig));
    } else {
        uint32_t dd = dig;
        asm volatile("" : "+s"(dd));
        koff += (int32_t)dd * g.st[T][q];
        asm volatile("" : "+s"(koff));
    }
}

// AKM / BKM: the first / second operand K-major (else MN-major: staged
// [k][row or column] and read through the transposing LDS read).
template <bool AKM, bool BKM, typename TO, int EPI, int CH = 0, bool YROW = false, int BNW = 256>
__device__ __forceinline__ void mfma4k16_body(const GemmView &v, const uint16_t *__restrict__ x,
                                              const uint16_t *__restrict__ y, TO *__restrict__ z,
                                              float *__restrict__ ws, const ChainEpi &ce)
{
    using namespace mf4k;
    // BNW: the tile's columns, 256 or 128 (each wave then 128 x 64)
    static_assert(BNW == 256 || BNW == 128, "256 x 256 or 256 x 128 tiles");
    constexpr int SBE = BNW * BK, SBB = SBE * 2;   // one stage of the second operand
    __shared__ __attribute__((aligned(16))) uint16_t sa[3 * STAGE_ELEMS];   // 96 + 64 (or 32) KiB
    __shared__ __attribute__((aligned(16))) uint16_t sb[2 * SBE];
    constexpr int NI = 2 * TM, NJ = BNW / 32;   // 16-row and 16-column blocks of a wave
    constexpr int NP = NI * NJ, HALF = NP / 2;   // products per k-step, and half of them

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / WN, wn = wave % WN;
    const uint32_t tiles_n = v.gn.total / BNW;
    const uint32_t nb = (v.gm.total / BM) * tiles_n;
    uint32_t tm, tn, bidx;
    mfma_tile_of(nb, tiles_n, v.gb.total, bidx, tm, tn);
    const uint32_t m0 = tm * BM, n0 = tn * BNW;
    const int32_t bx = p2off<0>(v.gb, bidx), by = p2off<1>(v.gb, bidx), bz = p2off<2>(v.gb, bidx);
    const uint32_t kbeg = blockIdx.z * (uint32_t)v.k_per_split;
    const uint32_t nk = (uint32_t)v.k_per_split / BK;

    typename std::conditional<AKM, DmaPlan8<0>, DmaPlanN8<0>>::type da;
    using DPB = typename std::conditional<BKM, DmaPlan8<1, BNW>, DmaPlanN8<1, BNW>>::type;
    DPB db;
    da.init(v.gm, v.gk, m0, bx, tid);
    db.init(v.gn, v.gk, n0, by, tid);
    typename std::conditional<AKM, FragAddr16<>, FragAddrN16<>>::type fa;
    typename std::conditional<BKM, FragAddr16<SBB>, FragAddrN16<BNW>>::type fb;
    fa.init(lds_addr(sa), wm, lane);
    fb.init(lds_addr(sb), wn, lane);
    using FA = typename std::conditional<AKM, Frag16<>, Frag16N<>>::type;
    using FB = typename std::conditional<BKM, Frag16<NJ>, Frag16N<NJ>>::type;
    constexpr int NAR = AKM ? 8 : 16, NBR = BKM ? NJ : 2 * NJ;   // fragment reads per operand and k-step
    constexpr int CB = DPB::N;                                  // the second operand's copies per k-tile

    floatx4_t acc[NI][NJ];
#pragma unroll
    for (int i = 0; i < NI; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[i][j][e] = 0.f;
    acc16_fence(acc);   // the zeroing lands before the first product reads it

    FA A0, A1;   // k-steps 0 and 1 of a stage
    FB B0, B1;

    // One 32-deep k-step: the 64 products on (Ac, Bc), one per slot; the
    // reads of k-step KR into An (X's stage at byte offset a_rd) in slots 4r
    // (K-major) or 2r (MN-major, two per block) of the first 32, into Bn (Y's
    // stage GBR) likewise in the last 32; in slots 8r + 6 copy r of a k-tile,
    // X's into the stage at element offset a_wr (XC, from ka) or Y's into
    // stage GBW (YC, from kb); in odd slots 4q + 1 and 4q + 3 the two pieces
    // of digit q of ka (DA, of k-tile ta) or kb (DB, of k-tile tb).  (Reads
    // gathered into the first slots instead measured 6% slower: one wave per
    // SIMD issues four instructions per 16-cycle product.)
    auto kstep = [&](auto RD, auto GBR, auto KR, auto XC, auto YC, auto GBW, auto DA, auto DB, const FA &Ac,
                     const FB &Bc, FA &An, FB &Bn, uint32_t a_rd, uint32_t a_wr, uint32_t ta, uint32_t tb,
                     int32_t &ka, int32_t &kb) {
        constexpr bool rd = decltype(RD)::value, xc = decltype(XC)::value, yc = decltype(YC)::value;
        constexpr bool dga = decltype(DA)::value, dgb = decltype(DB)::value;
        constexpr int gbr = decltype(GBR)::value, kr = decltype(KR)::value, gbw = decltype(GBW)::value;
        const uint32_t ka0 = kbeg + ta * BK, kb0 = kbeg + tb * BK;
        uint32_t dig = 0;
        if constexpr (dga) ka = 0;
        if constexpr (dgb) kb = 0;
        __builtin_amdgcn_sched_barrier(0);
        sfor<NP>([&](auto MC) {
            constexpr int m = decltype(MC)::value, i = m / NJ, j = m % NJ;
            if constexpr (AKM && BKM) mfma16x16x32(acc[i][j], Ac.k[i], Bc.k[j]);
            else if constexpr (AKM) mfma16x16x32(acc[i][j], Ac.k[i], Bc.op(j));
            else if constexpr (BKM) mfma16x16x32(acc[i][j], Ac.op(i), Bc.k[j]);
            else mfma16x16x32(acc[i][j], Ac.op(i), Bc.op(j));
            constexpr int AS = HALF / NAR, BS = HALF / NBR;   // slot spacing of the reads
            constexpr int XS = NP / COPIES, YS = NP / CB;     // and of the copies
            if constexpr (rd && m < HALF && m % AS == 0) fa.template read_rt<kr, m / AS>(An, a_rd);
            if constexpr (rd && m >= HALF && (m - HALF) % BS == 0)
                fb.template read_one<gbr, kr, (m - HALF) / BS>(Bn);
            if constexpr (xc && m % XS == XS - 2) da.issue_one(m / XS, x, ka, sa + a_wr, wave);
            if constexpr (yc && m % YS == YS - 2) db.issue_one(m / YS, y, kb, sb + gbw * SBE, wave);
            constexpr int u = (m - 1) / 2;
            if constexpr (dga && m % 2 == 1 && u / 2 < kP2Max) digit_piece<u % 2, 0>(ka0, u / 2, v.gk, dig, ka);
            if constexpr (dgb && m % 2 == 1 && u / 2 < kP2Max) digit_piece<u % 2, 1>(kb0, u / 2, v.gk, dig, kb);
            __builtin_amdgcn_sched_barrier(0);
        });
    };
    static_assert(NP % COPIES == 0 && NP % CB == 0 && 4 * kP2Max <= NP && HALF % NAR == 0 && HALF % NBR == 0,
                  "copies and reads spread evenly over a k-step, a digit per four of its slots");
    using T_ = std::true_type;
    using F_ = std::false_type;
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;

    // X's stages form a ring of three (k-tile t in slot t % 3), Y's a ring of
    // two (slot t % 2).  k-tile t: on entry F0 = (A0, B0) holds its k-step 0
    // (reads may be in flight).  k-step 0 reads k-step 1, copies X's k-tile
    // t + 2 into X slot (t + 2) % 3 (that of k-tile t - 1, free since the
    // barrier of k-tile t - 1) and takes the digits of Y's k-tile t + 2.  Then
    // the wave has read all its fragments of k-tile t and the copies of k-tile
    // t + 1 have landed (those of X's k-tile t + 2, issued last, may still be
    // in flight): a barrier publishes k-tile t + 1 and frees Y's slot t % 2.
    // k-step 1 reads k-step 0 of k-tile t + 1, copies Y's k-tile t + 2 into
    // slot t % 2 and takes the digits of X's k-tile t + 3.  So every copy has
    // a whole k-tile of products to land, and the copies of a k-tile spread
    // over both its k-steps.  Near the end the last k-tile is copied again (in
    // bounds, the count of copies per k-step fixed).  ia = t % 3.
    auto step = [&](auto GB, uint32_t t, uint32_t ia, int32_t &ka, int32_t &kb) {
        using GO = std::integral_constant<int, 1 - decltype(GB)::value>;
        const uint32_t i1 = ia == 2 ? 0 : ia + 1, i2 = i1 == 2 ? 0 : i1 + 1;
        lds_wait<0>();
        A0.ready();
        B0.ready();
        kstep(T_{}, GB, I1{}, T_{}, F_{}, GB, F_{}, T_{}, A0, B0, A1, B1, ia * STAGE_BYTES, i2 * STAGE_ELEMS, 0u,
              min(t + 2, nk - 1), ka, kb);
        lds_wait<0>();   // this wave's reads of k-tile t are done
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(COPIES));
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        A1.ready();
        B1.ready();
        kstep(T_{}, GO{}, I0{}, F_{}, T_{}, GB, T_{}, F_{}, A1, B1, A0, B0, i1 * STAGE_BYTES, 0u, min(t + 3, nk - 1),
              0u, ka, kb);
    };
    auto tail_step = [&](uint32_t ia, int32_t &ka, int32_t &kb) {
        lds_wait<0>();
        A0.ready();
        B0.ready();
        kstep(T_{}, I0{}, I1{}, F_{}, F_{}, I0{}, F_{}, F_{}, A0, B0, A1, B1, ia * STAGE_BYTES, 0u, 0u, 0u, ka, kb);
        lds_wait<0>();
        A1.ready();
        B1.ready();
        kstep(F_{}, I0{}, I0{}, F_{}, F_{}, I0{}, F_{}, F_{}, A1, B1, A0, B0, 0u, 0u, 0u, 0u, ka, kb);
    };

    // prologue: k-tiles 0 and 1 in flight into slots 0 and 1 of each ring,
    // X's offset of k-tile 2, k-step 0 of the first read
    int32_t ka, kb = 0;
    {
        const uint32_t k1 = min(1u, nk - 1);
        const int32_t a0 = p2off<0>(v.gk, kbeg), b0 = p2off<1>(v.gk, kbeg);
        const int32_t a1 = p2off<0>(v.gk, kbeg + k1 * BK), b1 = p2off<1>(v.gk, kbeg + k1 * BK);
        sfor<COPIES>([&](auto I) { da.issue_one(decltype(I)::value, x, a0, sa, wave); });
        sfor<CB>([&](auto I) { db.issue_one(decltype(I)::value, y, b0, sb, wave); });
        sfor<COPIES>([&](auto I) { da.issue_one(decltype(I)::value, x, a1, sa + STAGE_ELEMS, wave); });
        sfor<CB>([&](auto I) { db.issue_one(decltype(I)::value, y, b1, sb + SBE, wave); });
        ka = p2off<0>(v.gk, kbeg + min(2u, nk - 1) * BK);
    }
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(COPIES + CB));   // k-tile 0 has landed
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    sfor<NAR>([&](auto I) { fa.template read_rt<0, decltype(I)::value>(A0, 0u); });
    sfor<NBR>([&](auto I) { fb.template read_one<0, 0, decltype(I)::value>(B0); });
    lds_wait<0>();
    A0.ready();
    B0.ready();

    // two k-tiles per loop body; no read in flight at a branch or merge
    uint32_t t = 0, ia = 0;
    for (; t + 2 <= nk; t += 2) {
        step(I0{}, t, ia, ka, kb);
        ia = ia == 2 ? 0 : ia + 1;
        step(I1{}, t + 1, ia, ka, kb);
        ia = ia == 2 ? 0 : ia + 1;
        lds_wait<0>();
        A0.ready();
        B0.ready();
    }
    if (t < nk) tail_step(ia, ka, kb);
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    lds_wait<0>();
    acc16_fence(acc);   // every product has written its accumulator before any read

    const bool split = v.split > 1;
    float *wsp = split ? ws + (int64_t)blockIdx.z * v.z_elems : nullptr;
    if constexpr (BNW != 256) {
        // the narrow tile stores straight from the accumulators (its outputs
        // are small next to the operands it streams)
        static_assert(EPI == 0, "the 256 x 128 tile has the direct epilogue only");
        mfma4_store_direct16<TO, NJ>(v, z, wsp, split, acc, m0, n0, bz, wave);
        return;
    } else if constexpr (EPI == 2) {
        lds_barrier();
        mfma4_chain_staged<TO, CH, YROW>(v, z, ce, acc, lds_addr(sa), lds_addr(sb), m0, n0, bidx, bz, wave, lane);
        return;
    } else if constexpr (EPI == 1) {
        lds_barrier();
        if (split) mfma4_store_staged<float, false>(v, wsp, acc, lds_addr(sa), lds_addr(sb), m0, n0, bz, wave, lane);
        else mfma4_store_staged<TO, true>(v, z, acc, lds_addr(sa), lds_addr(sb), m0, n0, bz, wave, lane);
        return;
    } else {
        mfma4_store_direct16<TO, NJ>(v, z, wsp, split, acc, m0, n0, bz, wave);
    }
}

// The 64-deep tile's products: 16x16x32 (1) or 32x32x16 (0).
#ifndef TRA_K4K_M16
#define TRA_K4K_M16 1
#endif
// (The 32x32x16 body takes two K-major operands only.)
template <bool AKM, bool BKM, typename TO, int EPI, int CH = 0, bool YROW = false, int BNW = 256>
__device__ __forceinline__ void mfma4k_run(const GemmView &v, const uint16_t *__restrict__ x,
                                           const uint16_t *__restrict__ y, TO *__restrict__ z,
                                           float *__restrict__ ws, const ChainEpi &ce)
{
    if constexpr (TRA_K4K_M16 || !AKM || !BKM || BNW != 256)
        mfma4k16_body<AKM, BKM, TO, EPI, CH, YROW, BNW>(v, x, y, z, ws, ce);
    else mfma4k_body<TO, EPI, CH, YROW>(v, x, y, z, ws, ce);
}

// VEC: the staged epilogue (the output's four consecutive columns form one
// aligned vector, and z / the workspace are 16-byte aligned).  BNW: the
// tile's columns (256; 128 for the narrow tile, variant 5).
template <bool AKM, bool BKM, typename TO, bool VEC, int BNW = 256>
__global__ __launch_bounds__(mf4k::NT) void k_mfma4k_bf16(GemmView v, const uint16_t *__restrict__ x,
                                                          const uint16_t *__restrict__ y, TO *__restrict__ z,
                                                          float *__restrict__ ws)
{
    mfma4k_run<AKM, BKM, TO, VEC ? 1 : 0, 0, false, BNW>(v, x, y, z, ws, ChainEpi{});
}

// The product with a chain of two elementwise steps in its staged epilogue
template <bool AKM, bool BKM, typename TO, int CH, bool YROW>
__global__ __launch_bounds__(mf4k::NT) void k_mfma4k_chain(GemmView v, const uint16_t *__restrict__ x,
                                                           const uint16_t *__restrict__ y, TO *__restrict__ z,
                                                           ChainEpi ce)
{
    mfma4k_run<AKM, BKM, TO, 2, CH, YROW>(v, x, y, z, nullptr, ce);
}

// ---------------------------------------------------------------------------
// Short contractions (one or two 64-deep k-tiles, fp32 output), as a
// persistent loop over output tiles.  With so little k the tile's fp32 write
// (256 KiB) is most of its time: the attention scores S = Q·Kᵀ over a head
// dimension of 128 write 2 GiB.  A workgroup that ends after its stores holds
// its CU until they drain, and the next workgroup's copies and products wait
// behind them.  Here each workgroup keeps the CU and walks tiles vid,
// vid + gridDim.x, ... (the same XCD, the same order as a plain launch): once
// a tile's products are done it issues the next tile's copies (both k-tiles
// of both operands into slots 0-1 of the rings), then stages and stores its
// output in eight pieces of 32 rows through the free third slot of the first
// operand's ring.  Vector memory operations complete in issue order, so the
// next tile waits only for its copies (vmcnt 63: the copies and the first of
// the 64 stores that follow them), and its products run while the previous
// tile's stores drain.
//
// Staging piece p holds rows 32p .. +31 of the tile (accumulator block row p
// of every wave): row r at r * 1 KiB, column c at c ^ (((r >> 2) & 3) << 4),
// so the four 4-row groups of a wave's write land on distinct banks and each
// row stays 16-byte granular for the row reads.
template <bool AKM, bool BKM, int NK>
__global__ __launch_bounds__(mf4k::NT) void k_mfma4k_short(GemmView v, const uint16_t *__restrict__ x,
                                                           const uint16_t *__restrict__ y, float *__restrict__ z)
{
    using namespace mf4k;
    __shared__ __attribute__((aligned(16))) uint16_t sa[3 * STAGE_ELEMS];
    __shared__ __attribute__((aligned(16))) uint16_t sb[2 * STAGE_ELEMS];
    constexpr int NI = 2 * TM, NJ = 2 * TN;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / WN, wn = wave % WN;
    const uint32_t tiles_n = v.gn.total / BN;
    const uint32_t nb = (v.gm.total / BM) * tiles_n;
    const uint32_t n_lin = nb * v.gb.total;
    static_assert(NK == 1 || NK == 2, "one or two k-tiles (v.k_per_split == NK * BK)");
    uint32_t vid = blockIdx.x;
    if (vid >= n_lin) return;

    typename std::conditional<AKM, DmaPlan8<0>, DmaPlanN8<0>>::type da;
    typename std::conditional<BKM, DmaPlan8<1>, DmaPlanN8<1>>::type db;
    typename std::conditional<AKM, FragAddr16<>, FragAddrN16<>>::type fa;
    typename std::conditional<BKM, FragAddr16<>, FragAddrN16<>>::type fb;
    fa.init(lds_addr(sa), wm, lane);
    fb.init(lds_addr(sb), wn, lane);
    using FA = typename std::conditional<AKM, Frag16<>, Frag16N<>>::type;
    using FB = typename std::conditional<BKM, Frag16<>, Frag16N<>>::type;
    constexpr int NAR = AKM ? 8 : 16, NBR = BKM ? 8 : 16;
    constexpr uint32_t k1 = NK - 1;   // k-tile 0 again when there is one
    const int32_t a1 = p2off<0>(v.gk, k1 * BK), b1 = p2off<1>(v.gk, k1 * BK);

    // The copies' lane offsets within a tile are the same for every tile
    // (a tile's first row and column are multiples of 256, so its offset adds
    // to theirs digit by digit): the tile's part goes into the copies' scalar
    // offset.  Likewise the output's row and column offsets.
    da.init(v.gm, v.gk, 0, 0, tid);
    db.init(v.gn, v.gk, 0, 0, tid);
    int32_t ta, tb, tz;   // the tile's offsets in X, Y and Z
    auto setup = [&](uint32_t l, int32_t &oa, int32_t &ob, int32_t &oz) {
        uint32_t tm, tn, bidx;
        mfma_tile_at(l % nb, l / nb, nb, tiles_n, v.gb.total, bidx, tm, tn);
        const uint32_t m0 = tm * BM, n0 = tn * BN;
        oa = p2off<0>(v.gm, m0) + p2off<0>(v.gb, bidx);
        ob = p2off<0>(v.gn, n0) + p2off<1>(v.gb, bidx);
        oz = p2off<1>(v.gm, m0) + p2off<1>(v.gn, n0) + p2off<2>(v.gb, bidx);
    };
    // k-tile 1's copies (k-tile 0's go out in the product slots)
    auto issue_k1 = [&](int32_t oa, int32_t ob) {
        sfor<COPIES>([&](auto I) { da.issue_one(decltype(I)::value, x, oa + a1, sa + STAGE_ELEMS, wave); });
        sfor<COPIES>([&](auto I) { db.issue_one(decltype(I)::value, y, ob + b1, sb + STAGE_ELEMS, wave); });
    };

    // staging: per-lane write bases for even and odd 16-column blocks j
    // (their columns' bit 5 is j's bit 0, XORed with the row group's bit 1),
    // and row-read bases for the wave's rows 8 wave .. +7 of a piece
    const uint32_t st = lds_addr(sa) + 2 * STAGE_BYTES;
    const int g = lane >> 4, s16 = lane & 15;
    const uint32_t wrow = st + (uint32_t)((16 * wm + 4 * g) * 256) * 4;
    const uint32_t wbe = wrow + (uint32_t)((((wn ^ (g & 1)) * 16) + ((g >> 1) * 32) + s16) * 4);
    const uint32_t wbo = wrow + (uint32_t)((((wn ^ (g & 1)) * 16) + ((1 - (g >> 1)) * 32) + s16) * 4);
    uint32_t rbase[2];
#pragma unroll
    for (int h = 0; h < 2; ++h)
        rbase[h] = st + (uint32_t)(8 * wave * 256 + ((4 * lane) ^ (((2 * wave + h) & 3) << 4))) * 4;
    const int32_t band_row = p2off<1>(v.gm, lane & 31);         // row r < 32 of a piece
    const int32_t piece_row = p2off<1>(v.gm, 32 * (lane & 7));   // first row of piece p < 8
    const int32_t on = p2off<1>(v.gn, 4 * lane);                 // the lane's four columns

    Acc16 acc;
    FA A0, A1;
    FB B0, B1;
    // one 32-deep k-step: 64 products, the next k-step's reads in the slots
    // of the main kernel (A's in the first 32, B's in the last 32)
    // CP: the next tile's k-tile 0 copies into slot 0 in this k-step, X's
    // (bit 0, slots 8r + 6) and Y's (bit 1, slots 8r + 2), from offsets oa, ob
    auto kstep = [&](auto RD, auto GBR, auto KR, auto CP, const FA &Ac, const FB &Bc, FA &An, FB &Bn,
                     uint32_t a_rd, int32_t oa, int32_t ob) {
        constexpr bool rd = decltype(RD)::value;
        constexpr int gbr = decltype(GBR)::value, kr = decltype(KR)::value, cp = decltype(CP)::value;
        __builtin_amdgcn_sched_barrier(0);
        sfor<NI * NJ>([&](auto MC) {
            constexpr int m = decltype(MC)::value, i = m / NJ, j = m % NJ;
            if constexpr (AKM && BKM) mfma16x16x32(acc[i][j], Ac.k[i], Bc.k[j]);
            else if constexpr (AKM) mfma16x16x32(acc[i][j], Ac.k[i], Bc.op(j));
            else if constexpr (BKM) mfma16x16x32(acc[i][j], Ac.op(i), Bc.k[j]);
            else mfma16x16x32(acc[i][j], Ac.op(i), Bc.op(j));
            constexpr int AS = AKM ? 4 : 2, BS = BKM ? 4 : 2;
            if constexpr (rd && m < 32 && m % AS == 0 && m / AS < NAR) fa.template read_rt<kr, m / AS>(An, a_rd);
            if constexpr (rd && m >= 32 && (m - 32) % BS == 0 && (m - 32) / BS < NBR)
                fb.template read_one<gbr, kr, (m - 32) / BS>(Bn);
            if constexpr ((cp & 1) && m % 8 == 6) da.issue_one(m / 8, x, oa, sa, wave);
            if constexpr ((cp & 2) && m % 8 == 2) db.issue_one(m / 8, y, ob, sb, wave);
            __builtin_amdgcn_sched_barrier(0);
        });
    };
    static_assert(COPIES == 8, "one copy per eight product slots");
    using T_ = std::true_type;
    using F_ = std::false_type;
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using C0 = std::integral_constant<int, 0>;
    using C1 = std::integral_constant<int, 1>;
    using C2 = std::integral_constant<int, 2>;
    using C3 = std::integral_constant<int, 3>;

    setup(vid, ta, tb, tz);
    sfor<COPIES>([&](auto I) { da.issue_one(decltype(I)::value, x, ta, sa, wave); });
    sfor<COPIES>([&](auto I) { db.issue_one(decltype(I)::value, y, tb, sb, wave); });
    if constexpr (NK == 2) issue_k1(ta, tb);
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    for (;;) {
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        // the next tile (the last tile copies itself again: its slots are
        // free by then, and the count of copies stays fixed)
        const uint32_t next = vid + gridDim.x;
        const bool more = next < n_lin;
        int32_t nta = ta, ntb = tb, ntz = tz;
        if (more) setup(next, nta, ntb, ntz);
#pragma unroll
        for (int i = 0; i < NI; ++i)
#pragma unroll
            for (int j = 0; j < NJ; ++j)
#pragma unroll
                for (int e = 0; e < 4; ++e) acc[i][j][e] = 0.f;
        acc16_fence(acc);
        sfor<NAR>([&](auto I) { fa.template read_rt<0, decltype(I)::value>(A0, 0u); });
        sfor<NBR>([&](auto I) { fb.template read_one<0, 0, decltype(I)::value>(B0); });
        lds_wait<0>();
        A0.ready();
        B0.ready();
        kstep(T_{}, I0{}, I1{}, C0{}, A0, B0, A1, B1, 0u, 0, 0);
        lds_wait<0>();
        A1.ready();
        B1.ready();
        lds_barrier();   // every wave is done reading slot 0: the next tile's k-tile 0 may land there
        if constexpr (NK == 2) {
            kstep(T_{}, I1{}, I0{}, C1{}, A1, B1, A0, B0, (uint32_t)STAGE_BYTES, nta, ntb);
            lds_wait<0>();
            A0.ready();
            B0.ready();
            kstep(T_{}, I1{}, I1{}, C2{}, A0, B0, A1, B1, (uint32_t)STAGE_BYTES, nta, ntb);
            lds_wait<0>();
            A1.ready();
            B1.ready();
            kstep(F_{}, I0{}, I0{}, C0{}, A1, B1, A0, B0, 0u, 0, 0);
        } else {
            kstep(F_{}, I0{}, I0{}, C3{}, A1, B1, A0, B0, 0u, nta, ntb);
        }
        acc16_fence(acc);
        lds_barrier();   // every wave is done with the operand slots

        const int32_t ctz = tz + on;
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (NK == 2) issue_k1(nta, ntb);
        __builtin_amdgcn_sched_barrier(0);
        sfor<NI>([&](auto P) {
            constexpr int p = decltype(P)::value;
            __builtin_amdgcn_sched_barrier(0);   // one piece's values in registers at a time
            if constexpr (p > 0) lds_barrier();   // the previous piece's rows are read
            // bind the piece's accumulators here, so that their reads into
            // vector registers are not hoisted over earlier pieces
            asm volatile("" : "+a"(acc[p][0]), "+a"(acc[p][1]), "+a"(acc[p][2]), "+a"(acc[p][3]), "+a"(acc[p][4]),
                              "+a"(acc[p][5]), "+a"(acc[p][6]), "+a"(acc[p][7]));
            // the piece's 32 values first, then their writes: one register per
            // value, so the reads, products and writes pipeline instead of
            // waiting on each other through one register
            uint32_t val[NJ * 4];
            sfor<NJ * 4>([&](auto W) {
                constexpr int j = decltype(W)::value / 4, e = decltype(W)::value % 4;
                val[decltype(W)::value] = __builtin_bit_cast(uint32_t, acc[p][j][e] * v.post_scale);
            });
            __builtin_amdgcn_sched_barrier(0);
            sfor<NJ * 4>([&](auto W) {
                constexpr int j = decltype(W)::value / 4, e = decltype(W)::value % 4;
                constexpr int off = (e * 256 + (j >> 1) * 64) * 4;
                ds_write4_at<off>((j & 1) ? wbo : wbe, val[decltype(W)::value]);
            });
            lds_wait<0>();
            lds_barrier();
            const int32_t rowbase = ctz + __builtin_amdgcn_readlane(piece_row, p);
            u32x4_t d[8];
            sfor<8>([&](auto R) {
                constexpr int r = decltype(R)::value;
                d[r] = ds_read16_at<r * 1024>(rbase[r >> 2]);
            });
            lds_wait<0>();
            sfor<8>([&](auto R) {
                constexpr int r = decltype(R)::value;
                lds_ready(d[r]);
                const int32_t o = rowbase + __builtin_amdgcn_readlane(band_row, 8 * wave + r);
                // streaming stores: the tile is not read again here (13-14%
                // faster than plain stores on the attention scores)
                __builtin_nontemporal_store(d[r], (u32x4_t *)(z + o));
            });
        });
        if (!more) {
            // the last tile's own copies again: landed before the workgroup
            // gives up its LDS
            __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
            break;
        }
        vid = next;
        ta = nta;
        tb = ntb;
        tz = ntz;
        // the next tile's copies, then this tile's 64 stores per lane: the
        // copies have landed once at most 63 operations are outstanding (the
        // barrier at the top of the loop then publishes them; the last
        // piece's rows were read before their stores)
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(63));
    }
}

// Compute units of the current device (0 if it cannot be read), cached per
// device.
static int device_cus()
{
    static int cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
    if (!cache[dev]) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
        cache[dev] = n;
    }
    return cache[dev];
}
// TRA_NO_SHORT_TILE_LOOP=1 keeps short fp32 products on the one-tile-per-
// workgroup kernel (for comparisons).
static bool short_enabled()
{
    static const int on = [] {
        const char *e = getenv("TRA_NO_SHORT_TILE_LOOP");
        return (e && e[0] == '1') ? 0 : 1;
    }();
    return on != 0;
}

template <typename TO>
static int launch4k_t(const tra_plan_s &p, const void *x, const void *y, void *z, void *ws, hipStream_t s,
                      bool vec_ok)
{
    const GemmView &v = p.gv;
    dim3 grid((v.gm.total / mf4k::BM) * (v.gn.total / mf4k::BN), v.gb.total, v.split);
    const void *out = v.split > 1 ? ws : z;
    const bool vec = vec_ok && v.z_vec4 && ((uintptr_t)out % 16) == 0;
    if constexpr (std::is_same<TO, float>::value) {
        const uint32_t n_lin = grid.x * grid.y;
        const int cus = device_cus();
        if (p.tile == 4 && short_enabled() && vec && v.split == 1 && v.k_per_split <= 2 * mf4k::BK && cus >= 8 &&
            n_lin > (uint32_t)cus) {
            void (*ks)(GemmView, const uint16_t *, const uint16_t *, float *);
            const bool two = v.k_per_split == 2 * mf4k::BK;
#define TRA_PICKS(AK, BK) ks = two ? k_mfma4k_short<AK, BK, 2> : k_mfma4k_short<AK, BK, 1>
            if (p.a_kmajor) {
                if (p.b_kmajor) TRA_PICKS(true, true);
                else TRA_PICKS(true, false);
            } else {
                if (p.b_kmajor) TRA_PICKS(false, true);
                else TRA_PICKS(false, false);
            }
#undef TRA_PICKS
            const uint32_t g = (uint32_t)cus & ~7u;   // a multiple of 8: a workgroup's tiles stay on its XCD
            hipLaunchKernelGGL(ks, dim3(g), dim3(mf4k::NT), 0, s, v, (const uint16_t *)x, (const uint16_t *)y,
                               (float *)z);
            return (int)hipGetLastError();
        }
    }
    void (*kern)(GemmView, const uint16_t *, const uint16_t *, TO *, float *);
    if (p.tile == 5) {
        // the narrow tile: 256 x 128, direct epilogue
        grid.x = (v.gm.total / mf4k::BM) * (v.gn.total / 128);
        if (p.a_kmajor) kern = p.b_kmajor ? k_mfma4k_bf16<true, true, TO, false, 128> : k_mfma4k_bf16<true, false, TO, false, 128>;
        else kern = p.b_kmajor ? k_mfma4k_bf16<false, true, TO, false, 128> : k_mfma4k_bf16<false, false, TO, false, 128>;
        hipLaunchKernelGGL(kern, grid, dim3(mf4k::NT), 0, s, v, (const uint16_t *)x, (const uint16_t *)y, (TO *)z,
                           (float *)ws);
        return (int)hipGetLastError();
    }
#define TRA_PICK4K(AK, BK) kern = vec ? k_mfma4k_bf16<AK, BK, TO, true> : k_mfma4k_bf16<AK, BK, TO, false>
    if (p.a_kmajor) {
        if (p.b_kmajor) TRA_PICK4K(true, true);
        else TRA_PICK4K(true, false);
    } else {
        if (p.b_kmajor) TRA_PICK4K(false, true);
        else TRA_PICK4K(false, false);
    }
#undef TRA_PICK4K
    hipLaunchKernelGGL(kern, grid, dim3(mf4k::NT), 0, s, v, (const uint16_t *)x, (const uint16_t *)y, (TO *)z,
                       (float *)ws);
    return (int)hipGetLastError();
}

int launch_mfma4k(const tra_plan_s &p, const void *x, const void *y, void *z, void *ws, void *stream, bool out_f32,
                  bool vec_ok)
{
    hipStream_t s = (hipStream_t)stream;
    return out_f32 ? launch4k_t<float>(p, x, y, z, ws, s, vec_ok) : launch4k_t<bf16_t>(p, x, y, z, ws, s, vec_ok);
}

template <typename TO>
static int launch4k_chain_t(const tra_plan_s &p, const void *x, const void *y, void *z, const ChainEpi &ce,
                            hipStream_t s)
{
    const GemmView &v = p.gv;
    dim3 grid((v.gm.total / mf4k::BM) * (v.gn.total / mf4k::BN), v.gb.total, 1);
    bool yrow = true;
    for (int i = 0; i < kP2Max; ++i)
        if (ce.rn.mask[i] && ce.rn.st[0][i]) yrow = false;
    const bool ch = ce.join_a == J_SUB && ce.join_b == J_MUL;
    void (*k)(GemmView, const uint16_t *, const uint16_t *, TO *, ChainEpi);
#define TRA_PICK4KC(AK, BK)                                                                                    \
    k = !ch ? k_mfma4k_chain<AK, BK, TO, 0, false>                                                             \
            : (yrow ? k_mfma4k_chain<AK, BK, TO, 1, true> : k_mfma4k_chain<AK, BK, TO, 1, false>)
    if (p.a_kmajor) {
        if (p.b_kmajor) TRA_PICK4KC(true, true);
        else TRA_PICK4KC(true, false);
    } else {
        if (p.b_kmajor) TRA_PICK4KC(false, true);
        else TRA_PICK4KC(false, false);
    }
#undef TRA_PICK4KC
    hipLaunchKernelGGL(k, grid, dim3(mf4k::NT), 0, s, v, (const uint16_t *)x, (const uint16_t *)y, (TO *)z, ce);
    return (int)hipGetLastError();
}

int launch_mfma4k_chain(const tra_plan_s &p, const ChainEpi &ce, bool out_f32, const void *x, const void *y, void *z,
                        void *stream)
{
    hipStream_t s = (hipStream_t)stream;
    return out_f32 ? launch4k_chain_t<float>(p, x, y, z, ce, s) : launch4k_chain_t<bf16_t>(p, x, y, z, ce, s);
}

}  // namespace tra
