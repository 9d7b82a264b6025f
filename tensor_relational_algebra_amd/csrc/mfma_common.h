// mfma_common.h -- device helpers shared by the matrix-core tile kernels
// (k_mfma.hip: the eight-wave and four-wave 32-deep tiles; k_mfma4k.hip: the
// four-wave 64-deep tile): fragment types, tile order, LDS layouts and raw
// LDS reads, the direct global -> LDS copy plans, and the four-wave tile's
// epilogues.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdlib>
#include <type_traits>
#include <utility>

#include "device_common.h"
#include "graph.h"
#include "plan.h"

namespace tra {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx16_t __attribute__((ext_vector_type(16)));
typedef float floatx4_t __attribute__((ext_vector_type(4)));
typedef short shortx8_t __attribute__((ext_vector_type(8)));

struct MfmaCfg {
    int bm, bn, wm, wn;
};
// variant 0: 256x256 tile, 8 waves (2 x 4), wave tile 128x64
// variant 1: 128x128 tile, 4 waves (2 x 2), wave tile 64x64
// variant 2: 64x64 tile, 4 waves (2 x 2), wave tile 32x32
__host__ __device__ constexpr MfmaCfg mfma_cfg(int v)
{
    return v == 0 ? MfmaCfg{256, 256, 2, 4} : v == 1 ? MfmaCfg{128, 128, 2, 2} : MfmaCfg{64, 64, 2, 2};
}
constexpr int MF_BK = 32;       // k per pipeline stage
constexpr int MF_STAGES = 4;    // LDS ring: 3 k-tiles in flight while one is consumed


// Output group (batch index) and tile of this workgroup.  Consecutive
// workgroup ids land on different XCDs (round-robin dispatch); the ids are
// regrouped so that each XCD owns a contiguous run of tiles, and tile columns
// are swept within groups of 4 tile-rows so that neighbouring tiles share
// operand panels in L2.  With few tiles per output group (a batched product
// whose per-group operand is read by every tile of the group, such as the
// attention weighted sum) the run is taken over all groups, so that a
// group's tiles share one XCD and its operand is fetched once.
// (bx, by): the tile's index within its output group and the group; tile
// (bx, by) runs on XCD (bx + nb * by) % 8.
__device__ __forceinline__ void mfma_tile_at(uint32_t bx, uint32_t by, uint32_t nb, uint32_t tiles_n,
                                             uint32_t n_groups, uint32_t &bidx, uint32_t &tm, uint32_t &tn)
{
    uint32_t b = bx;
    bidx = by;
    const uint32_t n_lin = nb * n_groups;
    if (nb <= 64 && n_groups > 1 && n_lin % 8 == 0) {
        const uint32_t l = bx + nb * by;
        const uint32_t lin = (l % 8) * (n_lin / 8) + l / 8;
        bidx = lin / nb;
        b = lin % nb;
    } else if (nb % 8 == 0) {
        b = (b % 8) * (nb / 8) + b / 8;
    }
    const uint32_t G = 4;
    uint32_t tiles_m = nb / tiles_n;
    uint32_t per = G * tiles_n;
    uint32_t g = b / per, first = g * G;
    uint32_t gs = min(tiles_m - first, G);
    uint32_t r = b % per;
    tm = first + r % gs;
    tn = r / gs;
}
__device__ __forceinline__ void mfma_tile_of(uint32_t nb, uint32_t tiles_n, uint32_t n_groups, uint32_t &bidx,
                                             uint32_t &tm, uint32_t &tn)
{
    mfma_tile_at(blockIdx.x, blockIdx.y, nb, tiles_n, n_groups, bidx, tm, tn);
}

template <int... Is, typename F>
__device__ __forceinline__ void sfor_seq(std::integer_sequence<int, Is...>, F &&f)
{
    (f(std::integral_constant<int, Is>{}), ...);
}
// f(std::integral_constant<int, i>) for i = 0 .. N-1, unrolled at compile time
template <int N, typename F>
__device__ __forceinline__ void sfor(F &&f)
{
    sfor_seq(std::make_integer_sequence<int, N>{}, f);
}

typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void_t;

// LDS layouts (no padding; 16-byte granules permuted by XOR so that the
// matrix-core fragment reads hit distinct banks):
//  * K-major operand, [row][32 k]: 4 granules per row, granule c of row r
//    stored at c ^ swz_k(r);
//  * MN-major operand, [32 k][row]: granule g of k-row k stored at
//    g ^ swz_n(k), read back transposed by ds_read_b64_tr_b16.
__device__ __forceinline__ int swz_k(int r) { return ((r >> 1) ^ (r >> 2)) & 3; }
template <int ROWS>
__device__ __forceinline__ int swz_n(int k) { return ((k & 3) << 2) & (ROWS / 8 - 1); }

// s_waitcnt immediate that waits until at most n vector-memory loads are
// outstanding (expcnt and lgkmcnt left unconstrained).
constexpr int vmcnt_imm(int n) { return (n & 0xF) | ((n >> 4) << 14) | (0x7 << 4) | (0xF << 8); }

// LDS byte address of a pointer into a __shared__ array.
__device__ __forceinline__ uint32_t lds_addr(const void *p)
{
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void *)p;
}

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

// Fragment reads issued as raw LDS instructions.  The compiler neither waits
// for them nor reorders them against each other; lds_ready() then waits for
// all of them and hands every fragment register through an asm that follows
// the wait, so no consumer can be scheduled before the data has arrived.
// (Left to itself the compiler waits for every in-flight global->LDS copy
// before an LDS read it cannot prove disjoint from them.)
__device__ __forceinline__ u32x4_t ds_read16(uint32_t addr)
{
    u32x4_t v;
    asm volatile("ds_read_b128 %0, %1" : "=v"(v) : "v"(addr));
    return v;
}
__device__ __forceinline__ u32x2_t ds_read8_tr(uint32_t addr)
{
    u32x2_t v;
    asm volatile("ds_read_b64_tr_b16 %0, %1" : "=v"(v) : "v"(addr));
    return v;
}
__device__ __forceinline__ void lds_wait_all() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }
template <typename T>
__device__ __forceinline__ void lds_ready(T &v)
{
    asm volatile("" : "+v"(v));
}

// One 16-byte direct global -> LDS copy per lane, into the wave's 1 KiB of
// LDS at `stage`, from g + koff + the lane's offset (elements).
#ifndef TRA_DMA_BUFFER
#define TRA_DMA_BUFFER 1
#endif
__device__ __forceinline__ void dma_copy16(const uint16_t *__restrict__ g, int32_t koff, uint32_t lane_off,
                                           uint16_t *stage)
{
#if TRA_DMA_BUFFER
    // buffer form: the operand's base in a buffer descriptor, the k-tile term
    // as the scalar offset and the lane's byte offset as the vector offset,
    // so a copy needs no per-lane address arithmetic
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc((void *)g, (short)0, -1, 0x00020000);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t *)stage, 16, lane_off * 2u, (uint32_t)koff * 2u, 0, 0);
#else
    // (The empty asm keeps the 32-bit offset a 32-bit value at the copy, so the
    // address stays "scalar base + zero-extended lane offset" and the copy
    // takes the scalar-base form; a zero extension hoisted out of a loop turns
    // it into a 64-bit per-lane add per copy.)
    uint32_t byte_off = lane_off * 2u;
    asm volatile("" : "+v"(byte_off));
    __builtin_amdgcn_global_load_lds((const void *)((const char *)(g + koff) + byte_off), (lds_void_t *)stage, 16, 0,
                                     0);
#endif
}

// Per-thread plan of the direct global -> LDS copies of one operand tile
// (ROWS x 32 k).  Copy r of thread tid moves 16-byte granule p = r*NT + tid of
// the stage; a wave's 64 copies land on 64 consecutive granules, so the LDS
// address is wave-uniform and the source address carries the permutation.
template <int ROWS, int NT, bool KM, int T>
struct DmaPlan {
    static constexpr int N = ROWS * MF_BK / 8 / NT;   // copies per thread per stage
    int32_t src[N];                                    // source offset minus the k-tile term

    __device__ __forceinline__ void init(const Pow2Group &g_rows, const Pow2Group &gk, uint32_t r0, int32_t base,
                                         int tid)
    {
        const int32_t rbase = p2off<0>(g_rows, r0) + base;
#pragma unroll
        for (int i = 0; i < N; ++i) {
            const int p = i * NT + tid;
            if constexpr (KM) {
                const int row = p >> 2, c = (p & 3) ^ swz_k(p >> 2);
                src[i] = rbase + p2off<0>(g_rows, row) + p2off<T>(gk, c * 8);
            } else {
                const int k = p / (ROWS / 8), gl = (p % (ROWS / 8)) ^ swz_n<ROWS>(p / (ROWS / 8));
                src[i] = rbase + p2off<0>(g_rows, gl * 8) + p2off<T>(gk, k);
            }
        }
    }
    __device__ __forceinline__ void issue(const uint16_t *__restrict__ g, int32_t koff, uint16_t *stage, int wave)
    {
#pragma unroll
        for (int i = 0; i < N; ++i) issue_one(i, g, koff, stage, wave);
    }
    // copy i alone (i a compile-time constant at every call).  The address is
    // the wave-uniform k-tile base plus the lane's 32-bit byte offset, so the
    // copy takes the scalar-base form with no per-lane address arithmetic.
    __device__ __forceinline__ void issue_one(int i, const uint16_t *__restrict__ g, int32_t koff, uint16_t *stage,
                                              int wave)
    {
        dma_copy16(g, koff, (uint32_t)src[i], stage + (i * NT + wave * 64) * 8);
    }
};

// ---------------------------------------------------------------------------
// Four-wave 256 x 256 tile (variant 3).  Each wave owns a 128 x 128 block of
// the tile, 4 x 4 products of 32 x 32, so the 256 fp32 accumulators of a lane
// sit in the accumulator registers (one wave per SIMD leaves all 512 of a
// lane's registers to it) and each byte read from LDS feeds 1.5x the matrix
// work of the eight-wave tile.  With one wave per SIMD there is no second
// wave to hide the LDS latency, so the fragments of the next 16-deep k-step
// are read while the matrix cores work on the current one (two fragment sets
// in registers), and the barrier that publishes a stage sits between the two
// k-steps of the stage before it.
//
// Block i of a wave covers rows (i * WM + wm) * 32 .. +32 of the tile (and
// block j columns (j * WN + wn) * 32 ..): with the waves' blocks interleaved,
// a fragment's LDS address is a per-lane base plus a constant, so every
// fragment read is one instruction with an immediate offset (a handful of
// address registers instead of one per read).
namespace mf4 {
constexpr int BM = 256, BN = 256, BK = 32, WM = 2, WN = 2, NT = WM * WN * 64, TM = 4, TN = 4;
}

template <int OFF>
__device__ __forceinline__ u32x4_t ds_read16_at(uint32_t addr)
{
    static_assert(OFF >= 0 && OFF < 65536, "LDS immediate offset");
    u32x4_t v;
    asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(v) : "v"(addr), "i"(OFF));
    return v;
}
template <int OFF>
__device__ __forceinline__ u32x2_t ds_read8_tr_at(uint32_t addr)
{
    static_assert(OFF >= 0 && OFF < 65536, "LDS immediate offset");
    u32x2_t v;
    asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(v) : "v"(addr), "i"(OFF));
    return v;
}
// s_waitcnt lgkmcnt(n) (vmcnt and expcnt unconstrained)
template <int N>
__device__ __forceinline__ void lds_wait()
{
    static_assert(N >= 0 && N < 16, "lgkmcnt");
    asm volatile("s_waitcnt lgkmcnt(%0)" ::"n"(N) : "memory");
}

template <int OFF>
__device__ __forceinline__ u32x2_t ds_read8_at(uint32_t addr)
{
    static_assert(OFF >= 0 && OFF < 65536, "LDS immediate offset");
    u32x2_t v;
    asm volatile("ds_read_b64 %0, %1 offset:%2" : "=v"(v) : "v"(addr), "i"(OFF));
    return v;
}
template <int OFF>
__device__ __forceinline__ void ds_write4_at(uint32_t addr, uint32_t val)
{
    static_assert(OFF >= 0 && OFF < 65536, "LDS immediate offset");
    asm volatile("ds_write_b32 %0, %1 offset:%2" ::"v"(addr), "v"(val), "i"(OFF) : "memory");
}
template <int OFF>
__device__ __forceinline__ void ds_write2_at(uint32_t addr, uint32_t val)
{
    static_assert(OFF >= 0 && OFF < 65536, "LDS immediate offset");
    asm volatile("ds_write_b16 %0, %1 offset:%2" ::"v"(addr), "v"(val), "i"(OFF) : "memory");
}
__device__ __forceinline__ void lds_barrier()
{
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// One operand's fragments of one 16-deep k-step: KM ? one 16-byte read per
// block : two 8-byte transposing reads per block.
template <bool KM, int T>
struct Frag4 {
    u32x4_t k[T];
    u32x2_t t[T][2];
    __device__ __forceinline__ void ready()
    {
#pragma unroll
        for (int i = 0; i < T; ++i) {
            if constexpr (KM) {
                lds_ready(k[i]);
            } else {
                lds_ready(t[i][0]);
                lds_ready(t[i][1]);
            }
        }
    }
    __device__ __forceinline__ bf16x8_t op(int i) const
    {
        if constexpr (KM) {
            return __builtin_bit_cast(bf16x8_t, k[i]);
        } else {
            u32x4_t w = {t[i][0][0], t[i][0][1], t[i][1][0], t[i][1][1]};
            return __builtin_bit_cast(bf16x8_t, w);
        }
    }
    static constexpr int reads = KM ? T : 2 * T;
};

// Per-lane LDS bases of one operand's fragment reads (ROWS rows in the tile,
// W waves along them, wave index w, STAGES stages of ROWS x 32 bf16).
//  * K-major, stage [row][32 k]: block i of k-step ks reads row
//    (i W + w) 32 + l%32, 16-byte granule (2 ks + l/32) ^ swz_k(row); the
//    swizzle depends on row bits 1..3 only, so the base depends on ks alone.
//  * MN-major, stage [32 k][row]: the swizzle XORs granule bits 2..3 with
//    k & 3, which for W = 2 mixes in bit 0 of i: two bases (i & 1).
// Stages at or past 64 KiB take a second base 64 KiB up (the immediate
// offset of a DS instruction has 16 bits).
template <bool KM, int ROWS, int W, int STAGES>
struct FragAddr4 {
    static constexpr int STAGE_BYTES = ROWS * mf4::BK * 2;
    static constexpr int NB = KM ? 2 : (W >= 4 ? 1 : 4 / W);
    uint32_t base[2][NB];   // [stage >= 64 KiB][ks (K-major) or i % NB (MN-major)]

    __device__ __forceinline__ void init(uint32_t lds, int w, int lane)
    {
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            uint32_t a;
            if constexpr (KM) {
                const int r = w * 32 + (lane & 31);
                const int c = ((2 * b + (lane >> 5)) ^ swz_k(r));
                a = (uint32_t)(r * mf4::BK + c * 8) * 2;
            } else {
                const int g = lane >> 4, sl = lane & 15;
                const int kb = 8 * (g >> 1) + (sl >> 2);
                const int nb = (b * W + w) * 32 + 16 * (g & 1) + 4 * (sl & 3);
                a = (uint32_t)(kb * ROWS + (((nb >> 3) ^ swz_n<ROWS>(kb)) << 3) + (nb & 7)) * 2;
            }
            base[0][b] = lds + a;
            base[1][b] = lds + a + 65536;
        }
    }
    // Issue read R of k-step KS of stage G into f (K-major: block R;
    // MN-major: block R / 2, half R % 2).
    template <int G, int KS, int R, int T>
    __device__ __forceinline__ void read_one(Frag4<KM, T> &f) const
    {
        constexpr int SOFF = G * STAGE_BYTES, HI = SOFF >= 65536 ? 1 : 0, S0 = SOFF - HI * 65536;
        if constexpr (KM) {
            constexpr int off = S0 + R * W * 32 * mf4::BK * 2;
            f.k[R] = ds_read16_at<off>(base[HI][KS]);
        } else {
            constexpr int i = R / 2, h = R % 2, r = i % NB, q = i / NB;
            constexpr int off = S0 + KS * 16 * ROWS * 2 + q * NB * W * 32 * 2 + h * 4 * ROWS * 2;
            f.t[i][h] = ds_read8_tr_at<off>(base[HI][r]);
        }
    }
    // Issue the reads of k-step KS of stage G into f.
    template <int G, int KS, int T>
    __device__ __forceinline__ void read(Frag4<KM, T> &f) const
    {
        constexpr int SOFF = G * STAGE_BYTES, HI = SOFF >= 65536 ? 1 : 0, S0 = SOFF - HI * 65536;
        sfor<T>([&](auto I) {
            constexpr int i = decltype(I)::value;
            if constexpr (KM) {
                constexpr int off = S0 + i * W * 32 * mf4::BK * 2;
                f.k[i] = ds_read16_at<off>(base[HI][KS]);
            } else {
                // block i = q NB + r: r selects the base, q adds 4 W-blocks of
                // 32 rows' worth of granules (above the swizzled bits)
                constexpr int r = i % NB, q = i / NB;
                constexpr int off = S0 + KS * 16 * ROWS * 2 + q * NB * W * 32 * 2;
                f.t[i][0] = ds_read8_tr_at<off>(base[HI][r]);
                f.t[i][1] = ds_read8_tr_at<off + 4 * ROWS * 2>(base[HI][r]);
            }
        });
    }
};

// Epilogue of the four-wave tile through LDS, for outputs whose four
// consecutive columns are one aligned vector: the tile goes out in two halves
// of 128 rows; each wave writes its accumulators of the half (times sc, as S)
// into a row-major staging tile (rows 0-63 of the half in the freed stages of
// the first operand, rows 64-127 in those of the second), and after a barrier
// reads back 32 whole rows of it, four consecutive columns per lane, and hands
// each row to emit(PH, RR, data): half PH, row RR of the wave's 32, data
// holding columns 4*lane .. 4*lane + 3 of tile row PH*128 + wave*32 + RR.
// pre(PH) runs at the start of half PH, before its staging writes (loads a
// caller issues there are in flight during them).
//
// Accumulator layouts (the wave's blocks interleaved with the other waves'):
//  * Acc32 = floatx16_t[4][4] (32x32x16 products): element e of block (i, j)
//    holds row (2i + wm)*32 + 8(e/4) + 4(l/32) + e%4, column (2j + wn)*32 + l%32;
//  * Acc16 = floatx4_t[8][8] (16x16x32 products): element e of block (i, j)
//    holds row (2i + wm)*16 + 4(l/16) + e, column (2j + wn)*16 + l%16.
using Acc32 = floatx16_t[mf4::TM][mf4::TN];
using Acc16 = floatx4_t[2 * mf4::TM][2 * mf4::TN];

template <typename S, typename ACC, typename Pre, typename Emit>
__device__ __forceinline__ void mfma4_staged(const ACC &acc, uint32_t st_a, uint32_t st_b, float sc, int wave,
                                             int lane, Pre &&pre, Emit &&emit)
{
    constexpr bool L16 = std::is_same<ACC, Acc16>::value;
    using namespace mf4;
    constexpr int ES = sizeof(S);
    constexpr int RB = BN * ES;   // bytes of one staged row
    const int wm = wave / WN, wn = wave % WN;
    // Block ii of the half (rows ii*64 .. +63) goes to st_a (ii = 0) or st_b
    // (ii = 1); within it, the lane's row is wm*32 + 4*(lane/32) + 8q + r and
    // its column (j*2 + wn)*32 + lane%32.
    const uint32_t wl = L16 ? (uint32_t)(((wm * 16 + 4 * (lane >> 4)) * BN + wn * 16 + (lane & 15)) * ES)
                            : (uint32_t)(((wm * 32 + 4 * (lane >> 5)) * BN + wn * 32 + (lane & 31)) * ES);
    const uint32_t wb[2] = {st_a + wl, st_b + wl};
    // read base: rows (wave%2)*32 .. +31 of block wave/2, columns 4*lane .. +3
    const uint32_t rb = (wave < 2 ? st_a : st_b) + (uint32_t)(((wave & 1) * 32 * BN + 4 * lane) * ES);
    using D = typename std::conditional<ES == 4, u32x4_t, u32x2_t>::type;
    sfor<2>([&](auto PH) {
        constexpr int ph = decltype(PH)::value;
        if constexpr (ph == 1) lds_barrier();   // every wave done reading the first half
        pre(PH);
        if constexpr (L16) {
            // blocks i = 4 ph .. 4 ph + 3 of the 16-row blocks: block il = i - 4 ph
            // goes to st_a (il < 2) or st_b, at row (il % 2)*32 + wm*16 + 4(l/16) + e
            // per block row: its 32 values first, then their writes (one
            // register per value, so the accumulator reads, products and
            // writes pipeline instead of chaining through one register)
            sfor<4>([&](auto IL) {
                constexpr int il = decltype(IL)::value, i = 4 * ph + il;
                __builtin_amdgcn_sched_barrier(0);
                ACC &ma = const_cast<ACC &>(acc);   // the caller's (non-const) accumulators, values unchanged
                asm volatile("" : "+a"(ma[i][0]), "+a"(ma[i][1]), "+a"(ma[i][2]), "+a"(ma[i][3]), "+a"(ma[i][4]),
                                  "+a"(ma[i][5]), "+a"(ma[i][6]), "+a"(ma[i][7]));
                uint32_t val[2 * TN * 4];
                sfor<2 * TN * 4>([&](auto W) {
                    constexpr int w = decltype(W)::value, j = w / 4, e = w % 4;
                    const float f = ma[i][j][e] * sc;
                    if constexpr (ES == 4) val[w] = __builtin_bit_cast(uint32_t, f);
                    else val[w] = (uint32_t)f32_to_bf16(f);
                });
                __builtin_amdgcn_sched_barrier(0);
                sfor<2 * TN * 4>([&](auto W) {
                    constexpr int w = decltype(W)::value, j = w / 4, e = w % 4;
                    constexpr int off = (((il % 2) * 32 + e) * BN + j * WN * 16) * ES;
                    if constexpr (ES == 4) ds_write4_at<off>(wb[il / 2], val[w]);
                    else ds_write2_at<off>(wb[il / 2], val[w]);
                });
            });
        } else {
            sfor<2 * TN * 16>([&](auto W) {
                constexpr int w = decltype(W)::value;
                constexpr int ii = w / (TN * 16), j = (w / 16) % TN, q = (w / 4) % 4, r = w % 4;
                constexpr int off = ((8 * q + r) * BN + j * WN * 32) * ES;
                const float val = acc[2 * ph + ii][j][4 * q + r] * sc;
                if constexpr (ES == 4) ds_write4_at<off>(wb[ii], __builtin_bit_cast(uint32_t, val));
                else ds_write2_at<off>(wb[ii], (uint32_t)f32_to_bf16(val));
            });
        }
        lds_wait<0>();
        lds_barrier();
        // 32 rows of this wave, 8 at a time: reads, one wait, the rows
        sfor<4>([&](auto G) {
            constexpr int g = decltype(G)::value;
            D d[8];
            sfor<8>([&](auto R) {
                constexpr int off = (8 * g + decltype(R)::value) * RB;
                if constexpr (ES == 4) d[R] = ds_read16_at<off>(rb);
                else d[R] = ds_read8_at<off>(rb);
            });
            lds_wait<0>();
            sfor<8>([&](auto R) {
                lds_ready(d[R]);
                emit(PH, std::integral_constant<int, 8 * g + decltype(R)::value>{}, d[R]);
            });
        });
    });
}

// The plain staged epilogue: each row goes out as one 16-byte (fp32) or
// 8-byte (bf16) vector per lane, so that every store instruction writes one
// contiguous row of the tile.  Values and rounding are those of the direct
// epilogue.
template <typename T, bool SCALE, typename ACC>
__device__ __forceinline__ void mfma4_store_staged(const GemmView &v, T *__restrict__ out, const ACC &acc, uint32_t st_a,
                                                   uint32_t st_b, uint32_t m0, uint32_t n0, int32_t bz, int wave,
                                                   int lane)
{
    const int32_t on = p2off<1>(v.gn, n0 + 4 * lane);
    // lane r < 32 holds the Z offset of row r of a 32-row band
    const int32_t band_row = p2off<1>(v.gm, lane & 31);
    int32_t rowbase[2];
#pragma unroll
    for (int ph = 0; ph < 2; ++ph) rowbase[ph] = p2off<1>(v.gm, m0 + ph * 128 + wave * 32) + bz;
    mfma4_staged<T>(acc, st_a, st_b, SCALE ? v.post_scale : 1.f, wave, lane, [](auto) {}, [&](auto PH, auto RR, const auto &d) {
        const int32_t o = rowbase[decltype(PH)::value] + __builtin_amdgcn_readlane(band_row, decltype(RR)::value) + on;
        // streaming stores (1-2% on the blocked GEMM and on the re-cut that
        // reads its output next)
        __builtin_nontemporal_store(
            d, (typename std::remove_const<typename std::remove_reference<decltype(d)>::type>::type *)(out + o));
    });
}

// The chained epilogue on the staged rows (the product and the two
// elementwise steps of a ChainEpi, as the eight-wave chain computes them):
// the product's fp32 value av (times post_scale), t = join_a(av, ya) times
// scale_a, rounded to TO when TO is bf16, then join_b(xb, t) times scale_b,
// stored as TO.  xb and the output share the output's layout, so each lane
// loads and stores its four columns as one vector; the 32 xb vectors of a
// half are loaded together, before the half is staged.  YROW: ya does not
// vary along the output's columns; lane r then loads ya of row r of the
// wave's 32 once per half, and each row takes it by readlane.
template <typename TO, int CH, bool YROW, typename ACC>
__device__ __forceinline__ void mfma4_chain_staged(const GemmView &v, TO *__restrict__ out, const ChainEpi &ce,
                                                   const ACC &acc, uint32_t st_a,
                                                   uint32_t st_b, uint32_t m0, uint32_t n0, uint32_t bidx, int32_t bz,
                                                   int wave, int lane)
{
    const int32_t on = p2off<1>(v.gn, n0 + 4 * lane);
    const int32_t band_row = p2off<1>(v.gm, lane & 31);
    const int32_t yband_row = p2off<0>(ce.rm, lane & 31);
    int32_t rowbase[2], yrowbase[2];
#pragma unroll
    for (int ph = 0; ph < 2; ++ph) {
        rowbase[ph] = p2off<1>(v.gm, m0 + ph * 128 + wave * 32) + bz;
        yrowbase[ph] = p2off<0>(ce.rb, bidx) + p2off<0>(ce.rm, m0 + ph * 128 + wave * 32);
    }
    int32_t ycol[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) ycol[c] = YROW ? 0 : p2off<0>(ce.rn, n0 + 4 * lane + c);
    const float *__restrict__ ya = (const float *)ce.ya;
    const TO *__restrict__ xb = (const TO *)ce.xb;
    using XV = typename std::conditional<sizeof(TO) == 4, u32x4_t, u32x2_t>::type;
    XV xw[32];
    float yl = 0.f;
    auto pre = [&](auto PH) {
        constexpr int ph = decltype(PH)::value;
        sfor<32>([&](auto RR) {
            constexpr int rr = decltype(RR)::value;
            const int32_t o = rowbase[ph] + __builtin_amdgcn_readlane(band_row, rr) + on;
            xw[rr] = *(const XV *)(xb + o);
        });
        if constexpr (YROW) yl = ya[yrowbase[ph] + yband_row];
    };
    mfma4_staged<float>(acc, st_a, st_b, v.post_scale, wave, lane, pre, [&](auto PH, auto RR, const u32x4_t &d) {
        constexpr int ph = decltype(PH)::value, rr = decltype(RR)::value;
        const int32_t o = rowbase[ph] + __builtin_amdgcn_readlane(band_row, rr) + on;
        float xv[4];
        if constexpr (sizeof(TO) == 4) {
#pragma unroll
            for (int c = 0; c < 4; ++c) xv[c] = __uint_as_float((uint32_t)xw[rr][c]);
        } else {
#pragma unroll
            for (int c = 0; c < 4; ++c) xv[c] = bf16_to_f32((uint16_t)(xw[rr][c / 2] >> (16 * (c % 2))));
        }
        float yrow = 0.f;
        if constexpr (YROW) yrow = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, yl), rr));
        const int32_t yo = yrowbase[ph] + __builtin_amdgcn_readlane(yband_row, rr);
        float res[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            // (the element is read into a scalar first: a bit cast taken
            // directly of a vector element reference read element 0)
            const float av = __uint_as_float((uint32_t)d[c]);
            const float yv = YROW ? yrow : ya[yo + ycol[c]];
            float t;
            if constexpr (CH == 1) t = (av - yv) * ce.scale_a;
            else t = join_any(ce.join_a, av, yv) * ce.scale_a;
            if constexpr (std::is_same<TO, bf16_t>::value) t = bf16_to_f32(f32_to_bf16(t));
            float o4;
            if constexpr (CH == 1) o4 = xv[c] * t;
            else o4 = join_any(ce.join_b, xv[c], t);
            res[c] = o4 * ce.scale_b;
        }
        if constexpr (sizeof(TO) == 4) {
            u32x4_t w = {__builtin_bit_cast(uint32_t, res[0]), __builtin_bit_cast(uint32_t, res[1]),
                         __builtin_bit_cast(uint32_t, res[2]), __builtin_bit_cast(uint32_t, res[3])};
            *(u32x4_t *)(out + o) = w;
        } else {
            u32x2_t w = {(uint32_t)f32_to_bf16(res[0]) | ((uint32_t)f32_to_bf16(res[1]) << 16),
                         (uint32_t)f32_to_bf16(res[2]) | ((uint32_t)f32_to_bf16(res[3]) << 16)};
            *(u32x2_t *)(out + o) = w;
        }
    });
}

// The direct epilogue of the four-wave tile: each lane stores its
// accumulators one element at a time (the output times post_scale, or the
// raw fp32 partial into the split workspace).  Accumulator element e of lane
// l holds row 8*(e/4) + 4*(l/32) + e%4 and column l%32 of its 32x32 block.
template <typename TO>
__device__ __forceinline__ void mfma4_store_direct(const GemmView &v, TO *__restrict__ z, float *__restrict__ wsp,
                                                   bool split, const floatx16_t (&acc)[mf4::TM][mf4::TN],
                                                   uint32_t m0, uint32_t n0, int32_t bz, int wave)
{
    using namespace mf4;
    const int lane = threadIdx.x & 63, wm = wave / WN, wn = wave % WN;
    const int32_t zm0 = p2off<1>(v.gm, m0) + bz, zn0 = p2off<1>(v.gn, n0);
    int32_t lo[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) lo[r] = p2off<1>(v.gm, 4 * (lane >> 5) + r);
#pragma unroll
    for (int i = 0; i < TM; ++i) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int32_t hi = zm0 + p2off<1>(v.gm, (i * WM + wm) * 32 + 8 * q);
#pragma unroll
            for (int j = 0; j < TN; ++j) {
                const int32_t on = zn0 + p2off<1>(v.gn, (j * WN + wn) * 32 + (lane & 31));
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

// The direct epilogue for the 16x16 accumulator layout (Acc16).
template <typename TO, int NJ = 2 * mf4::TN>   // NJ: the wave's 16-column blocks (8, or 4 for 128-wide tiles)
__device__ __forceinline__ void mfma4_store_direct16(const GemmView &v, TO *__restrict__ z, float *__restrict__ wsp,
                                                     bool split, const floatx4_t (&acc)[2 * mf4::TM][NJ],
                                                     uint32_t m0, uint32_t n0, int32_t bz, int wave)
{
    using namespace mf4;
    const int lane = threadIdx.x & 63, wm = wave / WN, wn = wave % WN;
    const int32_t zm0 = p2off<1>(v.gm, m0) + bz, zn0 = p2off<1>(v.gn, n0);
    int32_t lo[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) lo[e] = p2off<1>(v.gm, 4 * (lane >> 4) + e);
#pragma unroll
    for (int i = 0; i < 2 * TM; ++i) {
        const int32_t hi = zm0 + p2off<1>(v.gm, (i * WM + wm) * 16);
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            const int32_t on = zn0 + p2off<1>(v.gn, (j * WN + wn) * 16 + (lane & 15));
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int32_t o = hi + lo[e] + on;
                const float val = acc[i][j][e];
                if (split) wsp[o] = val;
                else Scalar<TO>::store(z, o, val * v.post_scale);
            }
        }
    }
}

// The four-wave 64-deep tile (k_mfma4k.hip): plain product and product chain.
int launch_mfma4k(const tra_plan_s &p, const void *x, const void *y, void *z, void *ws, void *stream, bool out_f32,
                  bool vec_ok);
int launch_mfma4k_chain(const tra_plan_s &p, const ChainEpi &ce, bool out_f32, const void *x, const void *y, void *z,
                        void *stream);

}  // namespace tra
