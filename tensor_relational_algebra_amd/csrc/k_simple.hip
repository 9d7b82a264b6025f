// k_simple.hip -- generic join+aggregate, elementwise, row-reduction,
// split-fold and repartition kernels for gfx950.
//
// Page "EinDecomp：基于爱因斯坦求和与张量关系代数的自动张量并行分解算法",
// section 2.2: a join applies a kernel function to every key-matched pair of
// sub-tensors; an aggregation groups the results by the output part of the
// key and reduces each group; a repartition re-cuts a relation under another
// partition vector.  Here every output element belongs to one group, and the
// thread (or wavefront) that owns it walks the group's contracted partitions
// in ascending key order and each partition's in-block range in row-major
// order, folding the joined values as it goes; nothing is materialised.
#include <hip/hip_runtime.h>

#include "device_common.h"
#include "graph.h"
#include "plan.h"

namespace tra {

// ---------------------------------------------------------------- generic
// One thread per output element, any spec / join / aggregate / layout.
template <typename TI, typename TO>
__global__ __launch_bounds__(256) void k_generic(GenericDesc g, int join, int agg, int two,
                                                 const TI *__restrict__ x, const TI *__restrict__ y,
                                                 TO *__restrict__ z)
{
    using A = typename Scalar<TI>::acc;
    const int last = g.con.n - 1;
    const uint32_t E = last >= 0 ? g.con.ext[last] : 1;
    const int64_t sxl = last >= 0 ? g.con.st[0][last] : 0, syl = last >= 0 ? g.con.st[1][last] : 0;
    const int64_t n_outer = g.n_con / E;
    for (int64_t o = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; o < g.n_out;
         o += (int64_t)gridDim.x * blockDim.x) {
        int64_t xo = 0, yo = 0;
        radix_offsets(g.out, o, xo, yo);
        Fold<A> f;
        f.init(agg);
        for (int64_t c = 0; c < n_outer; ++c) {
            int64_t xc = xo, yc = yo;
            int64_t idx = c;
            for (int i = last - 1; i >= 0; --i) {
                uint32_t e = g.con.ext[i];
                int64_t q = idx / e;
                int64_t dgt = idx - q * e;
                idx = q;
                xc += dgt * g.con.st[0][i];
                yc += dgt * g.con.st[1][i];
            }
            for (uint32_t e = 0; e < E; ++e) {
                A xv = Scalar<TI>::load(x, xc + e * sxl);
                A yv = two ? Scalar<TI>::load(y, yc + e * syl) : A(0);
                f.add(agg, join_any(join, xv, yv));
            }
        }
        Scalar<TO>::store(z, o, (A)f.result(agg, g.post_scale));
    }
}

// ---------------------------------------------------------------- split reduction
// Few outputs, each over a long contracted range (a full reduction, a trace,
// a handful of long dot products).  Output o's range of n_con contracted
// indices (flattened in ascending key order, the last contracted sub-dim
// fastest) is cut into `split` chunks of `chunk` consecutive indices, and
// workgroup (s, o) folds chunk s:
//  * thread t takes the indices of each contracted row inside the chunk at
//    t, t + 256, ... (coalesced when the row is contiguous), folding in that
//    order;
//  * the 64 lanes of a wave combine by a butterfly, and the four waves'
//    partials are folded in wave order through LDS (aggregation tier ii);
//  * with split == 1 that is the output; otherwise partial s goes to
//    ws[s * n_out + o] (logsumexp as the chunk's own logsumexp) and
//    k_split_fold folds the chunks in order (tier iii).
// Every order is fixed, so runs are bitwise reproducible.
template <typename TI, typename TO>
__global__ __launch_bounds__(256) void k_reduce_split(GenericDesc g, int join, int agg, int two,
                                                      const TI *__restrict__ x, const TI *__restrict__ y,
                                                      TO *__restrict__ z, typename Scalar<TI>::acc *__restrict__ ws)
{
    using A = typename Scalar<TI>::acc;
    const int64_t o = blockIdx.y;
    const int64_t s = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    int64_t xo = 0, yo = 0;
    radix_offsets(g.out, o, xo, yo);
    const int last = g.con.n - 1;
    const int64_t inner = g.con.ext[last];
    const int64_t sxl = g.con.st[0][last], syl = g.con.st[1][last];
    const int64_t c0 = s * g.chunk, c1 = min(g.n_con, c0 + g.chunk);
    Fold<A> f;
    f.init(agg);
    for (int64_t r = c0 / inner; r * inner < c1; ++r) {
        int64_t xr = xo, yr = yo, idx = r;
        for (int i = last - 1; i >= 0; --i) {
            const uint32_t e = g.con.ext[i];
            const int64_t q = idx / e;
            const int64_t dgt = idx - q * e;
            idx = q;
            xr += dgt * g.con.st[0][i];
            yr += dgt * g.con.st[1][i];
        }
        const int64_t lo = max(c0 - r * inner, (int64_t)0), hi = min(inner, c1 - r * inner);
        for (int64_t e = lo + tid; e < hi; e += 256) {
            A xv = Scalar<TI>::load(x, xr + e * sxl);
            A yv = two ? Scalar<TI>::load(y, yr + e * syl) : A(0);
            f.add(agg, join_any(join, xv, yv));
        }
    }
    __shared__ A wm[4];
    __shared__ float wsum[4];
    if constexpr (std::is_same<A, float>::value) {
        for (int off = 32; off >= 1; off >>= 1) {
            float om = __shfl_xor(f.m, off, 64);
            float os = __shfl_xor(f.s, off, 64);
            f.merge(agg, om, os);
        }
        if (lane == 0) wsum[wave] = f.s;
    } else {
        for (int off = 32; off >= 1; off >>= 1) f.merge(agg, __shfl_xor(f.m, off, 64), 0);
    }
    if (lane == 0) wm[wave] = f.m;
    __syncthreads();
    if (tid == 0) {
        Fold<A> t;
        t.init(agg);
        for (int w = 0; w < 4; ++w) {
            if constexpr (std::is_same<A, float>::value) t.merge(agg, wm[w], wsum[w]);
            else t.merge(agg, wm[w], 0);
        }
        if (g.split == 1) Scalar<TO>::store(z, o, (A)t.result(agg, g.post_scale));
        else ws[s * g.n_out + o] = agg == A_LSE ? (A)t.result(agg, 1.f) : t.m;
    }
}

// ---------------------------------------------------------------- elementwise
// Aggregate NONE: z = join(x, y) (times post_scale); `vec` consecutive output
// elements share one digit decomposition.
template <typename TI, typename TO>
__global__ __launch_bounds__(256) void k_elemwise(ElemDesc g, int join, int two, const TI *__restrict__ x,
                                                  const TI *__restrict__ y, TO *__restrict__ z)
{
    using A = typename Scalar<TI>::acc;
    const int vec = g.vec;
    const int f = g.out.n - 1;
    const int64_t sx = f >= 0 ? g.out.st[0][f] : 0, sy = f >= 0 ? g.out.st[1][f] : 0;
    const int64_t n_vec = g.n_out / vec;
    for (int64_t v = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; v < n_vec;
         v += (int64_t)gridDim.x * blockDim.x) {
        const int64_t o = v * vec;
        int64_t xo = 0, yo = 0;
        radix_offsets(g.out, o, xo, yo);
        for (int i = 0; i < vec; ++i) {
            A xv = Scalar<TI>::load(x, xo + (vec > 1 ? i * sx : 0));
            A yv = two ? Scalar<TI>::load(y, yo + (vec > 1 ? i * sy : 0)) : A(0);
            A r = join_any(join, xv, yv);
            if constexpr (sizeof(A) == 4 && !std::is_same<A, int32_t>::value) r *= g.post_scale;
            Scalar<TO>::store(z, o + i, r);
        }
    }
}

// ---------------------------------------------------------------- row reduce
// One wavefront per output element.  Lanes stride over the contiguous last
// contracted run (X stride 1); the outer contracted digits (the contracted
// keys first, ascending) are walked in order; the 64 lane partials are then
// combined by a butterfly.
template <typename TI, typename TO>
__global__ __launch_bounds__(256) void k_rowreduce(RowDesc g, int join, int agg, int two,
                                                   const TI *__restrict__ x, const TI *__restrict__ y,
                                                   TO *__restrict__ z)
{
    using A = typename Scalar<TI>::acc;
    const int lane = threadIdx.x & 63;
    const int64_t wave = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
    const int64_t n_waves = ((int64_t)gridDim.x * blockDim.x) >> 6;
    for (int64_t o = wave; o < g.n_out; o += n_waves) {
        int64_t xo = 0, yo = 0;
        radix_offsets(g.out, o, xo, yo);
        Fold<A> f;
        f.init(agg);
        for (int64_t c = 0; c < g.n_outer; ++c) {
            int64_t xc = xo, yc = yo;
            radix_offsets(g.outer, c, xc, yc);
            for (int64_t e = lane; e < g.inner; e += 64) {
                A xv = Scalar<TI>::load(x, xc + e);
                A yv = two ? Scalar<TI>::load(y, yc + e * g.inner_sy) : A(0);
                f.add(agg, join_any(join, xv, yv));
            }
        }
        if constexpr (std::is_same<A, float>::value) {
            for (int off = 32; off >= 1; off >>= 1) {
                float om = __shfl_xor(f.m, off, 64);
                float os = __shfl_xor(f.s, off, 64);
                f.merge(agg, om, os);
            }
        } else {
            for (int off = 32; off >= 1; off >>= 1) f.merge(agg, __shfl_xor(f.m, off, 64), 0);
        }
        if (lane == 0) Scalar<TO>::store(z, o, (A)f.result(agg, g.post_scale));
    }
}

// Four consecutive elements of a tensor (16 bytes of fp32 / int32, 8 bytes of bf16).
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// 16- and 8-byte vector accesses, optionally with the streaming
// (non-temporal) hint for tensors far larger than the caches.
template <bool NT, typename U>
__device__ __forceinline__ U ld_hint(const U *p)
{
    if constexpr (NT) return __builtin_nontemporal_load(p);
    else return *p;
}
template <bool NT, typename U>
__device__ __forceinline__ void st_hint(U *p, U v)
{
    if constexpr (NT) __builtin_nontemporal_store(v, p);
    else *p = v;
}

// Four consecutive elements through native vector registers.
template <typename T> struct Vec4R;
template <> struct Vec4R<float> {
    template <bool NT> static __device__ __forceinline__ void load(const float *p, float v[4])
    {
        const u32x4 u = ld_hint<NT>((const u32x4 *)p);
        for (int i = 0; i < 4; ++i) v[i] = __uint_as_float(u[i]);
    }
    template <bool NT> static __device__ __forceinline__ void store(float *p, const float v[4])
    {
        st_hint<NT>((u32x4 *)p, u32x4{__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]),
                                      __float_as_uint(v[3])});
    }
};
template <> struct Vec4R<bf16_t> {
    template <bool NT> static __device__ __forceinline__ void load(const bf16_t *p, float v[4])
    {
        const u32x2 u = ld_hint<NT>((const u32x2 *)p);
        v[0] = __uint_as_float(u[0] << 16); v[1] = __uint_as_float(u[0] & 0xffff0000u);
        v[2] = __uint_as_float(u[1] << 16); v[3] = __uint_as_float(u[1] & 0xffff0000u);
    }
    template <bool NT> static __device__ __forceinline__ void store(bf16_t *p, const float v[4])
    {
        st_hint<NT>((u32x2 *)p, u32x2{(uint32_t)f32_to_bf16(v[0]) | ((uint32_t)f32_to_bf16(v[1]) << 16),
                                      (uint32_t)f32_to_bf16(v[2]) | ((uint32_t)f32_to_bf16(v[3]) << 16)});
    }
};
template <> struct Vec4R<int32_t> {
    template <bool NT> static __device__ __forceinline__ void load(const int32_t *p, int32_t v[4])
    {
        const u32x4 u = ld_hint<NT>((const u32x4 *)p);
        for (int i = 0; i < 4; ++i) v[i] = (int32_t)u[i];
    }
    template <bool NT> static __device__ __forceinline__ void store(int32_t *p, const int32_t v[4])
    {
        st_hint<NT>((u32x4 *)p, u32x4{(uint32_t)v[0], (uint32_t)v[1], (uint32_t)v[2], (uint32_t)v[3]});
    }
};

template <typename T> struct Vec4;
template <> struct Vec4<float> {
    static __device__ __forceinline__ void load(const float *p, float v[4])
    {
        float4 u = *(const float4 *)p;
        v[0] = u.x; v[1] = u.y; v[2] = u.z; v[3] = u.w;
    }
    static __device__ __forceinline__ void store(float *p, const float v[4]) { *(float4 *)p = float4{v[0], v[1], v[2], v[3]}; }
};
template <> struct Vec4<bf16_t> {
    static __device__ __forceinline__ void load(const bf16_t *p, float v[4])
    {
        uint2 u = *(const uint2 *)p;
        v[0] = __uint_as_float(u.x << 16); v[1] = __uint_as_float(u.x & 0xffff0000u);
        v[2] = __uint_as_float(u.y << 16); v[3] = __uint_as_float(u.y & 0xffff0000u);
    }
    static __device__ __forceinline__ void store(bf16_t *p, const float v[4])
    {
        uint2 u;
        u.x = (uint32_t)f32_to_bf16(v[0]) | ((uint32_t)f32_to_bf16(v[1]) << 16);
        u.y = (uint32_t)f32_to_bf16(v[2]) | ((uint32_t)f32_to_bf16(v[3]) << 16);
        *(uint2 *)p = u;
    }
};
template <> struct Vec4<int32_t> {
    static __device__ __forceinline__ void load(const int32_t *p, int32_t v[4])
    {
        int4 u = *(const int4 *)p;
        v[0] = u.x; v[1] = u.y; v[2] = u.z; v[3] = u.w;
    }
    static __device__ __forceinline__ void store(int32_t *p, const int32_t v[4]) { *(int4 *)p = int4{v[0], v[1], v[2], v[3]}; }
};

// Aggregate NONE, power-of-two digits: each thread owns UPT groups of 4
// consecutive outputs (contiguous in X and Z; Y contiguous or broadcast),
// 256 groups apart; every load is issued before the first store.
template <typename TI, typename TO, int UPT, bool NT>
__global__ __launch_bounds__(256) void k_elemwise_p2(ElemDesc g, int join, int two, const TI *__restrict__ x,
                                                     const TI *__restrict__ y, TO *__restrict__ z)
{
    using A = typename Scalar<TI>::acc;
    const uint32_t n_vec = (uint32_t)(g.n_out / 4);
    const uint32_t base = blockIdx.x * (256u * UPT) + threadIdx.x;
    A xv[UPT][4], yv[UPT][4];
#pragma unroll
    for (int u = 0; u < UPT; ++u) {
        const uint32_t v = base + 256u * u;
        for (int i = 0; i < 4; ++i) xv[u][i] = yv[u][i] = A(0);
        if (v < n_vec) {
            const uint32_t o = v * 4;
            Vec4R<TI>::template load<NT>(x + p2off<0>(g.out_p2, o), xv[u]);
            if (two) {
                const int32_t yo = p2off<1>(g.out_p2, o);
                if (g.y_step) Vec4R<TI>::template load<NT>(y + yo, yv[u]);
                else yv[u][0] = yv[u][1] = yv[u][2] = yv[u][3] = Scalar<TI>::load(y, yo);
            }
        }
    }
#pragma unroll
    for (int u = 0; u < UPT; ++u) {
        const uint32_t v = base + 256u * u;
        if (v >= n_vec) break;
        A r[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            r[i] = join_any(join, xv[u][i], yv[u][i]);
            if constexpr (!std::is_same<A, int32_t>::value) r[i] *= g.post_scale;
        }
        if constexpr (std::is_same<A, int32_t>::value || std::is_same<TO, float>::value || std::is_same<TO, bf16_t>::value)
            Vec4R<TO>::template store<NT>(z + v * 4, r);
    }
}

// Two elementwise EinSums as one pass (tra_execute_chain): t = join_a(xa, ya)
// rounded to plan a's output dtype, then z = join_b(xb, t), with t never
// written.  Both plans enumerate the same output positions in the same
// layout, and plan b's second operand is laid out as its output, so t for
// output group o is the value plan a would have stored at o: the result is
// bit-identical to the two launches.
template <typename TIA, typename TM, typename TO, int UPT, bool NT>
__global__ __launch_bounds__(256) void k_elemwise_chain_p2(ElemDesc ga, int join_a, int two_a, ElemDesc gb,
                                                           int join_b, const TIA *__restrict__ xa,
                                                           const TIA *__restrict__ ya, const TM *__restrict__ xb,
                                                           TO *__restrict__ z)
{
    const uint32_t n_vec = (uint32_t)(ga.n_out / 4);
    const uint32_t base = blockIdx.x * (256u * UPT) + threadIdx.x;
    float av[UPT][4], bv[UPT][4], cv[UPT][4];
#pragma unroll
    for (int u = 0; u < UPT; ++u) {
        const uint32_t v = base + 256u * u;
        for (int i = 0; i < 4; ++i) av[u][i] = bv[u][i] = cv[u][i] = 0.f;
        if (v < n_vec) {
            const uint32_t o = v * 4;
            Vec4R<TIA>::template load<NT>(xa + p2off<0>(ga.out_p2, o), av[u]);
            if (two_a) {
                const int32_t yo = p2off<1>(ga.out_p2, o);
                if (ga.y_step) Vec4R<TIA>::template load<NT>(ya + yo, bv[u]);
                else bv[u][0] = bv[u][1] = bv[u][2] = bv[u][3] = Scalar<TIA>::load(ya, yo);
            }
            Vec4R<TM>::template load<NT>(xb + p2off<0>(gb.out_p2, o), cv[u]);
        }
    }
#pragma unroll
    for (int u = 0; u < UPT; ++u) {
        const uint32_t v = base + 256u * u;
        if (v >= n_vec) break;
        float r[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float t = join_any(join_a, av[u][i], bv[u][i]) * ga.post_scale;
            if constexpr (std::is_same<TM, bf16_t>::value) t = bf16_to_f32(f32_to_bf16(t));
            r[i] = join_any(join_b, cv[u][i], t) * gb.post_scale;
        }
        Vec4R<TO>::template store<NT>(z + v * 4, r);
    }
}

// The same chain for layouts without the power-of-two form: one output
// element per thread, offsets from each plan's radix decomposition.
template <typename TIA, typename TM, typename TO>
__global__ __launch_bounds__(256) void k_elemwise_chain(ElemDesc ga, int join_a, int two_a, ElemDesc gb, int join_b,
                                                        const TIA *__restrict__ xa, const TIA *__restrict__ ya,
                                                        const TM *__restrict__ xb, TO *__restrict__ z)
{
    for (int64_t o = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; o < ga.n_out;
         o += (int64_t)gridDim.x * blockDim.x) {
        int64_t xo = 0, yo = 0, xbo = 0, ybo = 0;
        radix_offsets(ga.out, o, xo, yo);
        radix_offsets(gb.out, o, xbo, ybo);   // ybo == o: plan b's second operand is laid out as its output
        const float av = Scalar<TIA>::load(xa, xo), bv = two_a ? (float)Scalar<TIA>::load(ya, yo) : 0.f;
        float t = join_any(join_a, av, bv) * ga.post_scale;
        if constexpr (std::is_same<TM, bf16_t>::value) t = bf16_to_f32(f32_to_bf16(t));
        Scalar<TO>::store(z, o, join_any(join_b, (float)Scalar<TM>::load(xb, xbo), t) * gb.post_scale);
    }
}


// Row reduction, power-of-two digits: one wavefront per output; each lane
// folds 4 consecutive elements per step (one 16-byte load), the contracted
// keys outermost in ascending order; lanes are combined by a butterfly.
template <typename TI, typename TO>
__global__ __launch_bounds__(256) void k_rowreduce_p2(RowDesc g, int join, int agg, int two,
                                                      const TI *__restrict__ x, const TI *__restrict__ y,
                                                      TO *__restrict__ z)
{
    using A = typename Scalar<TI>::acc;
    const int lane = threadIdx.x & 63;
    const uint32_t wave = (blockIdx.x * blockDim.x + threadIdx.x) >> 6;
    const uint32_t n_waves = (gridDim.x * blockDim.x) >> 6;
    const uint32_t inner = (uint32_t)g.inner, n_outer = (uint32_t)g.n_outer;
    for (uint32_t o = wave; o < (uint32_t)g.n_out; o += n_waves) {
        const int32_t xo = p2off<0>(g.out_p2, o), yo = two ? p2off<1>(g.out_p2, o) : 0;
        Fold<A> f;
        f.init(agg);
        for (uint32_t c = 0; c < n_outer; ++c) {
            const int32_t xc = xo + p2off<0>(g.outer_p2, c);
            const int32_t yc = two ? yo + p2off<1>(g.outer_p2, c) : 0;
            // fold one lane's group of 4 (in ascending order of e)
            auto fold4 = [&](A v[4], const A w[4]) {
#pragma unroll
                for (int i = 0; i < 4; ++i) v[i] = join_any(join, v[i], w[i]);
                if constexpr (std::is_same<A, float>::value) {
                    if (agg == A_LSE) {
                        const float lm = fmaxf(fmaxf(v[0], v[1]), fmaxf(v[2], v[3]));
                        const float nm = fmaxf(f.m, lm);
                        if (nm != -INFINITY) {
                            f.s = f.s * __expf(f.m - nm) + __expf(v[0] - nm) + __expf(v[1] - nm) +
                                  __expf(v[2] - nm) + __expf(v[3] - nm);
                            f.m = nm;
                        }
                        return;
                    }
                }
#pragma unroll
                for (int i = 0; i < 4; ++i) f.add(agg, v[i]);
            };
            auto load4 = [&](uint32_t e, A v[4], A w[4]) {
                Vec4R<TI>::template load<false>(x + xc + e, v);
                w[0] = w[1] = w[2] = w[3] = A(0);
                if (two) {
                    if (g.inner_sy) Vec4R<TI>::template load<false>(y + yc + e, w);
                    else w[0] = w[1] = w[2] = w[3] = Scalar<TI>::load(y, yc);
                }
            };
            uint32_t e = lane * 4;
            // eight 16-byte loads per lane in flight, then their folds
            for (; e + 256 * 7 < inner; e += 256 * 8) {
                A v[8][4], w[8][4];
#pragma unroll
                for (int j = 0; j < 8; ++j) load4(e + 256 * j, v[j], w[j]);
#pragma unroll
                for (int j = 0; j < 8; ++j) fold4(v[j], w[j]);
            }
            for (; e < inner; e += 256) {
                A v[4], w[4];
                load4(e, v, w);
                fold4(v, w);
            }
        }
        if constexpr (std::is_same<A, float>::value) {
            for (int off = 32; off >= 1; off >>= 1) {
                float om = __shfl_xor(f.m, off, 64);
                float os = __shfl_xor(f.s, off, 64);
                f.merge(agg, om, os);
            }
        } else {
            for (int off = 32; off >= 1; off >>= 1) f.merge(agg, __shfl_xor(f.m, off, 64), 0);
        }
        if (lane == 0) Scalar<TO>::store(z, o, (A)f.result(agg, g.post_scale));
    }
}

// ---------------------------------------------------------------- split fold
// Deterministic cross-workgroup aggregation: partial s of output o sits at
// ws[s * n + o]; fold s = 0..S-1 in order, then finish.
template <typename A, typename TO>
__global__ __launch_bounds__(256) void k_split_fold(const A *__restrict__ ws, int64_t n, int split, int agg,
                                                    float scale, TO *__restrict__ z)
{
    for (int64_t o = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; o < n; o += (int64_t)gridDim.x * blockDim.x) {
        Fold<A> f;
        f.init(agg);
        for (int s = 0; s < split; ++s) f.merge(agg, ws[(int64_t)s * n + o], A(1));
        Scalar<TO>::store(z, o, (A)f.result(agg, scale));
    }
}

// ---------------------------------------------------------------- repartition

// Destination positions are enumerated in the destination's own layout, so
// writes are sequential; each digit of the destination index maps to a
// source stride.  U is the copy unit (vec elements).
template <typename U>
__global__ __launch_bounds__(256) void k_repartition(RepartDesc r, int vec, const U *__restrict__ src,
                                                     U *__restrict__ dst)
{
    const int64_t n_units = r.n_elems / vec;
    for (int64_t u = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; u < n_units;
         u += (int64_t)gridDim.x * blockDim.x) {
        int64_t so = 0, unused = 0;
        radix_offsets(r.dst, u * vec, so, unused);
        if (r.scatter) dst[so / vec] = src[u];
        else dst[u] = src[so / vec];
    }
}

// Power-of-two destination digits: 32-bit shifts and masks.  Each workgroup
// copies one contiguous chunk of 256 * UPT destination units; every thread
// issues its UPT independent source loads before any store, so that many
// 16-byte loads are in flight per wave (the copy is bound by HBM latency x
// bandwidth, not by issue).  Full chunks take no bounds checks; only the last
// workgroup's chunk can be partial.  NT marks both sides as streaming
// (non-temporal), for tensors far larger than the caches.
template <bool NT, typename U>
__device__ __forceinline__ U rep_load(const U *p)
{
    if constexpr (NT) return __builtin_nontemporal_load(p);
    else return *p;
}
template <bool NT, typename U>
__device__ __forceinline__ void rep_store(U *p, U v)
{
    if constexpr (NT) __builtin_nontemporal_store(v, p);
    else *p = v;
}

// SC: scatter form (the source read in order, the destination written at
// mapped offsets) instead of the gather form.
template <typename U, int UPT, bool NT, bool SC>
__global__ __launch_bounds__(256) void k_repartition_p2(Pow2Group g, int lvec, uint32_t n_units,
                                                        const U *__restrict__ src, U *__restrict__ dst)
{
    const uint32_t base = blockIdx.x * (256u * UPT) + threadIdx.x;
    if (base + 256u * (UPT - 1) < n_units) {
        U v[UPT];
#pragma unroll
        for (int i = 0; i < UPT; ++i) {
            const uint32_t u = base + 256u * i;
            v[i] = rep_load<NT>(src + (SC ? u : p2off<0>(g, u << lvec) >> lvec));
        }
#pragma unroll
        for (int i = 0; i < UPT; ++i) {
            const uint32_t u = base + 256u * i;
            rep_store<NT>(dst + (SC ? p2off<0>(g, u << lvec) >> lvec : u), v[i]);
        }
    } else {
#pragma unroll
        for (int i = 0; i < UPT; ++i) {
            const uint32_t u = base + 256u * i;
            if (u < n_units) {
                const uint32_t o = p2off<0>(g, u << lvec) >> lvec;
                if (SC) dst[o] = src[u];
                else dst[u] = src[o];
            }
        }
    }
}

template <typename U, bool SC>
static void launch_rep_p2(const Pow2Group &g, int lvec, int64_t n_units, const void *src, void *dst,
                          hipStream_t s)
{
    // Measured on MI355X for a 512 MiB fp32 re-blocking: 8 loads in flight per
    // thread with streaming hints reach 5.7 TB/s (a plain copy 6.3 TB/s);
    // smaller tensors keep more workgroups and cacheable accesses, since
    // their consumer usually reads them next.
    const int64_t bytes = n_units * (int64_t)sizeof(U);
    const uint32_t n = (uint32_t)n_units;
#define TRA_REP_GO(UPT, NT)                                                                               \
    hipLaunchKernelGGL((k_repartition_p2<U, UPT, NT, SC>), dim3((unsigned)((n_units + 256 * UPT - 1) / (256 * UPT))), \
                       dim3(256), 0, s, g, lvec, n, (const U *)src, (U *)dst)
    if (bytes >= (64ll << 20)) TRA_REP_GO(8, true);
    else if (n_units >= 256 * 256 * 4) TRA_REP_GO(4, false);
    else TRA_REP_GO(1, false);
#undef TRA_REP_GO
}

static int grid_for(int64_t work, int per_block = 256)
{
    int64_t b = (work + per_block - 1) / per_block;
    if (b < 1) b = 1;
    if (b > 65536) b = 65536;
    return (int)b;
}

#define TRA_DISPATCH_IO(IN, OUT, CALL)                                                      \
    do {                                                                                    \
        if (IN == D_F32 && OUT == D_F32) { using TI = float; using TO = float; CALL; }      \
        else if (IN == D_F32 && OUT == D_BF16) { using TI = float; using TO = bf16_t; CALL; } \
        else if (IN == D_BF16 && OUT == D_F32) { using TI = bf16_t; using TO = float; CALL; } \
        else if (IN == D_BF16 && OUT == D_BF16) { using TI = bf16_t; using TO = bf16_t; CALL; } \
        else { using TI = int32_t; using TO = int32_t; CALL; }                              \
    } while (0)

static int launch_fold(int64_t n, int split, int agg, float scale, bool int_acc, int out_dtype, const void *ws,
                       void *z, hipStream_t s);

// The split reduction (GenericDesc::split > 0) and, with more than one
// chunk, the in-order fold of its partials.
static int launch_reduce_split(const tra_plan_s &p, const void *x, const void *y, void *z, void *ws,
                               hipStream_t s)
{
    const GenericDesc &g = p.gen;
    dim3 grid((unsigned)g.split, (unsigned)g.n_out);
    TRA_DISPATCH_IO(p.in_dtype, p.out_dtype,
                    hipLaunchKernelGGL((k_reduce_split<TI, TO>), grid, dim3(256), 0, s, g, p.join, p.agg,
                                       p.n_ops == 2 ? 1 : 0, (const TI *)x, (const TI *)y, (TO *)z,
                                       (typename Scalar<TI>::acc *)ws));
    int err = (int)hipGetLastError();
    if (err || g.split == 1) return err;
    return launch_fold(g.n_out, g.split, p.agg, p.post_scale, p.in_dtype == D_I32, p.out_dtype, ws, z, s);
}

int launch_generic(const tra_plan_s &p, const void *x, const void *y, void *z, void *ws, void *stream)
{
    hipStream_t s = (hipStream_t)stream;
    if (p.gen.split > 0) return launch_reduce_split(p, x, y, z, ws, s);
    int grid = grid_for(p.gen.n_out);
    TRA_DISPATCH_IO(p.in_dtype, p.out_dtype,
                    hipLaunchKernelGGL((k_generic<TI, TO>), dim3(grid), dim3(256), 0, s, p.gen, p.join, p.agg,
                                       p.n_ops == 2 ? 1 : 0, (const TI *)x, (const TI *)y, (TO *)z));
    return (int)hipGetLastError();
}

int launch_elemwise(const tra_plan_s &p, const void *x, const void *y, void *z, void *stream)
{
    hipStream_t s = (hipStream_t)stream;
    if (p.el.p2) {
        // as the repartition: four groups per thread, and streaming accesses for
        // tensors far beyond the caches (the [h,s,t] tensors of attention)
        const int64_t n_vec = p.el.n_out / 4;
        const int64_t bytes = p.info.x_bytes + (p.el.y_step ? p.info.y_bytes : 0) + p.info.z_bytes;
        const bool big = bytes >= (64ll << 20), wide = n_vec >= 256 * 256 * 4;
        const int upt = big || wide ? 4 : 1;
        const unsigned grid = (unsigned)((n_vec + 256 * upt - 1) / (256 * upt));
#define TRA_EL_GO(UPT, NT)                                                                                    \
    TRA_DISPATCH_IO(p.in_dtype, p.out_dtype,                                                                  \
                    hipLaunchKernelGGL((k_elemwise_p2<TI, TO, UPT, NT>), dim3(grid), dim3(256), 0, s, p.el,     \
                                       p.join, p.n_ops == 2 ? 1 : 0, (const TI *)x, (const TI *)y, (TO *)z))
        if (big) TRA_EL_GO(4, true);
        else if (wide) TRA_EL_GO(4, false);
        else TRA_EL_GO(1, false);
#undef TRA_EL_GO
        return (int)hipGetLastError();
    }
    int grid = grid_for(p.el.n_out / p.el.vec);
    TRA_DISPATCH_IO(p.in_dtype, p.out_dtype,
                    hipLaunchKernelGGL((k_elemwise<TI, TO>), dim3(grid), dim3(256), 0, s, p.el, p.join,
                                       p.n_ops == 2 ? 1 : 0, (const TI *)x, (const TI *)y, (TO *)z));
    return (int)hipGetLastError();
}

// The softmax node in one pass over its rows: the logsumexp of the row and
// exp(S - LSE) at every element, with the row held in registers in between
// (rows of at most SM_GROUPS * 256 elements).  The two-kernel form reads S
// twice; this one reads it once.  One wavefront per row; lane l owns
// elements 4l..4l+3 of every 256-element group of the row, the groups walked
// as the row-reduce kernel walks them (contracted-key digits outer, the
// contiguous in-block run inner).  The logsumexp is the row maximum plus the
// log of the sum of exp(v - max), each combined across the wavefront by a
// butterfly.  S and the output share one relation layout, so an element's
// output offset is its input offset.
constexpr int SM_GROUPS = 16;
template <typename TO, int NG>
__global__ __launch_bounds__(256) void k_softmax_rows_p2(RowDesc g, const float *__restrict__ x,
                                                         float *__restrict__ lse, TO *__restrict__ z, int per_log2)
{
    // NG = n_outer * inner / 256 groups per row, a compile-time count so that
    // the row stays in registers
    const int lane = threadIdx.x & 63;
    const uint32_t wave = (blockIdx.x * blockDim.x + threadIdx.x) >> 6;
    const uint32_t n_waves = (gridDim.x * blockDim.x) >> 6;
    const int per_mask = (1 << per_log2) - 1;
    for (uint32_t o = wave; o < (uint32_t)g.n_out; o += n_waves) {
        const int32_t xo = p2off<0>(g.out_p2, o);
        float v[NG][4];
        int32_t off[NG];
#pragma unroll
        for (int j = 0; j < NG; ++j) {
            off[j] = xo + p2off<0>(g.outer_p2, (uint32_t)(j >> per_log2)) + (j & per_mask) * 256 + lane * 4;
            Vec4R<float>::load<true>(x + off[j], v[j]);
        }
        float m = -INFINITY;
#pragma unroll
        for (int j = 0; j < NG; ++j) m = fmaxf(m, fmaxf(fmaxf(v[j][0], v[j][1]), fmaxf(v[j][2], v[j][3])));
        for (int sh = 32; sh >= 1; sh >>= 1) m = fmaxf(m, __shfl_xor(m, sh, 64));
        float sum = 0.f;
        if (m != -INFINITY) {
#pragma unroll
            for (int j = 0; j < NG; ++j)
                sum += (__expf(v[j][0] - m) + __expf(v[j][1] - m)) + (__expf(v[j][2] - m) + __expf(v[j][3] - m));
        }
        for (int sh = 32; sh >= 1; sh >>= 1) sum += __shfl_xor(sum, sh, 64);
        const float l = m == -INFINITY ? -INFINITY : m + __logf(sum);
        if (lane == 0) lse[o] = l;
#pragma unroll
        for (int j = 0; j < NG; ++j) {
            float w[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) w[i] = __expf(v[j][i] - l);
            Vec4R<TO>::template store<true>(z + off[j], w);
        }
    }
}

bool softmax_one_pass(const tra_plan_s &lse, const tra_plan_s &norm)
{
    if (lse.kernel != TRA_KERNEL_ROWREDUCE || !lse.row.p2 || lse.agg != A_LSE || lse.n_ops != 1 ||
        lse.in_dtype != D_F32 || lse.post_scale != 1.0f)
        return false;
    if (norm.kernel != TRA_KERNEL_ELEMWISE || norm.join != J_EXP_SUB || norm.info.z_elems != lse.info.x_elems ||
        (norm.out_dtype != D_F32 && norm.out_dtype != D_BF16))
        return false;
    const int64_t inner = lse.row.inner, n_outer = lse.row.n_outer;
    if (inner < 256 || (inner & (inner - 1)) || n_outer < 1 || (n_outer & (n_outer - 1)) ||
        n_outer * inner > SM_GROUPS * 256)
        return false;
    return true;
}

template <typename TO, int NG>
static void launch_softmax_ng(const RowDesc &g, int grid, int per_log2, const void *s, void *lse_out, void *out,
                              hipStream_t st)
{
    hipLaunchKernelGGL((k_softmax_rows_p2<TO, NG>), dim3(grid), dim3(256), 0, st, g, (const float *)s,
                       (float *)lse_out, (TO *)out, per_log2);
}

template <typename TO>
static void launch_softmax_t(const RowDesc &g, int n_groups, int grid, int per_log2, const void *s, void *lse_out,
                             void *out, hipStream_t st)
{
    switch (n_groups) {
    case 1: launch_softmax_ng<TO, 1>(g, grid, per_log2, s, lse_out, out, st); break;
    case 2: launch_softmax_ng<TO, 2>(g, grid, per_log2, s, lse_out, out, st); break;
    case 4: launch_softmax_ng<TO, 4>(g, grid, per_log2, s, lse_out, out, st); break;
    case 8: launch_softmax_ng<TO, 8>(g, grid, per_log2, s, lse_out, out, st); break;
    default: launch_softmax_ng<TO, SM_GROUPS>(g, grid, per_log2, s, lse_out, out, st); break;
    }
}

int launch_softmax_rows(const tra_plan_s &lse, const tra_plan_s &norm, const void *s, void *lse_out, void *out,
                        void *stream)
{
    const RowDesc &g = lse.row;
    int per_log2 = 0;
    while ((int64_t)256 << per_log2 < g.inner) ++per_log2;
    const int n_groups = (int)(g.n_outer << per_log2);   // a power of two, at most SM_GROUPS (softmax_one_pass)
    const int grid = grid_for(g.n_out * 64);
    hipStream_t st = (hipStream_t)stream;
    if (norm.out_dtype == D_BF16) launch_softmax_t<bf16_t>(g, n_groups, grid, per_log2, s, lse_out, out, st);
    else launch_softmax_t<float>(g, n_groups, grid, per_log2, s, lse_out, out, st);
    return (int)hipGetLastError();
}

static bool is_float_dtype(int dt) { return dt == D_F32 || dt == D_BF16; }

bool elemwise_chainable(const tra_plan_s &a, const tra_plan_s &b)
{
    if (a.kernel != TRA_KERNEL_ELEMWISE || b.kernel != TRA_KERNEL_ELEMWISE) return false;
    if (b.n_ops != 2 || a.info.z_elems != b.info.z_elems) return false;
    if (!is_float_dtype(a.in_dtype) || !is_float_dtype(a.out_dtype) || b.in_dtype != a.out_dtype ||
        !is_float_dtype(b.out_dtype))
        return false;
    // t is plan a's output and plan b's second operand: both must be the
    // output relation of plan b (same labels in the same order, same d)
    if (a.zl != b.zl || b.yl != b.zl) return false;
    for (char c : b.zl)
        if (a.d[(int)c] != b.d[(int)c] || a.B[(int)c] != b.B[(int)c]) return false;
    return true;
}

template <typename TIA, typename TM, typename TO>
static int launch_chain_t(const tra_plan_s &a, const tra_plan_s &b, const void *xa, const void *ya, const void *xb,
                          void *z, hipStream_t s)
{
    if (!a.el.p2 || !b.el.p2 || !b.el.y_step) {
        hipLaunchKernelGGL((k_elemwise_chain<TIA, TM, TO>), dim3(grid_for(a.el.n_out)), dim3(256), 0, s, a.el,
                           a.join, a.n_ops == 2 ? 1 : 0, b.el, b.join, (const TIA *)xa, (const TIA *)ya,
                           (const TM *)xb, (TO *)z);
        return (int)hipGetLastError();
    }
    const int64_t n_vec = a.el.n_out / 4;
    const int64_t bytes = a.info.x_bytes + (a.el.y_step ? a.info.y_bytes : 0) + b.info.x_bytes + b.info.z_bytes;
    const bool big = bytes >= (64ll << 20), wide = n_vec >= 256 * 256 * 4;
    const int upt = big || wide ? 4 : 1;
    const unsigned grid = (unsigned)((n_vec + 256 * upt - 1) / (256 * upt));
#define TRA_CH_GO(UPT, NT)                                                                                  \
    hipLaunchKernelGGL((k_elemwise_chain_p2<TIA, TM, TO, UPT, NT>), dim3(grid), dim3(256), 0, s, a.el, a.join, \
                       a.n_ops == 2 ? 1 : 0, b.el, b.join, (const TIA *)xa, (const TIA *)ya, (const TM *)xb,  \
                       (TO *)z)
    if (big) TRA_CH_GO(4, true);
    else if (wide) TRA_CH_GO(4, false);
    else TRA_CH_GO(1, false);
#undef TRA_CH_GO
    return (int)hipGetLastError();
}

int launch_elemwise_chain(const tra_plan_s &a, const tra_plan_s &b, const void *xa, const void *ya, const void *xb,
                          void *z, void *stream)
{
    if (a.el.n_out == 0) return 0;
    hipStream_t s = (hipStream_t)stream;
    const bool ia = a.in_dtype == D_BF16, im = a.out_dtype == D_BF16, ob = b.out_dtype == D_BF16;
    if (!ia && !im && !ob) return launch_chain_t<float, float, float>(a, b, xa, ya, xb, z, s);
    if (!ia && !im && ob) return launch_chain_t<float, float, bf16_t>(a, b, xa, ya, xb, z, s);
    if (!ia && im && !ob) return launch_chain_t<float, bf16_t, float>(a, b, xa, ya, xb, z, s);
    if (!ia && im && ob) return launch_chain_t<float, bf16_t, bf16_t>(a, b, xa, ya, xb, z, s);
    if (ia && !im && !ob) return launch_chain_t<bf16_t, float, float>(a, b, xa, ya, xb, z, s);
    if (ia && !im && ob) return launch_chain_t<bf16_t, float, bf16_t>(a, b, xa, ya, xb, z, s);
    if (ia && im && !ob) return launch_chain_t<bf16_t, bf16_t, float>(a, b, xa, ya, xb, z, s);
    return launch_chain_t<bf16_t, bf16_t, bf16_t>(a, b, xa, ya, xb, z, s);
}

int launch_rowreduce(const tra_plan_s &p, const void *x, const void *y, void *z, void *ws, void *stream)
{
    hipStream_t s = (hipStream_t)stream;
    if (p.gen.split > 0) return launch_reduce_split(p, x, y, z, ws, s);
    if (p.row.p2) {
        int grid = grid_for(p.row.n_out * 64);
        TRA_DISPATCH_IO(p.in_dtype, p.out_dtype,
                        hipLaunchKernelGGL((k_rowreduce_p2<TI, TO>), dim3(grid), dim3(256), 0, s, p.row, p.join,
                                           p.agg, p.n_ops == 2 ? 1 : 0, (const TI *)x, (const TI *)y, (TO *)z));
        return (int)hipGetLastError();
    }
    int grid = grid_for(p.row.n_out * 64);
    TRA_DISPATCH_IO(p.in_dtype, p.out_dtype,
                    hipLaunchKernelGGL((k_rowreduce<TI, TO>), dim3(grid), dim3(256), 0, s, p.row, p.join, p.agg,
                                       p.n_ops == 2 ? 1 : 0, (const TI *)x, (const TI *)y, (TO *)z));
    return (int)hipGetLastError();
}

static int launch_fold(int64_t n, int split, int agg, float scale, bool int_acc, int out_dtype, const void *ws,
                       void *z, hipStream_t s)
{
    int grid = grid_for(n);
    if (int_acc) {
        hipLaunchKernelGGL((k_split_fold<int32_t, int32_t>), dim3(grid), dim3(256), 0, s, (const int32_t *)ws, n,
                           split, agg, 1.0f, (int32_t *)z);
    } else if (out_dtype == D_BF16) {
        hipLaunchKernelGGL((k_split_fold<float, bf16_t>), dim3(grid), dim3(256), 0, s, (const float *)ws, n, split,
                           agg, scale, (bf16_t *)z);
    } else {
        hipLaunchKernelGGL((k_split_fold<float, float>), dim3(grid), dim3(256), 0, s, (const float *)ws, n, split,
                           agg, scale, (float *)z);
    }
    return (int)hipGetLastError();
}

int launch_split_fold(const tra_plan_s &p, const void *ws, void *z, void *stream)
{
    return launch_fold(p.info.z_elems, p.gv.split, p.agg, p.post_scale, p.in_dtype == D_I32, p.out_dtype, ws, z,
                       (hipStream_t)stream);
}

int launch_repartition(const RepartDesc &r, int esz, const void *src, void *dst, void *stream)
{
    hipStream_t s = (hipStream_t)stream;
    const int unit = r.vec * esz;
    const int64_t n_units = r.n_elems / r.vec;
    // power-of-two digits (at most kP2Max of them): shift/mask path.  The
    // element index and the source offset are 32-bit there.
    bool p2 = r.n_elems < (1ll << 31) && r.dst.n <= kP2Max;
    Pow2Group g{};
    g.n = r.dst.n;
    uint32_t sh = 0;
    for (int i = r.dst.n - 1; i >= 0 && p2; --i) {
        uint32_t e = r.dst.ext[i];
        if (e & (e - 1)) p2 = false;
        g.sh[i] = sh;
        g.mask[i] = e - 1;
        g.st[0][i] = (int32_t)r.dst.st[0][i];
        while ((1u << sh) < e * (1u << g.sh[i])) ++sh;
    }
    if (p2) {
        int lvec = 0;
        while ((1 << lvec) < r.vec) ++lvec;
        const bool sc = r.scatter != 0;
        switch (unit) {
        case 16: sc ? launch_rep_p2<u32x4, true>(g, lvec, n_units, src, dst, s)
                    : launch_rep_p2<u32x4, false>(g, lvec, n_units, src, dst, s); break;
        case 8: sc ? launch_rep_p2<u32x2, true>(g, lvec, n_units, src, dst, s)
                   : launch_rep_p2<u32x2, false>(g, lvec, n_units, src, dst, s); break;
        case 4: sc ? launch_rep_p2<uint32_t, true>(g, lvec, n_units, src, dst, s)
                   : launch_rep_p2<uint32_t, false>(g, lvec, n_units, src, dst, s); break;
        default: sc ? launch_rep_p2<uint16_t, true>(g, lvec, n_units, src, dst, s)
                    : launch_rep_p2<uint16_t, false>(g, lvec, n_units, src, dst, s); break;
        }
        return (int)hipGetLastError();
    }
    int grid = grid_for(n_units);
#define TRA_REP(U) hipLaunchKernelGGL((k_repartition<U>), dim3(grid), dim3(256), 0, s, r, r.vec, (const U *)src, (U *)dst)
    switch (unit) {
    case 16: TRA_REP(uint4); break;
    case 8: TRA_REP(uint2); break;
    case 4: TRA_REP(uint32_t); break;
    default: TRA_REP(uint16_t); break;
    }
#undef TRA_REP
    return (int)hipGetLastError();
}

const char *hip_error_text(int err) { return hipGetErrorString((hipError_t)err); }

}  // namespace tra
