// device_common.h -- scalar helpers shared by the gfx950 kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tra_internal.h"

namespace tra {

// bfloat16 is stored as its raw 16 bits.
struct bf16_t {
    uint16_t bits;
};

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// float -> bfloat16, round to nearest, ties to even; NaN stays a quiet NaN
// (sign and top payload bits kept, quiet bit set).  gfx950 converts in one
// instruction (v_cvt_pk_bf16_f32, two values at a time); its result equals
// the integer form (u + 0x7fff + bit 16 of u) >> 16, and (u >> 16) | 0x40 for
// a NaN, on every 32-bit pattern.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }

template <typename T> struct Scalar;
template <> struct Scalar<float> {
    using acc = float;
    static __device__ __forceinline__ float load(const float *p, int64_t i) { return p[i]; }
    static __device__ __forceinline__ void store(float *p, int64_t i, float v) { p[i] = v; }
};
template <> struct Scalar<bf16_t> {
    using acc = float;
    static __device__ __forceinline__ float load(const bf16_t *p, int64_t i) { return bf16_to_f32(p[i].bits); }
    static __device__ __forceinline__ void store(bf16_t *p, int64_t i, float v) { p[i].bits = f32_to_bf16(v); }
};
template <> struct Scalar<int32_t> {
    using acc = int32_t;
    static __device__ __forceinline__ int32_t load(const int32_t *p, int64_t i) { return p[i]; }
    static __device__ __forceinline__ void store(int32_t *p, int64_t i, int32_t v) { p[i] = v; }
};

// Integer arithmetic wraps (two's complement), done in uint32.
__device__ __forceinline__ int32_t wadd(int32_t a, int32_t b) { return (int32_t)((uint32_t)a + (uint32_t)b); }
__device__ __forceinline__ int32_t wsub(int32_t a, int32_t b) { return (int32_t)((uint32_t)a - (uint32_t)b); }
__device__ __forceinline__ int32_t wmul(int32_t a, int32_t b) { return (int32_t)((uint32_t)a * (uint32_t)b); }

__device__ __forceinline__ float join_f(int j, float x, float y)
{
    switch (j) {
    case J_MUL: return x * y;
    case J_SQDIFF: { float t = x - y; return t * t; }
    case J_ADD: return x + y;
    case J_IDENT: return x;
    case J_SUB: return x - y;
    default: return __expf(x - y);
    }
}
__device__ __forceinline__ int32_t join_i(int j, int32_t x, int32_t y)
{
    switch (j) {
    case J_MUL: return wmul(x, y);
    case J_SQDIFF: { int32_t t = wsub(x, y); return wmul(t, t); }
    case J_ADD: return wadd(x, y);
    case J_SUB: return wsub(x, y);
    default: return x;
    }
}

// Running aggregate.  lse keeps (max m, sum s of exp(v - m)).
template <typename A> struct Fold;
template <> struct Fold<float> {
    float m, s;
    __device__ __forceinline__ void init(int agg)
    {
        s = 0.f;
        m = agg == A_MAX || agg == A_LSE ? -INFINITY : (agg == A_MIN ? INFINITY : 0.f);
    }
    __device__ __forceinline__ void add(int agg, float v)
    {
        switch (agg) {
        case A_SUM: m += v; break;
        case A_MAX: m = fmaxf(m, v); break;
        case A_MIN: m = fminf(m, v); break;
        case A_LSE:
            if (v > m) {
                s = s * __expf(m - v) + 1.f;
                m = v;
            } else if (v != -INFINITY) {
                s += __expf(v - m);
            }
            break;
        default: m = v; break;
        }
    }
    // combine with another partial of the same aggregate
    __device__ __forceinline__ void merge(int agg, float om, float os)
    {
        if (agg == A_LSE) {
            if (om == -INFINITY) return;
            if (m == -INFINITY) {
                m = om;
                s = os;
                return;
            }
            float nm = fmaxf(m, om);
            s = s * __expf(m - nm) + os * __expf(om - nm);
            m = nm;
        } else {
            add(agg, om);
        }
    }
    __device__ __forceinline__ float result(int agg, float scale) const
    {
        float r = agg == A_LSE ? (m == -INFINITY ? -INFINITY : m + __logf(s)) : m;
        return r * scale;
    }
};
template <> struct Fold<int32_t> {
    int32_t m;
    __device__ __forceinline__ void init(int agg) { m = agg == A_MAX ? INT32_MIN : (agg == A_MIN ? INT32_MAX : 0); }
    __device__ __forceinline__ void add(int agg, int32_t v)
    {
        switch (agg) {
        case A_SUM: m = wadd(m, v); break;
        case A_MAX: m = max(m, v); break;
        case A_MIN: m = min(m, v); break;
        default: m = v; break;
        }
    }
    __device__ __forceinline__ void merge(int agg, int32_t om, int32_t) { add(agg, om); }
    __device__ __forceinline__ int32_t result(int, float) const { return m; }
};

__device__ __forceinline__ float join_any(int j, float x, float y) { return join_f(j, x, y); }
__device__ __forceinline__ int32_t join_any(int j, int32_t x, int32_t y) { return join_i(j, x, y); }

// Decompose a flattened index over a Radix (last digit fastest); add strides.
__device__ __forceinline__ void radix_offsets(const Radix &r, int64_t idx, int64_t &o0, int64_t &o1)
{
    for (int i = r.n - 1; i >= 0; --i) {
        uint32_t e = r.ext[i];
        int64_t q = idx / e;
        int64_t d = idx - q * e;
        idx = q;
        o0 += d * r.st[0][i];
        o1 += d * r.st[1][i];
    }
}

// Offset of a flattened index within a power-of-two group, tensor t.
template <int T>
__device__ __forceinline__ int32_t p2off(const Pow2Group &g, uint32_t idx)
{
    int32_t o = 0;
#pragma unroll
    for (int i = 0; i < kP2Max; ++i) o += (int32_t)((idx >> g.sh[i]) & g.mask[i]) * g.st[T][i];
    return o;
}

}  // namespace tra
