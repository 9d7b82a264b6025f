// k_probe.hip -- the machine's own ceilings, measured beside the published
// ones: a loop of bf16 matrix-core products with nothing else in it (no
// memory traffic besides one store per lane at the end).  The copy ceiling is
// measured with tra_repartition between identical blockings.
#include <hip/hip_runtime.h>

#include "tra.h"

namespace tra {

typedef __bf16 bf16x8_p __attribute__((ext_vector_type(8)));
typedef float floatx16_p __attribute__((ext_vector_type(16)));
typedef float floatx4_p __attribute__((ext_vector_type(4)));

// Four waves per workgroup, one per SIMD; each wave runs `iters` rounds of 8
// independent 32x32x16 products (8 accumulator sets, so no product waits on
// the one before it), from operands that stay in registers.  DISTINCT: each
// of the 8 products has operands of its own, random bf16 values of the size
// of N(0, 0.02) inputs, different in every lane, so consecutive products
// switch operands as they do in a real product (the multipliers toggle, and
// the clock the chip holds under that load is lower); otherwise all 8 take
// one operand pair.
__device__ __forceinline__ uint32_t probe_hash(uint32_t x)
{
    // a 32-bit integer mixer (multiply / xor-shift rounds)
    x ^= x >> 16;
    x *= 0x7feb352du;
    x ^= x >> 15;
    x *= 0x846ca68bu;
    x ^= x >> 16;
    return x;
}

template <bool DISTINCT>
__global__ __launch_bounds__(256) void k_probe_mfma(int iters, float seed, float *__restrict__ out)
{
    const int lane = threadIdx.x & 63;
    constexpr int NP = DISTINCT ? 8 : 1;
    bf16x8_p a[NP], b[NP];
#pragma unroll
    for (int s = 0; s < NP; ++s)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            if constexpr (DISTINCT) {
                const uint32_t h = probe_hash((uint32_t)(((blockIdx.x * 256 + threadIdx.x) * 8 + s) * 8 + e));
                // two uniform values in [-0.05, 0.05) per hash
                a[s][e] = (__bf16)(((float)(h & 0xffffu) / 65536.f - 0.5f) * 0.1f);
                b[s][e] = (__bf16)(((float)(h >> 16) / 65536.f - 0.5f) * 0.1f);
            } else {
                a[s][e] = (__bf16)(seed * (float)(lane + e));
                b[s][e] = (__bf16)(seed * (float)(lane - e));
            }
        }
    floatx16_p acc[8];
#pragma unroll
    for (int s = 0; s < 8; ++s)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[s][e] = 0.f;
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int s = 0; s < 8; ++s)
            acc[s] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[s % NP], b[s % NP], acc[s], 0, 0, 0);
    }
    float r = 0.f;
#pragma unroll
    for (int s = 0; s < 8; ++s)
#pragma unroll
        for (int e = 0; e < 16; ++e) r += acc[s][e];
    out[blockIdx.x * blockDim.x + threadIdx.x] = r;
}

// The same with 16x16x32 products: each wave runs `iters` rounds of 64
// independent products (64 accumulators of four values, 256 accumulator
// registers per lane, as the 64-deep matrix-core tile holds), random operands
// as above.  The products are issued from asm with the accumulators bound to
// the accumulator registers (the compiler's own form moves 64 small
// accumulators around the register file); s_nop wait states separate the
// zeroing and the final reads from them.
__global__ __launch_bounds__(256) void k_probe_mfma16(int iters, float *__restrict__ out)
{
    bf16x8_p a[8], b[8];
#pragma unroll
    for (int s = 0; s < 8; ++s)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const uint32_t h = probe_hash((uint32_t)(((blockIdx.x * 256 + threadIdx.x) * 8 + s) * 8 + e));
            a[s][e] = (__bf16)(((float)(h & 0xffffu) / 65536.f - 0.5f) * 0.1f);
            b[s][e] = (__bf16)(((float)(h >> 16) / 65536.f - 0.5f) * 0.1f);
        }
    floatx4_p acc[64];
#pragma unroll
    for (int s = 0; s < 64; ++s)
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[s][e] = 0.f;
    auto bind = [&]() {
#pragma unroll
        for (int s = 0; s < 64; s += 8)
            asm volatile("" : "+a"(acc[s]), "+a"(acc[s + 1]), "+a"(acc[s + 2]), "+a"(acc[s + 3]), "+a"(acc[s + 4]),
                         "+a"(acc[s + 5]), "+a"(acc[s + 6]), "+a"(acc[s + 7]));
    };
    bind();
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7");
    bind();
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int s = 0; s < 64; ++s)
            asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(acc[s]) : "v"(a[s % 8]), "v"(b[(s / 8 + s) % 8]));
    }
    bind();
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7");
    bind();
    float r = 0.f;
#pragma unroll
    for (int s = 0; s < 64; ++s)
#pragma unroll
        for (int e = 0; e < 4; ++e) r += acc[s][e];
    out[blockIdx.x * blockDim.x + threadIdx.x] = r;
}

}  // namespace tra

extern "C" int tra_probe_mfma_loop(int workgroups, int iters, int distinct_operands, float *out, void *hip_stream)
{
    if (!out) return TRA_E_NULL;
    if (workgroups < 1 || iters < 1) return TRA_E_OP;
    if (distinct_operands == 2)
        hipLaunchKernelGGL(tra::k_probe_mfma16, dim3(workgroups), dim3(256), 0, (hipStream_t)hip_stream, iters, out);
    else if (distinct_operands)
        hipLaunchKernelGGL(tra::k_probe_mfma<true>, dim3(workgroups), dim3(256), 0, (hipStream_t)hip_stream, iters,
                           1.0f / 64, out);
    else
        hipLaunchKernelGGL(tra::k_probe_mfma<false>, dim3(workgroups), dim3(256), 0, (hipStream_t)hip_stream, iters,
                           1.0f / 64, out);
    return hipGetLastError() == hipSuccess ? TRA_OK : TRA_E_HIP;
}
