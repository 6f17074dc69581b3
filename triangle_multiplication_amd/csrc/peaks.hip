// peaks.hip -- measured ceilings for the roofline figures of the benchmark.
//
// The spec peaks (2.5 PFLOP/s dense bf16, 8 TB/s HBM) assume the 2.4 GHz
// clock and an ideal memory system.  These kernels measure what the chip
// delivers to the simplest possible code on the same box:
//  - peak_mfma_bf16<SHAPE>: every wave issues nothing but independent bf16
//    MFMAs on operands held in registers (two waves per SIMD as in the
//    contraction), on random bf16 data, so the matrix cores toggle like they
//    do on real operands: 16 accumulator tiles of v_mfma_f32_16x16x32_bf16
//    (SHAPE 0, the instruction the kernels use) or 4 tiles of
//    v_mfma_f32_32x32x16_bf16 (SHAPE 1, measured about 3 % faster), the same
//    registers and FLOPs per iteration;
//  - peak_stream<R, W, NT>: one 16-byte chunk per thread over a grid that
//    covers the arrays, R source arrays read and W destination arrays written
//    per chunk (copy: 1/1; the output stage's mix: 2/1; the projection's
//    mix: 1/2), with plain or non-temporal loads and stores.  This form
//    measured fastest on gfx950: the workgroups in flight then always cover
//    one contiguous window of each array, while a grid-stride loop over a
//    CU-sized grid (workgroups drifting apart in memory) streamed a copy at
//    4.4-5.2 TB/s against 6.2-6.5.
// Neither is part of the forward pass.
#include "trimul_device.hpp"
#include "trimul_launch.hpp"

namespace trimul {

constexpr int PEAK_THREADS = 256;

typedef float f32x16 __attribute__((ext_vector_type(16)));

template <int SHAPE>
__global__ __launch_bounds__(PEAK_THREADS) void peak_mfma_bf16(const u32x4* __restrict__ seed, int iters,
                                                               float* __restrict__ sink)
{
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    u32x4 a[4], b[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        a[i] = seed[(lane + 64 * i + 16 * wave) & 255];
        b[i] = seed[(lane + 64 * i + 128 + 16 * wave) & 255];
    }
    float s = 0.f;
    if constexpr (SHAPE == 0) {
        f32x4 acc[16];
#pragma unroll
        for (int t = 0; t < 16; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
        for (int it = 0; it < iters; ++it) {
#pragma unroll
            for (int m = 0; m < 4; ++m)
#pragma unroll
                for (int n = 0; n < 4; ++n) acc[4 * m + n] = Elem<bf16>::mma(a[m], b[n], acc[4 * m + n]);
        }
#pragma unroll
        for (int t = 0; t < 16; ++t) s += acc[t][0] + acc[t][1] + acc[t][2] + acc[t][3];
    } else {
        f32x16 acc[4];
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[t][e] = 0.f;
        for (int it = 0; it < iters; ++it) {
#pragma unroll
            for (int m = 0; m < 2; ++m)
#pragma unroll
                for (int n = 0; n < 2; ++n) {
                    acc[2 * m + n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                        __builtin_bit_cast(bf16x8, a[m]), __builtin_bit_cast(bf16x8, b[n]), acc[2 * m + n], 0, 0, 0);
                    acc[2 * m + n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                        __builtin_bit_cast(bf16x8, a[m + 2]), __builtin_bit_cast(bf16x8, b[n + 2]), acc[2 * m + n], 0, 0, 0);
                }
        }
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int e = 0; e < 16; ++e) s += acc[t][e];
    }
    sink[(size_t)blockIdx.x * PEAK_THREADS + threadIdx.x] = s;
}

template <int R, int W, bool NT>
__global__ __launch_bounds__(PEAK_THREADS) void peak_stream(const u32x4* __restrict__ s0,
                                                            const u32x4* __restrict__ s1,
                                                            u32x4* __restrict__ d0, u32x4* __restrict__ d1,
                                                            size_t n16)
{
    const size_t i = (size_t)blockIdx.x * PEAK_THREADS + threadIdx.x;
    if (i >= n16) return;
    u32x4 v = NT ? __builtin_nontemporal_load(s0 + i) : s0[i];
    if (R == 2) v ^= NT ? __builtin_nontemporal_load(s1 + i) : s1[i];
    if (NT) {
        __builtin_nontemporal_store(v, d0 + i);
        if (W == 2) __builtin_nontemporal_store(v, d1 + i);
    } else {
        d0[i] = v;
        if (W == 2) d1[i] = v;
    }
}

hipError_t launch_peak_mfma(const void* seed, int blocks, int iters, int shape, float* sink, hipStream_t s)
{
    if (shape == 0)
        hipLaunchKernelGGL((peak_mfma_bf16<0>), dim3((unsigned)blocks), dim3(PEAK_THREADS), 0, s,
                           (const u32x4*)seed, iters, sink);
    else if (shape == 1)
        hipLaunchKernelGGL((peak_mfma_bf16<1>), dim3((unsigned)blocks), dim3(PEAK_THREADS), 0, s,
                           (const u32x4*)seed, iters, sink);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

template <bool NT>
static hipError_t launch_stream_nt(const void* s0, const void* s1, void* d0, void* d1, size_t n16, int reads,
                                   int writes, hipStream_t s)
{
    const dim3 grid((unsigned)((n16 + PEAK_THREADS - 1) / PEAK_THREADS));
    const u32x4* a = (const u32x4*)s0;
    const u32x4* b = (const u32x4*)s1;
    u32x4* c = (u32x4*)d0;
    u32x4* d = (u32x4*)d1;
    if (reads == 1 && writes == 1) hipLaunchKernelGGL((peak_stream<1, 1, NT>), grid, dim3(PEAK_THREADS), 0, s, a, b, c, d, n16);
    else if (reads == 2 && writes == 1) hipLaunchKernelGGL((peak_stream<2, 1, NT>), grid, dim3(PEAK_THREADS), 0, s, a, b, c, d, n16);
    else if (reads == 1 && writes == 2) hipLaunchKernelGGL((peak_stream<1, 2, NT>), grid, dim3(PEAK_THREADS), 0, s, a, b, c, d, n16);
    else return hipErrorInvalidValue;
    return hipGetLastError();
}

hipError_t launch_peak_stream(const void* s0, const void* s1, void* d0, void* d1, size_t n16, int reads,
                              int writes, int nontemporal, hipStream_t s)
{
    return nontemporal ? launch_stream_nt<true>(s0, s1, d0, d1, n16, reads, writes, s)
                       : launch_stream_nt<false>(s0, s1, d0, d1, n16, reads, writes, s);
}

}  // namespace trimul
