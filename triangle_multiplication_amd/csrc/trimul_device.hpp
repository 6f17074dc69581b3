// trimul_device.hpp -- gfx950 device helpers shared by the three TriMul kernels.
//
// Every kernel moves data in 16-byte chunks (one dwordx4 per lane) and feeds
// matrix cores with 16x16 output tiles:
//   bf16: one chunk = 8 elements; v_mfma_f32_16x16x32_bf16 consumes one chunk of
//         A and one of B per lane (a K-group of 32 = 4 lane groups x 8).
//   fp32: one chunk = 4 elements; four v_mfma_f32_16x16x4_f32 consume one chunk
//         of A and of B per lane (a K-group of 16 = 4 lane groups x 4).
// In both cases lane l supplies row (l % 16) of its 16-row operand block and
// the chunk (l / 16) of the K-group; A and B use the same K assignment, so the
// hardware's internal K order inside a group does not matter.  The 16x16 fp32
// result sits with lane l holding column (l % 16), rows 4 * (l / 16) + r,
// r = 0..3.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace trimul {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int WAVE = 64;

template <typename T> struct Elem;

template <> struct Elem<bf16> {
    static constexpr int CE = 8;  // elements per 16-byte chunk
    __device__ static inline f32x4 mma(u32x4 a, u32x4 b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                       __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
    }
    __device__ static inline void unpack(u32x4 v, float* f) {
        bf16x8 h = __builtin_bit_cast(bf16x8, v);
#pragma unroll
        for (int e = 0; e < 8; ++e) f[e] = (float)h[e];
    }
    __device__ static inline u32x4 pack(const float* f) {
        bf16x8 h;
#pragma unroll
        for (int e = 0; e < 8; ++e) h[e] = (bf16)f[e];
        return __builtin_bit_cast(u32x4, h);
    }
    __device__ static inline float load1(const void* p, size_t i) {
        return (float)reinterpret_cast<const bf16*>(p)[i];
    }
    // Store four consecutive elements (8 bytes).
    __device__ static inline void store4(void* p, size_t i, f32x4 v) {
        bf16x4 h;
        h[0] = (bf16)v[0]; h[1] = (bf16)v[1]; h[2] = (bf16)v[2]; h[3] = (bf16)v[3];
        *reinterpret_cast<bf16x4*>(reinterpret_cast<bf16*>(p) + i) = h;
    }
};

template <> struct Elem<float> {
    static constexpr int CE = 4;
    __device__ static inline f32x4 mma(u32x4 a, u32x4 b, f32x4 c) {
        f32x4 fa = __builtin_bit_cast(f32x4, a), fb = __builtin_bit_cast(f32x4, b);
        c = __builtin_amdgcn_mfma_f32_16x16x4f32(fa[0], fb[0], c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_16x16x4f32(fa[1], fb[1], c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_16x16x4f32(fa[2], fb[2], c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_16x16x4f32(fa[3], fb[3], c, 0, 0, 0);
        return c;
    }
    __device__ static inline void unpack(u32x4 v, float* f) {
        f32x4 h = __builtin_bit_cast(f32x4, v);
#pragma unroll
        for (int e = 0; e < 4; ++e) f[e] = h[e];
    }
    __device__ static inline u32x4 pack(const float* f) {
        f32x4 h = {f[0], f[1], f[2], f[3]};
        return __builtin_bit_cast(u32x4, h);
    }
    __device__ static inline float load1(const void* p, size_t i) {
        return reinterpret_cast<const float*>(p)[i];
    }
    __device__ static inline void store4(void* p, size_t i, f32x4 v) {
        *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(p) + i) = v;
    }
};

__device__ inline u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ inline void st16(void* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }

// Logistic sigmoid in fp32.
__device__ inline float sigmoidf_(float t) { return 1.0f / (1.0f + __expf(-t)); }

// Sum over the four lanes {l, l^16, l^32, l^48} that share one MFMA row.
__device__ inline float sum_row_lanes(float v) {
    v += __shfl_xor(v, 16);
    v += __shfl_xor(v, 32);
    return v;
}

// bf16 storage of the gated projections a and b is K-blocked: a slab of N
// rows is cut into blocks of 32 consecutive k, and a block holds all N rows
// of those 32 k (64 bytes per row), i.e. [ceil(N/32)][N][32].  A K-step of the
// contraction then reads one contiguous 64-byte run per row, and 16 rows in
// one contiguous kilobyte.  Element offset of (row, k); below 2^31 for every
// N the library accepts.
__device__ inline uint32_t kblk_off(uint32_t row, uint32_t k, uint32_t N)
{
    return ((k >> 5) * N + row) * 32u + (k & 31u);
}

// LDS swizzle for row-major tiles of 16-byte chunks: the low three bits of the
// chunk index are XORed with the row, so eight consecutive rows reading the same
// logical chunk hit eight distinct 128-byte bank groups.
__device__ inline int swz(int row, int chunk) { return chunk ^ (row & 7); }

// XOR mask for rows of n chunks: the largest of 7, 3, 1, 0 that keeps every
// swizzled index inside the row (n is a multiple of 4 for all widths used).
constexpr int swz_mask(int n) { return n % 8 == 0 ? 7 : n % 4 == 0 ? 3 : n % 2 == 0 ? 1 : 0; }

// Global -> LDS DMA of 16 bytes per lane: lane l's 16 bytes at gaddr land at
// LDS byte lds_addr + 16 l (lds_addr wave-uniform; it goes through M0).
// Issued as inline asm rather than through the builtin: after the builtin the
// compiler cannot tell which LDS reads a pending DMA may feed, and answers
// every later LDS read wait with a full lgkmcnt(0) (or, before a transposing
// read, vmcnt(0)).  Completion is the caller's business: each kernel waits
// on vmcnt explicitly before a barrier that publishes the slot.
__device__ inline void dma16_to_lds(const void* gaddr, uint32_t lds_addr)
{
    asm volatile("global_load_lds_dwordx4 %0, off" ::"v"(gaddr), "{m0}"(lds_addr) : "memory");
}

// The same with the non-temporal hint, for data a kernel reads exactly once
// (it is then not kept in L2 at the expense of data that is re-read).
__device__ inline void dma16_to_lds_nt(const void* gaddr, uint32_t lds_addr)
{
    asm volatile("global_load_lds_dwordx4 %0, off nt" ::"v"(gaddr), "{m0}"(lds_addr) : "memory");
}

// LDS byte address of a pointer into a __shared__ array.
__device__ inline uint32_t lds_addr_of(const void* p)
{
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// s_waitcnt immediate for "vmcnt <= n" leaving expcnt and lgkmcnt unconstrained
// (gfx9 encoding: vmcnt bits [3:0] and [15:14], expcnt [6:4], lgkmcnt [11:8]).
constexpr int waitcnt_vm(int n) { return (n & 15) | (((n >> 4) & 3) << 14) | (7 << 4) | (15 << 8); }
// ... and additionally "lgkmcnt == 0" (every LDS read of this wave has completed).
constexpr int waitcnt_vm_lds0(int n) { return (n & 15) | (((n >> 4) & 3) << 14) | (7 << 4); }

}  // namespace trimul
