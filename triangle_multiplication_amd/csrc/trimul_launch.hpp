// trimul_launch.hpp -- host-side launchers of the three TriMul kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

namespace trimul {

enum class DType { BF16 = 0, FP32 = 1 };

// Device-resident packed parameters (owned by the handle).
struct Params {
    int D, C;
    DType dtype;
    float eps;
    // [4C][D]: for a then b, per 16-channel group g: 16 rows of p_in then the
    // same 16 channels' rows of g_in.  The projection kernel's 64-row weight
    // stage therefore holds (p, g) for 32 channels of one of a or b.
    const void* w_proj;
    const void* w_gout;    // [D][D]  g_out, rows = output channel
    const void* w_pout;    // [D][C]  p_out, rows = output channel
    const float* ln_in_w;  // [D]
    const float* ln_in_b;  // [D]
    const float* ln_out_w; // [C]
    const float* ln_out_b; // [C]
    // bf16 handles only (null otherwise): the output GEMMs with the LayerNorm
    // scales folded in, for kernels that apply LayerNorm algebraically.
    const void* w_gout_f;  // [D][D]  g_out[d][k] * ln_in_w[k]
    const void* w_pout_f;  // [D][C]  p_out[d][c] * ln_out_w[c]
    // [D][8] per output row: S_h, S_l, S_h, T_h, T_l, T_h, 0, 0, where S is the
    // sum of the folded bf16 row, T the dot product of the unfolded row with the
    // LayerNorm bias, each split into a bf16 high part and a bf16 remainder.
    const void* x_gout;
    const void* x_pout;
    // The projection with ln_in_w folded in, rows in w_proj's order, and its
    // [4C][8] correction rows (same form as x_gout).
    const void* w_proj_f;
    const void* x_proj;
    // 4 KB of device memory that kernels with a fixed number of stores per
    // step write their out-of-range lanes to; never read.
    void* sink;
};

// Elements of one (batch, channel) slab of a and b in the workspace.  bf16:
// K-blocked [Kp/32][N][32] with Kp = N rounded up to a multiple of 32 (k >= N
// is padding that no kernel reads); fp32: plain row-major [N][N].
__host__ __device__ inline size_t ab_slab_elems(DType t, int N)
{
    const size_t n = (size_t)N;
    return t == DType::BF16 ? n * ((n + 31) & ~(size_t)31) : n * n;
}

hipError_t launch_project(const Params& p, const void* z, const void* mask, int B, int N,
                          int incoming, void* a_cm, void* b_cm, hipStream_t s);
hipError_t launch_contract(const Params& p, const void* a_cm, const void* b_cm, int B, int N,
                           void* o, hipStream_t s);
hipError_t launch_output(const Params& p, const void* z, const void* o, int B, int N, void* out,
                         hipStream_t s);

// Host mirrors of the kernels' static launch geometry (used for validation).
bool project_supported(int D, int C, DType t);
bool output_supported(int D, int C, DType t);

}  // namespace trimul
