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
    // The projection with ln_in_w folded in, rows in w_proj's order with the
    // gate rows scaled by -log2(e), and per row the fp32 vector (T, T, T, T) of
    // its (equally scaled) dot product with ln_in_b: [4C][4] floats.
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

// Kernel variants chosen per shape (by trimul_tune, or the defaults below).
// None changes what is computed; each only changes the order of the work.
struct Plan {
    // Contraction (bf16): which XCD receives which tiles.
    //  0: the launch's tiles are cut into 8 contiguous bands, one per XCD.
    //  1: every round of G tiles (one per workgroup) is cut into 8 contiguous
    //     blocks, so all XCDs work on the same channels at the same time and
    //     their panel re-reads beyond L2 hit the shared last-level cache.
    int k2_order = 0;
    // Row panels per group when a channel's tiles are walked (4, 8 or 16).
    int k2_gm = 8;
    // Projection variant.  One kernel today (two 4-wave workgroups per CU,
    // one per 256 pairs); the field keeps the plan format stable for more.
    int k1_variant = 0;
    // Contraction tile side: 256 (32 keys per step) or 128 (64 keys per step,
    // a quarter of the outputs per tile; less work lost on ragged edges).
    int k2_tile = 256;
};

// Tile height of the bf16 contraction; the mask-range table has one entry per
// row tile of this many rows.
constexpr int K2_TILE = 256;
constexpr int K2_KSTEP = 32;

// Table of a masked contraction (int32 units, T = ceil(N / K2_TILE) row tiles):
//   [0, 2BT)              ranges[b][t] = (lo, hi): K-steps (32 keys) outside
//                         which every row of row tile t of A and B is zero;
//   [2BT, 2BT + 4)        header; [0] = most live tile pairs of any batch;
//   [2BT + 4, + B T^2)    pairs[b][q] = ti | tj << 16: batch b's T^2 tile pairs,
//                         those with a live step first, each part in the
//                         plan's walk order.
inline size_t mask_table_ints(int B, int N)
{
    const size_t T = (size_t)((N + K2_TILE - 1) / K2_TILE);
    return 2 * (size_t)B * T + 4 + (size_t)B * T * T;
}

// One launch of the contraction: operand slabs [bc0, bc0 + nbc) of the B*C
// slabs (bc = b * C + c), output of slab bc0 + t at o + t * o_stride elements.
// table: null, or a mask table whose ranges and pairs are filled (bf16 only).
struct ContractJob {
    int bc0, nbc;
    void* o;
    size_t o_stride;
    const int* table;
};

// Where the output stage reads o: slab bc at o_lo + bc * N * N for bc < split,
// else at o_hi + (bc - split) * hi_stride elements.
struct OutputSrc {
    const void* o_lo;
    const void* o_hi;
    int split;
    size_t hi_stride;
};

hipError_t launch_project(const Params& p, const Plan& plan, const void* z, const void* mask, int B, int N,
                          int incoming, void* a_cm, void* b_cm, hipStream_t s);
// Scan the pair mask for each row tile's live key range (the ranges of the
// mask table; also clears its header).  incoming: rows of A and B are columns
// of the mask.
hipError_t launch_mask_ranges(const Params& p, const void* mask, int B, int N, int incoming,
                              int* table, hipStream_t s);
// Order each batch's tile pairs live-first in the walk of plan.k2_gm (the
// pairs and header of the mask table; its ranges must be filled).  Nothing
// to do for 128-row tiles, which do not read the lists.
hipError_t launch_tile_pairs(const Plan& plan, int* table, int B, int N, hipStream_t s);
hipError_t launch_contract(const Params& p, const Plan& plan, const void* a_cm, const void* b_cm,
                           int B, int N, const ContractJob& job, hipStream_t s);
hipError_t launch_output(const Params& p, const void* z, const OutputSrc& o, int B, int N,
                         void* out, hipStream_t s);

// Measured ceilings (not part of the forward pass): an MFMA-only loop and
// plain 16-byte streams with `reads` sources and `writes` destinations.
hipError_t launch_peak_mfma(const void* seed, int blocks, int iters, int shape, float* sink, hipStream_t s);
hipError_t launch_peak_stream(const void* s0, const void* s1, void* d0, void* d1, size_t n16, int reads,
                              int writes, int nontemporal, hipStream_t s);

// Host mirrors of the kernels' static launch geometry (used for validation).
bool project_supported(int D, int C, DType t);
bool output_supported(int D, int C, DType t);

}  // namespace trimul
