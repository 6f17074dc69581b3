/*
 * trimul_internal.h -- stage entry points of libtrimul, for stage-level tests.
 *
 * Each launches exactly the kernel trimul_fwd launches for that stage (same
 * code, same tiling); they are not a second implementation.  Layouts are the
 * ones trimul_fwd uses inside its workspace.  Same conventions as trimul.h:
 * caller-owned device pointers, asynchronous on `stream`, all arguments
 * checked before anything is enqueued.
 */
#ifndef TRIMUL_INTERNAL_H
#define TRIMUL_INTERNAL_H

#include "trimul.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * LayerNorm_in, gated input projection and mask (the first three lines of the
 * formula in trimul.h), stored channel-major for the contraction:
 *   outgoing: A[b][c](i, k) = a_(b,i,k,c),  B[b][c](j, k) = b_(b,j,k,c)
 *   incoming: A[b][c](i, k) = a_(b,k,i,c),  B[b][c](j, k) = b_(b,k,j,c)
 * so that the contraction is always o[b][c][i][j] = sum_k A(i, k) B(j, k).
 * Storage of one (b, c) slab of A or B (a_cm, b_cm are [B][C][slab]):
 *   fp32 handles: plain, element (r, k) at r * N + k (slab N * N);
 *   bf16 handles: K-blocked, element (r, k) at ((k / 32) * N + r) * 32 + k % 32
 *                 (slab N * Kp, Kp = N rounded up to 32; entries with k >= N
 *                 are padding, never written or read).
 * a_cm, b_cm: 16-byte aligned.
 */
trimul_status trimul_internal_project(trimul_handle *h, const void *z, const void *pair_mask,
                                      int B, int N, trimul_direction dir, void *a_cm, void *b_cm,
                                      hipStream_t stream);

/*
 * Triangle contraction, C*B independent N x N x N products with fp32
 * accumulation: o[b][c][i][j] = sum_k A[b][c](i, k) * B[b][c](j, k), rounded
 * once to the dtype.  a_cm, b_cm in the storage described above; o: plain
 * [B][C][N][N].
 */
trimul_status trimul_internal_contract(trimul_handle *h, const void *a_cm, const void *b_cm,
                                       int B, int N, void *o, hipStream_t stream);

/*
 * Output stage: out[b][i][j][:] = (p_out LayerNorm_out(o[b][:][i][j]))
 *                                 * sg(g_out LayerNorm_in(z[b][i][j][:])).
 * o: [B][C][N][N] channel-major; z, out: [B][N][N][D].
 */
trimul_status trimul_internal_output(trimul_handle *h, const void *z, const void *o, int B,
                                     int N, void *out, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* TRIMUL_INTERNAL_H */
