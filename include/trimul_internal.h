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
 * The mask table of a masked bf16 contraction: int32 [mask_table_ints] with
 * T = ceil(N/256) row tiles, mask_table_ints = 2 B T + 4 + B T^2:
 *   [0, 2BT)          ranges[b][t] = (lo, hi) in steps of 32 keys such that for
 *                     every row r of tile t and every key k outside
 *                     [32 lo, 32 hi), M[r][k] == 0, with M[r][k] = mask[b][r][k]
 *                     (outgoing) or mask[b][k][r] (incoming); lo is the first
 *                     live key's step, hi one past the last one's; (0, 0) when
 *                     no key is live;
 *   [2BT, 2BT + 4)    header ([0]: live tile pairs of the fullest batch);
 *   [2BT + 4, ...)    per batch, its T^2 tile pairs (ti | tj << 16), pairs with
 *                     a live key step first.
 * mask_ranges fills the ranges and clears the header (the scan trimul_fwd runs
 * before a masked bf16 contraction); pair_mask and table 16-byte aligned.
 */
trimul_status trimul_internal_mask_ranges(trimul_handle *h, const void *pair_mask, int B, int N,
                                          trimul_direction dir, int *table, hipStream_t stream);

/*
 * Triangle contraction, C*B independent N x N x N products with fp32
 * accumulation: o[b][c][i][j] = sum_k A[b][c](i, k) * B[b][c](j, k), rounded
 * once to the dtype.  a_cm, b_cm in the storage described above; o: plain
 * [B][C][N][N].  table: NULL, or a mask table whose ranges were filled by
 * trimul_internal_mask_ranges (bf16 only): the pair lists are built, then the
 * kernel runs only the key steps inside both row tiles' ranges, which must
 * hold every key where A or B can be nonzero.  dir selects only which of the
 * handle's plans is used, (B, N, dir, masked = table != NULL).
 */
trimul_status trimul_internal_contract(trimul_handle *h, const void *a_cm, const void *b_cm,
                                       int *table, int B, int N, trimul_direction dir, void *o,
                                       hipStream_t stream);

/*
 * Output stage: out[b][i][j][:] = (p_out LayerNorm_out(o[b][:][i][j]))
 *                                 * sg(g_out LayerNorm_in(z[b][i][j][:])).
 * o: [B][C][N][N] channel-major; z, out: [B][N][N][D].
 */
trimul_status trimul_internal_output(trimul_handle *h, const void *z, const void *o, int B,
                                     int N, void *out, hipStream_t stream);

/*
 * Plans (see trimul_tune): the projection variant (only 0 today), the
 * contraction's XCD tile order (0, 1), row-panel group (4, 8, 16) and tile
 * side (256, 128).  set_plan records a plan for a call shape in the
 * handle (as trimul_tune does, without timing or writing the cache), so tests
 * can run every candidate; get_plan returns the plan trimul_fwd would use.
 * plan_candidates writes up to cap candidates and returns how many exist.
 */
trimul_status trimul_internal_set_plan(trimul_handle *h, int B, int N, trimul_direction dir,
                                       int masked, int k1_variant, int k2_order, int k2_gm,
                                       int k2_tile);
trimul_status trimul_internal_get_plan(trimul_handle *h, int B, int N, trimul_direction dir,
                                       int masked, int *k1_variant, int *k2_order, int *k2_gm,
                                       int *k2_tile);
int trimul_internal_plan_candidates(int *k1_variant, int *k2_order, int *k2_gm, int *k2_tile,
                                    int cap);

/*
 * The plan cache file, host only (no device needed): store one entry
 * (replacing the entry with the same key), look one up (returns 1 and fills
 * the plan if found, 0 if not, -1 if the file cannot be read), and the path
 * the library uses (written to buf, length returned; 0 when disabled).
 */
trimul_status trimul_internal_cache_store(const char *path, const char *device, int D, int C,
                                          int dtype, int B, int N, int dir, int masked,
                                          int k1_variant, int k2_order, int k2_gm, int k2_tile,
                                          double ms);
int trimul_internal_cache_lookup(const char *path, const char *device, int D, int C, int dtype,
                                 int B, int N, int dir, int masked, int *k1_variant, int *k2_order,
                                 int *k2_gm, int *k2_tile);
int trimul_internal_cache_path(char *buf, int cap);

/*
 * Measured ceilings for roofline figures (not part of the forward pass; the
 * benchmark reports each kernel against these as well as against the spec
 * peaks).  Both enqueue one kernel on `stream` and return at once.
 *
 * trimul_internal_peak_mfma: `blocks` workgroups of 256 threads (four waves);
 * every wave loads bf16 operands once from `seed` (4096 bytes: 256 chunks of
 * 16 bytes, 16-byte aligned) and then issues, per iteration, 16 independent
 * 16x16x32 bf16 MFMAs (shape 0) or 8 32x32x16 bf16 MFMAs on 4 accumulator
 * tiles (shape 1), 262144 FLOP either way: 4 * 262144 * iters * blocks FLOP
 * in all.  Thread t of workgroup g writes one float (a sum of its
 * accumulators) to sink[g * 256 + t].  blocks in [1, 2^20], iters in
 * [1, 2^24], shape 0 or 1.
 *
 * trimul_internal_peak_stream: over n16 chunks of 16 bytes
 * (1 <= n16 <= 2^38), one per thread, v = src0[i] (reads = 1) or
 * src0[i] ^ src1[i] (reads = 2), then dst0[i] = v and, with writes = 2,
 * dst1[i] = v: (reads + writes) * 16 * n16 bytes moved; nontemporal != 0
 * marks every load and store non-temporal.
 * Pointers the mode uses must be non-NULL and 16-byte aligned (unused ones
 * may be NULL); (reads, writes) must be (1, 1), (2, 1) or (1, 2).
 * Overlapping buffers give unspecified values but no access outside them.
 */
trimul_status trimul_internal_peak_mfma(const void *seed, int blocks, int iters, int shape, float *sink,
                                        hipStream_t stream);
trimul_status trimul_internal_peak_stream(const void *src0, const void *src1, void *dst0, void *dst1,
                                          size_t n16, int reads, int writes, int nontemporal,
                                          hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* TRIMUL_INTERNAL_H */
