/*
 * trimul.h -- C ABI of libtrimul: the forward triangle multiplicative update
 * (TriMul) on one AMD Instinct MI355X (gfx950).
 *
 * The layer is the one in the "Use" section of the fold-cp-ops README: a
 * module with six submodules, norm_in and norm_out (LayerNorm), p_in and g_in
 * (Linear(D, 2D), no bias), p_out and g_out (Linear(D, D), no bias), a
 * direction ("outgoing" shown there; "incoming" is its transposed twin), an
 * optional pair mask of shape (B, N, N) in the input's dtype, inference only.
 * The README gives names and shapes, not the formula; libtrimul computes, for
 * every batch b and pair (i, j), with sg(t) = 1 / (1 + exp(-t)):
 *
 *   x_ij   = LayerNorm_in(z_ij)                 (over D, biased variance)
 *   a_ijc  = m_ij * (p_in x_ij)_c     * sg((g_in x_ij)_c)          c in [0, C)
 *   b_ijc  = m_ij * (p_in x_ij)_(C+c) * sg((g_in x_ij)_(C+c))
 *   o_ijc  = sum_k a_ikc b_jkc   (outgoing)     sum_k a_kic b_kjc   (incoming)
 *   out_ij = (p_out LayerNorm_out(o_ij)) * sg(g_out x_ij)
 *
 * generalised to a hidden width C (the README's layer has C = D).
 *
 * Conventions for every entry point:
 *  - Tensors are dense and row-major.  Device pointers are caller-owned and
 *    must stay valid until the work enqueued on the stream has finished.
 *  - Element type is the handle's dtype: TRIMUL_BF16 (bf16 storage, fp32
 *    LayerNorm statistics and fp32 MFMA accumulation) or TRIMUL_FP32.
 *  - Errors are returned as trimul_status; trimul_last_error() (thread-local)
 *    names the failing argument and the value found.  All arguments are
 *    checked before anything is enqueued, so an error leaves no partial work.
 *    No C++ exception crosses this ABI.
 */
#ifndef TRIMUL_H
#define TRIMUL_H

#include <stddef.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    TRIMUL_OK = 0,
    TRIMUL_ERR_INVALID_ARG = 1,  /* null/misaligned/aliasing pointer, bad size or enum */
    TRIMUL_ERR_UNSUPPORTED = 2,  /* valid request outside what the kernels implement */
    TRIMUL_ERR_ARCH = 3,         /* device is not gfx950 */
    TRIMUL_ERR_WORKSPACE = 4,    /* workspace missing or smaller than required */
    TRIMUL_ERR_HIP = 5           /* a HIP runtime call failed (message has the HIP error) */
} trimul_status;

typedef enum { TRIMUL_BF16 = 0, TRIMUL_FP32 = 1 } trimul_dtype;

/* The README's direction argument: outgoing o_ij = sum_k a_ik b_jk,
 * incoming o_ij = sum_k a_ki b_kj. */
typedef enum { TRIMUL_OUTGOING = 0, TRIMUL_INCOMING = 1 } trimul_direction;

/* Host fp32 parameters of one layer, mirroring the README's six submodules
 * (Linear weights stored [out][in]).  Read only during trimul_create. */
typedef struct {
    const float *norm_in_weight;   /* [D]                                        */
    const float *norm_in_bias;     /* [D]                                        */
    const float *p_in;             /* [2C][D]: rows [0,C) give a, [C,2C) give b   */
    const float *g_in;             /* [2C][D]: rows [0,C) gate a, [C,2C) gate b   */
    const float *norm_out_weight;  /* [C]                                        */
    const float *norm_out_bias;    /* [C]                                        */
    const float *p_out;            /* [D][C]                                     */
    const float *g_out;            /* [D][D]                                     */
    float eps;                     /* LayerNorm epsilon (nn.LayerNorm default 1e-5) */
} trimul_weights;

typedef struct trimul_handle trimul_handle;

/*
 * Build a handle for widths D and C on the current HIP device.
 * D and C must be multiples of 32 in [32, 256].  The weights are copied,
 * rounded to the dtype (round to nearest even for bf16; LayerNorm parameters
 * stay fp32) and packed into device memory the handle owns.  Fails with
 * TRIMUL_ERR_ARCH on any device other than gfx950 (the message names the
 * device's architecture), TRIMUL_ERR_UNSUPPORTED for other widths.
 * The handle is read-only afterwards: concurrent trimul_fwd calls on
 * different streams with different workspaces are safe.
 */
trimul_status trimul_create(int D, int C, trimul_dtype dtype, const trimul_weights *w,
                            trimul_handle **out);

/* Release the handle's device memory.  Accepts NULL.  The caller must make
 * sure no enqueued trimul_fwd still uses the handle. */
void trimul_destroy(trimul_handle *h);

/* Bytes of workspace trimul_fwd needs for (B, N): the gated projections a and
 * b, each B*C*N*Kp elements of the dtype (Kp = N rounded up to a multiple of
 * 32 for bf16, Kp = N for fp32), and the contraction o, B*C*N*N elements; each
 * of the three rounded up to 256 bytes. */
trimul_status trimul_workspace_size(const trimul_handle *h, int B, int N, size_t *bytes);

/* Same figure from the widths alone (host arithmetic only; no device needed). */
trimul_status trimul_workspace_query(int D, int C, trimul_dtype dtype, int B, int N,
                                     size_t *bytes);

/*
 * Forward pass, asynchronous on `stream` (three kernel launches; no sync, no
 * allocation).
 *   z          [B][N][N][D] device, dtype of the handle, 16-byte aligned.
 *   pair_mask  [B][N][N] device, same dtype, or NULL for all ones.  Values are
 *              used as multipliers (0/1 in practice).
 *   out        [B][N][N][D] device, 16-byte aligned; must not overlap z, the
 *              mask or the workspace.
 *   workspace  device, >= trimul_workspace_size bytes, 256-byte aligned.
 * Requires B >= 1, N >= 8, N % 8 == 0, N <= 32768, B * C <= 65535 and
 * B * N * N < 2^31.
 */
trimul_status trimul_fwd(trimul_handle *h, const void *z, const void *pair_mask, int B, int N,
                         trimul_direction dir, void *out, void *workspace,
                         size_t workspace_bytes, hipStream_t stream);

/* Host-only check of a device architecture name such as "gfx950:sramecc+:xnack-". */
trimul_status trimul_check_arch(const char *gcn_arch_name);

const char *trimul_status_string(trimul_status s);
const char *trimul_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* TRIMUL_H */
