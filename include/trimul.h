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
 *  - LayerNorm range (bf16 handles): both LayerNorms take their statistics in
 *    one fp32 pass (var = E[v^2] - mean^2); the output stage applies them
 *    algebraically to the raw bf16 rows of z (for the output gate) and o.
 *    Results stay within the bf16 tolerance (normalised max error 2e-2
 *    against an fp64 evaluation) for rows whose |mean| is up to 128 standard
 *    deviations; the cancellation grows like (mean / std)^2 and rows far
 *    beyond that lose accuracy.  fp32 handles normalise explicitly (two
 *    passes) and have no such limit.
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
 *
 * Defined by the fold-cp-ops README, "Use", step 2 (the constructor takes the
 * layer, the direction-independent configuration and the dtype, and makes
 * every data-independent choice, so that forward makes none), with the layer
 * of step 1b (the six submodules, mirrored by trimul_weights), and by its
 * "Hardware" section (a device of another architecture is refused up front
 * with a message naming what was found, rather than failing inside a launch).
 *
 * Arguments: D, C widths (multiples of 32 in [32, 256]); dtype of every
 * tensor later passed to trimul_fwd; w: host fp32 weights, read only during
 * the call (the caller keeps ownership); *out receives the new handle (NULL on
 * failure).  The weights are copied, rounded to the dtype (round to nearest
 * even for bf16; LayerNorm parameters stay fp32) and packed into device memory
 * the handle owns, on the device current at the call.  Any plan recorded for
 * this (D, C, dtype) in the tuning cache (trimul_tune) is loaded here.
 * Errors: TRIMUL_ERR_INVALID_ARG (NULL pointer, bad dtype or eps),
 * TRIMUL_ERR_UNSUPPORTED (other widths), TRIMUL_ERR_ARCH (device is not
 * gfx950; the message names its architecture), TRIMUL_ERR_HIP (device query,
 * allocation or copy failed).  Nothing is allocated on failure.
 * The handle is read-only afterwards except for trimul_tune: concurrent
 * trimul_fwd calls on different streams with different workspaces are safe.
 */
trimul_status trimul_create(int D, int C, trimul_dtype dtype, const trimul_weights *w,
                            trimul_handle **out);

/* Release the handle and its device memory (the packed weights).
 * Defined by the fold-cp-ops README, "Use", step 4 (release what construction
 * built, after the last forward).  Accepts NULL.  The caller must make sure no
 * enqueued trimul_fwd still uses the handle (synchronise its streams first);
 * caller-owned tensors and workspaces are not touched. */
void trimul_destroy(trimul_handle *h);

/* Bytes of workspace trimul_fwd needs for (B, N).
 * This is the shape-time step of the fold-cp-ops README, "Use", step 2b (the
 * optional call made once the token count and batch are known, before the
 * first forward; there it pre-compiles, here the kernels are compiled ahead of
 * time and what depends on the shape is the scratch memory the caller must
 * provide).  The workspace holds the gated projections a and b, each
 * B*C*N*Kp elements of the dtype (Kp = N rounded up to a multiple of 32 for
 * bf16, Kp = N for fp32), the contraction o, B*C*N*N elements, and a table
 * for masked calls (per 256-token tile, its live key range; per batch element,
 * the order of its tile pairs): 4 * (2*B*T + 4 + B*T*T) bytes with
 * T = ceil(N/256); each of the four rounded up to 256 bytes.  Errors: TRIMUL_ERR_INVALID_ARG (NULL handle
 * or bytes, B or N < 1). */
trimul_status trimul_workspace_size(const trimul_handle *h, int B, int N, size_t *bytes);

/* Same figure from the widths alone (host arithmetic only; no device needed). */
trimul_status trimul_workspace_query(int D, int C, trimul_dtype dtype, int B, int N,
                                     size_t *bytes);

/* Smallest workspace trimul_fwd accepts for (B, N): the lean layout, for
 * shapes where memory is the constraint (the fold-cp-ops README sizes its
 * problems by what one device holds, "Use", step 0).  a and b as above; o gets
 * memory of its own for one chunk of the B*C (batch, channel) slabs only: the
 * contraction then runs chunk by chunk and stores each later chunk's o over
 * the a slabs of the chunk before it, which that chunk has finished reading.
 * At B=1, N=8192, C=128 in bf16 this is 35.4 GB against 51.5 GB.  trimul_fwd
 * uses the full layout whenever the workspace it is given holds it, and the
 * lean one otherwise; results are identical.  Errors: TRIMUL_ERR_INVALID_ARG
 * (NULL handle or bytes, B or N < 1). */
trimul_status trimul_workspace_size_lean(const trimul_handle *h, int B, int N, size_t *bytes);

/*
 * Forward pass, asynchronous on `stream` (no sync, no allocation).
 *
 * Defined by the fold-cp-ops README, "Use", step 3 (the caller allocates its
 * own x of shape (B, N, N, D) and pair mask of shape (B, N, N) and gets back a
 * tensor of the same shape), with the shape rule of step 0 (N a multiple of 8,
 * the 16-byte vector floor) and the direction chosen as in step 2.  The
 * arithmetic is the formula at the top of this file; the kernels are the
 * LayerNorm + gated projection, the per-channel contraction (preceded, when a
 * mask is given, by a scan of the mask for the key ranges it leaves live) and
 * the LayerNorm + output projection + gate.
 *   z          [B][N][N][D] device, dtype of the handle, 16-byte aligned.
 *   pair_mask  [B][N][N] device, same dtype, 16-byte aligned, or NULL for all
 *              ones.  Values are used as multipliers (0/1 in practice); keys
 *              whose mask is zero for a whole 256-row tile are skipped by the
 *              contraction (their products are exact zeros).
 *   out        [B][N][N][D] device, 16-byte aligned; must not overlap z, the
 *              mask or the workspace.
 *   workspace  device, 256-byte aligned, at least trimul_workspace_size_lean
 *              bytes; with trimul_workspace_size bytes or more the full layout
 *              is used (one contraction launch), else the lean one.
 * Requires B >= 1, N >= 8, N % 8 == 0, N <= 32768, B * C <= 65535 and
 * B * N * N < 2^31.  Device pointers stay caller-owned and must stay valid
 * until the enqueued work has finished.  Errors (nothing is enqueued):
 * TRIMUL_ERR_INVALID_ARG (NULL, misaligned or overlapping pointers, bad sizes
 * or direction, handle from another device), TRIMUL_ERR_UNSUPPORTED (sizes
 * beyond the limits above), TRIMUL_ERR_WORKSPACE (workspace NULL or too
 * small), TRIMUL_ERR_HIP (a launch failed; the message has the HIP error).
 */
trimul_status trimul_fwd(trimul_handle *h, const void *z, const void *pair_mask, int B, int N,
                         trimul_direction dir, void *out, void *workspace,
                         size_t workspace_bytes, hipStream_t stream);

/*
 * trimul_fwd for callers that cannot allocate (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc): the same kernels and
 * arguments without the workspace, which comes from a static device array of
 * TRIMUL_NOALLOC_MAX_BYTES per GPU (loaded with the library, held until the
 * process ends).  The call allocates nothing and makes no allocating call.
 * Shapes whose workspace (lean layout when the full one does not fit) exceeds
 * the array fail with TRIMUL_ERR_UNSUPPORTED before anything is enqueued; at
 * D = C = 128, B = 1 that allows N up to 416.  Every call on one GPU
 * uses the same array: calls that overlap in time on one GPU (different
 * streams, no ordering between them) race and give wrong results; calls
 * ordered on one stream are safe.  The array's contents are left over from
 * the previous call, and nothing the kernels read from it needs clearing
 * (every byte read in a call is written earlier in the same call).  Other
 * errors as trimul_fwd.
 */
#define TRIMUL_NOALLOC_MAX_BYTES (128u << 20)
trimul_status trimul_fwd_noalloc(trimul_handle *h, const void *z, const void *pair_mask, int B,
                                 int N, trimul_direction dir, void *out, hipStream_t stream);

/*
 * Tune the kernel plan for this call's shape, then leave the forward result in
 * out.  Blocking: returns after the work on `stream` has finished.
 *
 * Defined by the fold-cp-ops README's autotuned single-device path ("Use":
 * the single-device kernel is the autotuned one) and its on-disk tuning store
 * ("Environment": kept apart from the compile cache; cold and warm runs of an
 * autotuning path differ by about 2x).  Arguments, layouts and errors are
 * those of trimul_fwd.  Every candidate plan computes bitwise the same result
 * (plans reorder or resize the contraction's tiles, and every output still sums
 * its keys in the same order); each is run on the caller's inputs and
 * timed with HIP events, and the fastest is recorded in the handle for
 * (B, N, direction, masked) and in the plan cache file ($TRIMUL_PLAN_CACHE,
 * else $XDG_CACHE_HOME/libtrimul/plans.txt, else ~/.cache/libtrimul/plans.txt;
 * TRIMUL_PLAN_CACHE=0 disables it), from which trimul_create of a later process
 * loads it.  trimul_fwd then uses the recorded plan, and the default plan for
 * shapes never tuned.  An unwritable cache is not an error.  Must not run
 * concurrently with another call on the same handle.
 */
trimul_status trimul_tune(trimul_handle *h, const void *z, const void *pair_mask, int B, int N,
                          trimul_direction dir, void *out, void *workspace,
                          size_t workspace_bytes, hipStream_t stream);

/* Host-only check of a device architecture name such as "gfx950:sramecc+:xnack-",
 * the test used by trimul_create (fold-cp-ops README, "Hardware": refuse other
 * architectures with a message that names the one found).  Returns TRIMUL_OK
 * for gfx950 with any feature suffix, TRIMUL_ERR_ARCH otherwise (message
 * "libtrimul requires gfx950 (MI355X); got <name>"), TRIMUL_ERR_INVALID_ARG for
 * NULL.  Needs no device. */
trimul_status trimul_check_arch(const char *gcn_arch_name);

/* Name of a status code ("TRIMUL_OK", ...; "TRIMUL_ERR_UNKNOWN" for others).
 * The string is static. */
const char *trimul_status_string(trimul_status s);
/* Message of the last failing call on this thread (empty after a success).
 * Valid until the next libtrimul call on the same thread. */
const char *trimul_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* TRIMUL_H */
