/*
 * trimul_oracle.c -- plain, slow, fp64 CPU oracle for the forward triangle
 * multiplicative update (TriMul).  TEST INFRASTRUCTURE ONLY: nothing on the
 * product path may include, link or call this file; only the test suite, the
 * smoke check and the CPU-baseline leg of the benchmark use it.  It shares no
 * code, header, table or helper with the HIP library.
 *
 * What it computes follows the "Use" section of the fold-cp-ops README (the
 * layer with the six submodules norm_in, norm_out = LayerNorm(D); p_in, g_in =
 * Linear(D, 2D, bias=False); p_out, g_out = Linear(D, D, bias=False); the
 * direction argument "outgoing"; the optional pair mask; inference only).  The
 * README gives module names and shapes but no formula, so the composition is
 * the plainest reading the page supports, written out here step by step:
 *
 *   x_ij   = LayerNorm_in(z_ij)                     over the D channels
 *   a_ijc  = m_ij * (p_in x_ij)_c       * sigm((g_in x_ij)_c)        c <  C
 *   b_ijc  = m_ij * (p_in x_ij)_(C + c) * sigm((g_in x_ij)_(C + c))
 *   o_ijc  = sum_k a_ikc * b_jkc            (outgoing)
 *   o_ijc  = sum_k a_kic * b_kjc            (incoming)
 *   y_ij   = LayerNorm_out(o_ij)                    over the C channels
 *   out_ij = (p_out y_ij) * sigm(g_out x_ij)
 *
 * with sigm(t) = 1 / (1 + exp(-t)), LayerNorm with biased variance, eps added
 * under the square root and an affine gamma/beta, and Linear(W) x = W x with W
 * stored [out][in].  Every sum runs in ascending index order in double
 * precision.  Inputs arrive as float (they are exactly the values the GPU sees:
 * bf16-rounded or fp32) and are widened to double on read.
 *
 * Two entry points:
 *   orc_trimul_full  -- every output of B x N x N, optional stage dumps.
 *   orc_trimul_grid  -- the outputs at an (I x J) grid of (i, j) pairs of one
 *                       batch element, from the z vectors those outputs need
 *                       (gathered by the caller), for N too large to run whole.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

typedef struct {
    const float *ln_in_w, *ln_in_b;   /* [D]                                   */
    const float *p_in, *g_in;         /* [2C][D]  rows [0,C) -> a, [C,2C) -> b  */
    const float *ln_out_w, *ln_out_b; /* [C]                                   */
    const float *p_out;               /* [D][C]                                */
    const float *g_out;               /* [D][D]                                */
    double eps;
    int D, C;
} orc_weights;

static double sigm(double t) { return 1.0 / (1.0 + exp(-t)); }

/* LayerNorm of one vector of length L: mean, biased variance, affine. */
static void layer_norm(const double *v, int L, const float *gamma, const float *beta,
                       double eps, double *out)
{
    double mu = 0.0;
    for (int d = 0; d < L; ++d) mu += v[d];
    mu /= (double)L;
    double var = 0.0;
    for (int d = 0; d < L; ++d) var += (v[d] - mu) * (v[d] - mu);
    var /= (double)L;
    double inv = 1.0 / sqrt(var + eps);
    for (int d = 0; d < L; ++d) out[d] = (v[d] - mu) * inv * (double)gamma[d] + (double)beta[d];
}

/* y = W x for W stored [rows][cols] (float), x double. */
static double dot_row(const float *w_row, const double *x, int cols)
{
    double s = 0.0;
    for (int e = 0; e < cols; ++e) s += (double)w_row[e] * x[e];
    return s;
}

/* LayerNorm_in of one pair, then its gated a and b vectors (mask applied). */
static void project_pair(const orc_weights *w, const float *z_pair, double m,
                         double *x, double *a, double *b)
{
    const int D = w->D, C = w->C;
    double zd[256];
    for (int d = 0; d < D; ++d) zd[d] = (double)z_pair[d];
    layer_norm(zd, D, w->ln_in_w, w->ln_in_b, w->eps, x);
    for (int c = 0; c < C; ++c) {
        if (a) {
            double pa = dot_row(w->p_in + (size_t)c * D, x, D);
            double ga = dot_row(w->g_in + (size_t)c * D, x, D);
            a[c] = m * pa * sigm(ga);
        }
        if (b) {
            double pb = dot_row(w->p_in + (size_t)(C + c) * D, x, D);
            double gb = dot_row(w->g_in + (size_t)(C + c) * D, x, D);
            b[c] = m * pb * sigm(gb);
        }
    }
}

/* out_d = (p_out LN_out(o))_d * sigm((g_out x)_d) for one pair. */
static void output_pair(const orc_weights *w, const double *o, const double *x, double *out)
{
    const int D = w->D, C = w->C;
    double y[256];
    layer_norm(o, C, w->ln_out_w, w->ln_out_b, w->eps, y);
    for (int d = 0; d < D; ++d) {
        double lin = dot_row(w->p_out + (size_t)d * C, y, C);
        double gate = sigm(dot_row(w->g_out + (size_t)d * D, x, D));
        out[d] = lin * gate;
    }
}

static int check_dims(int D, int C)
{
    if (D < 1 || D > 256 || C < 1 || C > 256) return 1;
    return 0;
}

int orc_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/*
 * Full mode.  z: [B][N][N][D]; mask: [B][N][N] or NULL (all ones);
 * direction 0 = outgoing, 1 = incoming.  out: [B][N][N][D].
 * Optional dumps (NULL to skip): x [B][N][N][D], a and b [B][N][N][C] (pair
 * layout a_bijc), o [B][N][N][C].
 * Returns 0 on success, nonzero on bad arguments or allocation failure.
 */
int orc_trimul_full(int B, int N, int D, int C, int direction,
                    const float *z, const float *mask,
                    const float *ln_in_w, const float *ln_in_b,
                    const float *p_in, const float *g_in,
                    const float *ln_out_w, const float *ln_out_b,
                    const float *p_out, const float *g_out, double eps,
                    double *out, double *x_dump, double *a_dump, double *b_dump,
                    double *o_dump)
{
    if (B < 1 || N < 1 || check_dims(D, C) || (direction != 0 && direction != 1)) return 1;
    orc_weights w = {ln_in_w, ln_in_b, p_in, g_in, ln_out_w, ln_out_b, p_out, g_out, eps, D, C};
    const int64_t P = (int64_t)N * N;
    double *x = (double *)malloc(sizeof(double) * (size_t)(P * D));
    double *a = (double *)malloc(sizeof(double) * (size_t)(P * C));
    double *b = (double *)malloc(sizeof(double) * (size_t)(P * C));
    double *o = (double *)malloc(sizeof(double) * (size_t)(P * C));
    if (!x || !a || !b || !o) { free(x); free(a); free(b); free(o); return 2; }

    for (int bb = 0; bb < B; ++bb) {
        const float *zb = z + (size_t)bb * P * D;
        const float *mb = mask ? mask + (size_t)bb * P : NULL;
        /* LayerNorm_in and the gated projections, pair by pair. */
        #pragma omp parallel for schedule(static)
        for (int64_t p = 0; p < P; ++p) {
            double m = mb ? (double)mb[p] : 1.0;
            project_pair(&w, zb + (size_t)p * D, m, x + (size_t)p * D, a + (size_t)p * C,
                         b + (size_t)p * C);
        }
        /* Triangle contraction, k ascending. */
        #pragma omp parallel for schedule(static)
        for (int i = 0; i < N; ++i) {
            for (int j = 0; j < N; ++j) {
                double *oij = o + ((size_t)i * N + j) * C;
                for (int c = 0; c < C; ++c) oij[c] = 0.0;
                for (int k = 0; k < N; ++k) {
                    const double *ta, *tb;
                    if (direction == 0) {          /* a_ikc * b_jkc */
                        ta = a + ((size_t)i * N + k) * C;
                        tb = b + ((size_t)j * N + k) * C;
                    } else {                       /* a_kic * b_kjc */
                        ta = a + ((size_t)k * N + i) * C;
                        tb = b + ((size_t)k * N + j) * C;
                    }
                    for (int c = 0; c < C; ++c) oij[c] += ta[c] * tb[c];
                }
            }
        }
        /* LayerNorm_out, output projection and output gate. */
        double *ob = out + (size_t)bb * P * D;
        #pragma omp parallel for schedule(static)
        for (int64_t p = 0; p < P; ++p)
            output_pair(&w, o + (size_t)p * C, x + (size_t)p * D, ob + (size_t)p * D);

        if (x_dump) memcpy(x_dump + (size_t)bb * P * D, x, sizeof(double) * (size_t)(P * D));
        if (a_dump) memcpy(a_dump + (size_t)bb * P * C, a, sizeof(double) * (size_t)(P * C));
        if (b_dump) memcpy(b_dump + (size_t)bb * P * C, b, sizeof(double) * (size_t)(P * C));
        if (o_dump) memcpy(o_dump + (size_t)bb * P * C, o, sizeof(double) * (size_t)(P * C));
    }
    free(x); free(a); free(b); free(o);
    return 0;
}

/*
 * Grid mode, one batch element.  For output rows I (ni of them) and output
 * columns J (nj), the caller gathers
 *   zA[ii][k][:] -- the z vector whose a-term enters o_(I[ii], j) at index k:
 *                   z_(i,k) for outgoing, z_(k,i) for incoming;
 *   mA[ii][k]    -- the mask value of that same pair (NULL: ones);
 *   zB[jj][k][:], mB[jj][k] -- likewise for the b-term of column J[jj]:
 *                   z_(j,k) for outgoing, z_(k,j) for incoming;
 *   zG[ii][jj][:] -- z_(i,j), the input of the output gate at that pair.
 * out: [ni][nj][D]; o_dump: [ni][nj][C] or NULL.
 * t_stage (may be NULL) receives wall seconds of {projection, contraction,
 * output} for the CPU baseline's extrapolation.
 */
int orc_trimul_grid(int N, int D, int C, int ni, int nj,
                    const float *zA, const float *mA, const float *zB, const float *mB,
                    const float *zG,
                    const float *ln_in_w, const float *ln_in_b,
                    const float *p_in, const float *g_in,
                    const float *ln_out_w, const float *ln_out_b,
                    const float *p_out, const float *g_out, double eps,
                    double *out, double *o_dump, double *t_stage)
{
    if (N < 1 || ni < 1 || nj < 1 || check_dims(D, C)) return 1;
    orc_weights w = {ln_in_w, ln_in_b, p_in, g_in, ln_out_w, ln_out_b, p_out, g_out, eps, D, C};
    double *ar = (double *)malloc(sizeof(double) * (size_t)ni * N * C);
    double *br = (double *)malloc(sizeof(double) * (size_t)nj * N * C);
    if (!ar || !br) { free(ar); free(br); return 2; }
    double t0 = 0, t1 = 0, t2 = 0, t3 = 0;
#ifdef _OPENMP
    t0 = omp_get_wtime();
#endif
    #pragma omp parallel
    {
        double xs[256];
        #pragma omp for schedule(static)
        for (int64_t r = 0; r < (int64_t)ni * N; ++r) {
            double m = mA ? (double)mA[r] : 1.0;
            project_pair(&w, zA + (size_t)r * D, m, xs, ar + (size_t)r * C, NULL);
        }
        #pragma omp for schedule(static)
        for (int64_t r = 0; r < (int64_t)nj * N; ++r) {
            double m = mB ? (double)mB[r] : 1.0;
            project_pair(&w, zB + (size_t)r * D, m, xs, NULL, br + (size_t)r * C);
        }
    }
#ifdef _OPENMP
    t1 = omp_get_wtime();
#endif
    double *o = (double *)malloc(sizeof(double) * (size_t)ni * nj * C);
    if (!o) { free(ar); free(br); return 2; }
    #pragma omp parallel for schedule(static)
    for (int64_t q = 0; q < (int64_t)ni * nj; ++q) {
        int ii = (int)(q / nj), jj = (int)(q % nj);
        double *oq = o + (size_t)q * C;
        for (int c = 0; c < C; ++c) oq[c] = 0.0;
        for (int k = 0; k < N; ++k) {
            const double *ta = ar + ((size_t)ii * N + k) * C;
            const double *tb = br + ((size_t)jj * N + k) * C;
            for (int c = 0; c < C; ++c) oq[c] += ta[c] * tb[c];
        }
    }
#ifdef _OPENMP
    t2 = omp_get_wtime();
#endif
    #pragma omp parallel
    {
        double xs[256], zd[256];
        #pragma omp for schedule(static)
        for (int64_t q = 0; q < (int64_t)ni * nj; ++q) {
            const float *zq = zG + (size_t)q * D;
            for (int d = 0; d < D; ++d) zd[d] = (double)zq[d];
            layer_norm(zd, D, w.ln_in_w, w.ln_in_b, w.eps, xs);
            output_pair(&w, o + (size_t)q * C, xs, out + (size_t)q * D);
        }
    }
#ifdef _OPENMP
    t3 = omp_get_wtime();
#endif
    if (o_dump) memcpy(o_dump, o, sizeof(double) * (size_t)ni * nj * C);
    if (t_stage) { t_stage[0] = t1 - t0; t_stage[1] = t2 - t1; t_stage[2] = t3 - t2; }
    free(ar); free(br); free(o);
    return 0;
}

/*
 * Output stage alone: for P pairs with given o [P][C] and z [P][D] (both float
 * inputs widened to double), out[p] = (p_out LayerNorm_out(o_p)) *
 * sigm(g_out LayerNorm_in(z_p)).  Used to check the output kernel by itself.
 */
int orc_output_stage(int64_t P, int D, int C, const float *z, const float *o,
                     const float *ln_in_w, const float *ln_in_b,
                     const float *ln_out_w, const float *ln_out_b,
                     const float *p_out, const float *g_out, double eps, double *out)
{
    if (P < 0 || check_dims(D, C)) return 1;
    orc_weights w = {ln_in_w, ln_in_b, NULL, NULL, ln_out_w, ln_out_b, p_out, g_out, eps, D, C};
    #pragma omp parallel
    {
        double xs[256], zd[256], od[256];
        #pragma omp for schedule(static)
        for (int64_t p = 0; p < P; ++p) {
            for (int d = 0; d < D; ++d) zd[d] = (double)z[(size_t)p * D + d];
            for (int c = 0; c < C; ++c) od[c] = (double)o[(size_t)p * C + c];
            layer_norm(zd, D, w.ln_in_w, w.ln_in_b, w.eps, xs);
            output_pair(&w, od, xs, out + (size_t)p * D);
        }
    }
    return 0;
}
