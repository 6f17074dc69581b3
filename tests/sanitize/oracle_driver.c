/*
 * oracle_driver.c -- drives the fp64 oracle (oracle/trimul_oracle.c) under
 * AddressSanitizer and UndefinedBehaviorSanitizer: full mode with every stage
 * dump, grid mode and the output stage, both directions, with and without a
 * mask, and checks that grid mode and the output stage reproduce full mode
 * (grid bitwise, output stage to 1e-12).  Test infrastructure only.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int orc_trimul_full(int B, int N, int D, int C, int direction, const float *z, const float *mask,
                    const float *ln_in_w, const float *ln_in_b, const float *p_in, const float *g_in,
                    const float *ln_out_w, const float *ln_out_b, const float *p_out,
                    const float *g_out, double eps, double *out, double *x_dump, double *a_dump,
                    double *b_dump, double *o_dump);
int orc_trimul_grid(int N, int D, int C, int ni, int nj, const float *zA, const float *mA,
                    const float *zB, const float *mB, const float *zG, const float *ln_in_w,
                    const float *ln_in_b, const float *p_in, const float *g_in,
                    const float *ln_out_w, const float *ln_out_b, const float *p_out,
                    const float *g_out, double eps, double *out, double *o_dump, double *t_stage);
int orc_output_stage(int64_t P, int D, int C, const float *z, const float *o, const float *ln_in_w,
                     const float *ln_in_b, const float *ln_out_w, const float *ln_out_b,
                     const float *p_out, const float *g_out, double eps, double *out);

static uint32_t rng = 12345u;
static float urand(void)   /* uniform in [-1, 1) */
{
    rng = rng * 1664525u + 1013904223u;
    return (float)((rng >> 8) * (1.0 / 8388608.0)) - 1.0f;
}
static float *fill(size_t n, float scale, float offset)
{
    float *p = (float *)malloc(n * sizeof(float));
    for (size_t i = 0; i < n; ++i) p[i] = offset + scale * urand();
    return p;
}

#define B 2
#define N 7
#define D 16
#define C 8

int main(void)
{
    float *z = fill((size_t)B * N * N * D, 1.5f, 0.2f);
    float *lw = fill(D, 0.1f, 1.0f), *lb = fill(D, 0.1f, 0.0f);
    float *pin = fill(2 * C * D, 0.25f, 0.0f), *gin = fill(2 * C * D, 0.25f, 0.0f);
    float *low = fill(C, 0.1f, 1.0f), *lob = fill(C, 0.1f, 0.0f);
    float *pout = fill(D * C, 0.25f, 0.0f), *gout = fill(D * D, 0.25f, 0.0f);
    float tok[N] = {1, 1, 0, 1, 1, 1, 0};
    float *mask = (float *)malloc(sizeof(float) * B * N * N);
    for (int b = 0; b < B; ++b)
        for (int i = 0; i < N; ++i)
            for (int j = 0; j < N; ++j) mask[((size_t)b * N + i) * N + j] = tok[i] * tok[j];
    const size_t P = (size_t)B * N * N;
    double *out = malloc(sizeof(double) * P * D), *x = malloc(sizeof(double) * P * D);
    double *a = malloc(sizeof(double) * P * C), *bb = malloc(sizeof(double) * P * C);
    double *o = malloc(sizeof(double) * P * C), *os = malloc(sizeof(double) * P * D);
    const int I[3] = {0, 3, 6}, J[3] = {1, 2, 6};
    float *zA = malloc(sizeof(float) * 3 * N * D), *zB = malloc(sizeof(float) * 3 * N * D);
    float *zG = malloc(sizeof(float) * 9 * D), *mA = malloc(sizeof(float) * 3 * N);
    float *mB = malloc(sizeof(float) * 3 * N), *o32 = malloc(sizeof(float) * P * C);
    double gout_[9 * D], go_[9 * C], t[3];
    int bad = 0;
    for (int dir = 0; dir < 2; ++dir)
        for (int masked = 0; masked < 2; ++masked) {
            const float *m = masked ? mask : NULL;
            if (orc_trimul_full(B, N, D, C, dir, z, m, lw, lb, pin, gin, low, lob, pout, gout, 1e-5, out, x,
                                a, bb, o))
                return 2;
            for (int b = 0; b < B; ++b) {
                const float *zb = z + (size_t)b * N * N * D, *mb = mask + (size_t)b * N * N;
                for (int r = 0; r < 3; ++r)
                    for (int k = 0; k < N; ++k) {
                        const size_t ia = dir ? ((size_t)k * N + I[r]) : ((size_t)I[r] * N + k);
                        const size_t ib = dir ? ((size_t)k * N + J[r]) : ((size_t)J[r] * N + k);
                        memcpy(zA + ((size_t)r * N + k) * D, zb + ia * D, sizeof(float) * D);
                        memcpy(zB + ((size_t)r * N + k) * D, zb + ib * D, sizeof(float) * D);
                        mA[r * N + k] = mb[ia];
                        mB[r * N + k] = mb[ib];
                    }
                for (int r = 0; r < 3; ++r)
                    for (int c = 0; c < 3; ++c)
                        memcpy(zG + ((size_t)r * 3 + c) * D, zb + ((size_t)I[r] * N + J[c]) * D, sizeof(float) * D);
                if (orc_trimul_grid(N, D, C, 3, 3, zA, masked ? mA : NULL, zB, masked ? mB : NULL, zG, lw, lb, pin,
                                    gin, low, lob, pout, gout, 1e-5, gout_, go_, t))
                    return 3;
                for (int r = 0; r < 3; ++r)
                    for (int c = 0; c < 3; ++c)
                        for (int d = 0; d < D; ++d)
                            if (gout_[((size_t)r * 3 + c) * D + d] !=
                                out[(((size_t)b * N + I[r]) * N + J[c]) * D + d])
                                ++bad;
            }
            for (size_t i = 0; i < P * C; ++i) o32[i] = (float)o[i];
            if (orc_output_stage((int64_t)P, D, C, z, o32, lw, lb, low, lob, pout, gout, 1e-5, os)) return 4;
            /* the output stage from the (float-rounded) o of full mode agrees closely */
            for (size_t i = 0; i < P * D; ++i)
                if (fabs(os[i] - out[i]) > 1e-4 * (1.0 + fabs(out[i]))) ++bad;
        }
    /* argument checks return errors, not crashes */
    if (orc_trimul_full(B, N, 0, C, 0, z, NULL, lw, lb, pin, gin, low, lob, pout, gout, 1e-5, out, NULL, NULL,
                        NULL, NULL) == 0)
        ++bad;
    if (orc_trimul_grid(N, 300, C, 3, 3, zA, NULL, zB, NULL, zG, lw, lb, pin, gin, low, lob, pout, gout, 1e-5,
                        gout_, NULL, NULL) == 0)
        ++bad;
    free(z); free(lw); free(lb); free(pin); free(gin); free(low); free(lob); free(pout); free(gout);
    free(mask); free(out); free(x); free(a); free(bb); free(o); free(os); free(zA); free(zB); free(zG);
    free(mA); free(mB); free(o32);
    printf("oracle driver: %d mismatches\n", bad);
    return bad ? 1 : 0;
}
