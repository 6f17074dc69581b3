/*
 * host_driver.c -- drives every host-side path of libtrimul that runs without
 * a GPU, in a build with AddressSanitizer and UndefinedBehaviorSanitizer on
 * the host code: the architecture gate, status strings, workspace queries,
 * argument validation of create / fwd / tune / noalloc / stage entry points
 * (each must fail cleanly with the documented status before touching a
 * device), the no-device path of create, and the plan cache file (store,
 * replace, look up, malformed lines, unwritable location).  Exits non-zero on
 * any unexpected status; the sanitizers abort on any memory or UB error.
 */
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "trimul.h"
#include "trimul_internal.h"

static int failures = 0;
#define EXPECT(cond)                                                         \
    do {                                                                     \
        if (!(cond)) {                                                       \
            fprintf(stderr, "%s:%d: expectation failed: %s\n", __FILE__, __LINE__, #cond); \
            ++failures;                                                      \
        }                                                                    \
    } while (0)

int main(int argc, char **argv)
{
    const char *dir = argc > 1 ? argv[1] : "/tmp";
    /* architecture gate */
    EXPECT(trimul_check_arch("gfx950") == TRIMUL_OK);
    EXPECT(trimul_check_arch("gfx950:sramecc+:xnack-") == TRIMUL_OK);
    EXPECT(trimul_check_arch("gfx942") == TRIMUL_ERR_ARCH);
    EXPECT(strstr(trimul_last_error(), "gfx942") != NULL);
    EXPECT(trimul_check_arch(NULL) == TRIMUL_ERR_INVALID_ARG);
    {
        char longname[2048];
        memset(longname, 'x', sizeof longname - 1);
        longname[sizeof longname - 1] = 0;
        EXPECT(trimul_check_arch(longname) == TRIMUL_ERR_ARCH);   /* message is truncated, not overrun */
    }
    for (int s = -1; s <= 7; ++s) EXPECT(trimul_status_string((trimul_status)s) != NULL);
    /* workspace queries */
    size_t bytes = 0;
    EXPECT(trimul_workspace_query(256, 256, TRIMUL_BF16, 1, 4096, &bytes) == TRIMUL_OK && bytes > 0);
    EXPECT(trimul_workspace_query(48, 32, TRIMUL_BF16, 1, 64, &bytes) == TRIMUL_ERR_UNSUPPORTED);
    EXPECT(trimul_workspace_query(32, 32, (trimul_dtype)9, 1, 64, &bytes) == TRIMUL_ERR_INVALID_ARG);
    EXPECT(trimul_workspace_query(32, 32, TRIMUL_FP32, 0, 64, &bytes) == TRIMUL_ERR_INVALID_ARG);
    EXPECT(trimul_workspace_query(32, 32, TRIMUL_FP32, 1, 64, NULL) == TRIMUL_ERR_INVALID_ARG);
    EXPECT(trimul_workspace_size(NULL, 1, 64, &bytes) == TRIMUL_ERR_INVALID_ARG);
    EXPECT(trimul_workspace_size_lean(NULL, 1, 64, &bytes) == TRIMUL_ERR_INVALID_ARG);
    /* create: argument checks, then the device query fails without a GPU */
    const int Dw = 32, Cw = 32;
    float *buf = (float *)calloc((size_t)(2 * Dw + 2 * Cw + 4 * Cw * Dw + Dw * Cw + Dw * Dw), sizeof(float));
    trimul_weights w = {buf, buf + Dw, buf + 2 * Dw, buf + 2 * Dw + 2 * Cw * Dw, buf + 2 * Dw + 4 * Cw * Dw,
                        buf + 2 * Dw + 4 * Cw * Dw + Cw, buf + 2 * Dw + 4 * Cw * Dw + 2 * Cw,
                        buf + 2 * Dw + 4 * Cw * Dw + 2 * Cw + Dw * Cw, 1e-5f};
    trimul_handle *h = (trimul_handle *)0x1;
    EXPECT(trimul_create(Dw, Cw, TRIMUL_BF16, &w, NULL) == TRIMUL_ERR_INVALID_ARG);
    EXPECT(trimul_create(Dw, Cw, TRIMUL_BF16, NULL, &h) == TRIMUL_ERR_INVALID_ARG && h == NULL);
    EXPECT(trimul_create(40, Cw, TRIMUL_BF16, &w, &h) == TRIMUL_ERR_UNSUPPORTED);
    trimul_weights w0 = w;
    w0.g_out = NULL;
    EXPECT(trimul_create(Dw, Cw, TRIMUL_BF16, &w0, &h) == TRIMUL_ERR_INVALID_ARG);
    w0 = w;
    w0.eps = -1.0f;
    EXPECT(trimul_create(Dw, Cw, TRIMUL_BF16, &w0, &h) == TRIMUL_ERR_INVALID_ARG);
    const trimul_status cs = trimul_create(Dw, Cw, TRIMUL_BF16, &w, &h);
    if (cs == TRIMUL_OK) {   /* a device is present: release it */
        trimul_destroy(h);
    } else {
        EXPECT(cs == TRIMUL_ERR_HIP && h == NULL);
    }
    free(buf);
    /* every entry point refuses a NULL handle before anything else */
    char dummy[64];
    EXPECT(trimul_fwd(NULL, dummy, NULL, 1, 64, TRIMUL_OUTGOING, dummy, dummy, 64, NULL) == TRIMUL_ERR_INVALID_ARG);
    EXPECT(trimul_tune(NULL, dummy, NULL, 1, 64, TRIMUL_OUTGOING, dummy, dummy, 64, NULL) == TRIMUL_ERR_INVALID_ARG);
    EXPECT(trimul_fwd_noalloc(NULL, dummy, NULL, 1, 64, TRIMUL_OUTGOING, dummy, NULL) == TRIMUL_ERR_INVALID_ARG);
    EXPECT(trimul_internal_project(NULL, dummy, NULL, 1, 64, TRIMUL_OUTGOING, dummy, dummy, NULL) ==
           TRIMUL_ERR_INVALID_ARG);
    EXPECT(trimul_internal_contract(NULL, dummy, dummy, NULL, 1, 64, TRIMUL_OUTGOING, dummy, NULL) ==
           TRIMUL_ERR_INVALID_ARG);
    EXPECT(trimul_internal_output(NULL, dummy, dummy, 1, 64, dummy, NULL) == TRIMUL_ERR_INVALID_ARG);
    EXPECT(trimul_internal_mask_ranges(NULL, dummy, 1, 64, TRIMUL_OUTGOING, (int *)dummy, NULL) ==
           TRIMUL_ERR_INVALID_ARG);
    int v = 0, o = 0, g = 0, t = 0;
    EXPECT(trimul_internal_get_plan(NULL, 1, 64, TRIMUL_OUTGOING, 0, &v, &o, &g, &t) == TRIMUL_ERR_INVALID_ARG);
    EXPECT(trimul_internal_set_plan(NULL, 1, 64, TRIMUL_OUTGOING, 0, 0, 0, 8, 256) == TRIMUL_ERR_INVALID_ARG);
    trimul_destroy(NULL);
    /* plan candidates */
    const int n = trimul_internal_plan_candidates(NULL, NULL, NULL, NULL, 0);
    EXPECT(n >= 2);
    int *cv = (int *)calloc((size_t)n, sizeof(int)), *co = (int *)calloc((size_t)n, sizeof(int)),
        *cg = (int *)calloc((size_t)n, sizeof(int)), *ct = (int *)calloc((size_t)n, sizeof(int));
    EXPECT(trimul_internal_plan_candidates(cv, co, cg, ct, n) == n);
    EXPECT(trimul_internal_plan_candidates(cv, co, cg, ct, 1) == n);   /* cap respected */
    /* plan cache file */
    char path[1024];
    snprintf(path, sizeof path, "%s/sub/dir/plans.txt", dir);
    for (int i = 0; i < n; ++i)
        EXPECT(trimul_internal_cache_store(path, "gfx950-256cu", 256, 256, 0, 1, 4096 + 8 * i, i % 2, i % 2, cv[i],
                                           co[i], cg[i], ct[i], 1.5 * i) == TRIMUL_OK);
    for (int i = 0; i < n; ++i) {
        EXPECT(trimul_internal_cache_lookup(path, "gfx950-256cu", 256, 256, 0, 1, 4096 + 8 * i, i % 2, i % 2, &v, &o,
                                            &g, &t) == 1);
        EXPECT(v == cv[i] && o == co[i] && g == cg[i] && t == ct[i]);
    }
    EXPECT(trimul_internal_cache_lookup(path, "gfx950-256cu", 256, 256, 0, 1, 4095, 0, 0, &v, &o, &g, &t) == 0);
    EXPECT(trimul_internal_cache_store(path, "gfx950-256cu", 256, 256, 0, 1, 4096, 0, 0, cv[n - 1], co[n - 1],
                                       cg[n - 1], ct[n - 1], 2.0) == TRIMUL_OK);
    EXPECT(trimul_internal_cache_lookup(path, "gfx950-256cu", 256, 256, 0, 1, 4096, 0, 0, &v, &o, &g, &t) == 1 &&
           o == co[n - 1] && g == cg[n - 1] && t == ct[n - 1]);
    EXPECT(trimul_internal_cache_store(path, "gfx950-256cu", 256, 256, 0, 1, 64, 0, 0, 0, 3, 8, 256, 1.0) ==
           TRIMUL_ERR_INVALID_ARG);
    EXPECT(trimul_internal_cache_store(path, "gfx950-256cu", 256, 256, 0, 1, 64, 0, 0, 0, 0, 8, 96, 1.0) ==
           TRIMUL_ERR_INVALID_ARG);
    {
        FILE *f = fopen(path, "a");
        if (f) {
            fputs("trimul-plan v3 gfx950-256cu 256 256 0 1 77 0 0 0 1\n", f);   /* truncated */
            fputs("trimul-plan v3 gfx950-256cu 256 256 0 1 78 0 0 0 1 8 256 nan-ish trailing junk\n", f);
            fputs("#\n\n", f);
            for (int i = 0; i < 300; ++i) fputc('z', f);   /* a long line */
            fputc('\n', f);
            fclose(f);
        }
        EXPECT(trimul_internal_cache_lookup(path, "gfx950-256cu", 256, 256, 0, 1, 77, 0, 0, &v, &o, &g, &t) == 0);
    }
    char blocker[1024], bad[1100];
    snprintf(blocker, sizeof blocker, "%s/blocker", dir);
    FILE *bf = fopen(blocker, "w");
    if (bf) fclose(bf);
    snprintf(bad, sizeof bad, "%s/plans.txt", blocker);
    EXPECT(trimul_internal_cache_store(bad, "d", 32, 32, 0, 1, 64, 0, 0, 0, 0, 8, 256, 1.0) == TRIMUL_ERR_INVALID_ARG);
    EXPECT(trimul_internal_cache_lookup(bad, "d", 32, 32, 0, 1, 64, 0, 0, &v, &o, &g, &t) <= 0);
    char pbuf[8];
    EXPECT(trimul_internal_cache_path(pbuf, (int)sizeof pbuf) >= 0);   /* truncated into a small buffer */
    free(cv); free(co); free(cg); free(ct);
    printf("host driver: %d failures\n", failures);
    return failures ? 1 : 0;
}
