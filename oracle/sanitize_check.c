/*
 * Standalone driver for sanitizer builds of oracle.c -- TEST INFRASTRUCTURE.
 *
 * tests/test_oracle_sanitize.py compiles this file together with oracle.c
 * twice with gcc: with AddressSanitizer + UndefinedBehaviorSanitizer, and
 * with ThreadSanitizer (the oracle splits rows over pthreads).  It calls
 * every entry point on small inputs, single-threaded and with several
 * threads, over all rows and over a row subset, plus the argument
 * rejections, and checks results that follow from the definitions alone:
 *   - attention over one key returns that key's value row, with LSE the one
 *     scaled logit;
 *   - causal attention of query row 0 sees key 0 only;
 *   - the row-subset call equals the same rows of the all-rows call, and the
 *     threaded calls equal the single-threaded ones;
 *   - RMSNorm + rotary with w = 1, cos = 1, sin = 0 leaves a row whose mean
 *     square is 1 / (1 + eps / mean(x^2));
 *   - merging with a side whose LSE is -inf returns the other side.
 * Exit status 0 when every check passes.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int oracle_attn(const uint16_t *q, const uint16_t *k, const uint16_t *v, int B, int H, int Sq, int Skv, int D,
                double scale, int causal, const int64_t *rows, int64_t n_rows, double *out, double *lse,
                int nthreads);
int oracle_qk_norm_rope(const uint16_t *x, const float *w, const float *cos_t, const float *sin_t, double eps,
                        int B, int H, int S, int D, double *out, int nthreads);
int oracle_merge(const double *out_a, const double *lse_a, const double *out_b, const double *lse_b,
                 int64_t rows, int D, double *out, double *lse);

static int failures = 0;

static void check(int ok, const char *what)
{
    if (!ok) {
        fprintf(stderr, "FAILED: %s\n", what);
        ++failures;
    }
}

/* bf16 bits of small exactly representable values: k/8 for |k| <= 64. */
static uint16_t bf16_of(double x)
{
    float f = (float)x;
    uint32_t u;
    memcpy(&u, &f, 4);
    return (uint16_t)(u >> 16);
}

static double bf16_val(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

static uint32_t lcg(uint32_t *s)
{
    *s = *s * 1664525u + 1013904223u;
    return *s >> 8;
}

static void fill(uint16_t *x, size_t n, uint32_t seed)
{
    for (size_t i = 0; i < n; ++i)
        x[i] = bf16_of(((int)(lcg(&seed) % 129) - 64) / 32.0);
}

static void test_attention(void)
{
    enum { B = 2, H = 2, Sq = 5, Skv = 7, D = 8 };
    const int n = B * H * Sq;
    uint16_t *q = malloc(sizeof(uint16_t) * B * H * Sq * D);
    uint16_t *k = malloc(sizeof(uint16_t) * B * H * Skv * D);
    uint16_t *v = malloc(sizeof(uint16_t) * B * H * Skv * D);
    double *o1 = malloc(sizeof(double) * n * D), *l1 = malloc(sizeof(double) * n);
    double *o3 = malloc(sizeof(double) * n * D), *l3 = malloc(sizeof(double) * n);
    fill(q, (size_t)B * H * Sq * D, 1);
    fill(k, (size_t)B * H * Skv * D, 2);
    fill(v, (size_t)B * H * Skv * D, 3);
    const double scale = 0.35;
    for (int causal = 0; causal < 2; ++causal) {
        check(oracle_attn(q, k, v, B, H, Sq, Skv, D, scale, causal, NULL, n, o1, l1, 1) == 0, "attn 1 thread");
        check(oracle_attn(q, k, v, B, H, Sq, Skv, D, scale, causal, NULL, n, o3, l3, 3) == 0, "attn 3 threads");
        check(memcmp(o1, o3, sizeof(double) * n * D) == 0 && memcmp(l1, l3, sizeof(double) * n) == 0,
              "threads give the same results");
        const int64_t rows[3] = {n - 1, 0, 7};
        double os[3 * D], ls[3];
        check(oracle_attn(q, k, v, B, H, Sq, Skv, D, scale, causal, rows, 3, os, ls, 2) == 0, "attn rows");
        for (int r = 0; r < 3; ++r)
            check(memcmp(os + r * D, o1 + rows[r] * D, sizeof(double) * D) == 0 && ls[r] == l1[rows[r]],
                  "row subset equals the same rows of the full call");
        if (causal) {
            /* Row 0 of each head sees key 0 only. */
            for (int bh = 0; bh < B * H; ++bh) {
                const uint16_t *qr = q + (size_t)bh * Sq * D, *kr = k + (size_t)bh * Skv * D;
                const uint16_t *vr = v + (size_t)bh * Skv * D;
                double dot = 0.0;
                for (int d = 0; d < D; ++d)
                    dot += bf16_val(qr[d]) * bf16_val(kr[d]);
                for (int d = 0; d < D; ++d)
                    check(o1[(size_t)bh * Sq * D + d] == bf16_val(vr[d]), "causal row 0 equals v[0]");
                check(fabs(l1[(size_t)bh * Sq] - scale * dot) <= 1e-12 * (1.0 + fabs(scale * dot)),
                      "causal row 0 LSE is the one scaled logit");
            }
        }
    }
    /* One key: out = v[0] exactly, lse = the scaled logit. */
    double o_one[D], l_one;
    const int64_t row0 = 0;
    check(oracle_attn(q, k, v, 1, 1, 1, 1, D, scale, 0, &row0, 1, o_one, &l_one, 1) == 0, "attn one key");
    for (int d = 0; d < D; ++d)
        check(o_one[d] == bf16_val(v[d]), "one key: out equals v");
    /* Rejections. */
    const int64_t bad = n;
    check(oracle_attn(NULL, k, v, B, H, Sq, Skv, D, scale, 0, NULL, n, o1, l1, 1) == -1, "NULL q rejected");
    check(oracle_attn(q, k, v, B, H, Sq, Skv, D, scale, 0, NULL, n - 1, o1, l1, 1) == -1, "row count rejected");
    check(oracle_attn(q, k, v, B, H, Sq, Skv, D, scale, 0, &bad, 1, o1, l1, 1) == -1, "row id rejected");
    free(q);
    free(k);
    free(v);
    free(o1);
    free(l1);
    free(o3);
    free(l3);
}

static void test_prologue(void)
{
    enum { B = 1, H = 3, S = 4, D = 16 };
    const int n = B * H * S * D;
    uint16_t *x = malloc(sizeof(uint16_t) * n);
    float w[D], cs[S * D], sn[S * D];
    double *y1 = malloc(sizeof(double) * n), *y4 = malloc(sizeof(double) * n);
    fill(x, (size_t)n, 4);
    for (int d = 0; d < D; ++d)
        w[d] = 1.0f;
    for (int i = 0; i < S * D; ++i) {
        cs[i] = 1.0f;
        sn[i] = 0.0f;
    }
    const double eps = 1e-3;
    check(oracle_qk_norm_rope(x, w, cs, sn, eps, B, H, S, D, y1, 1) == 0, "prologue 1 thread");
    check(oracle_qk_norm_rope(x, w, cs, sn, eps, B, H, S, D, y4, 4) == 0, "prologue 4 threads");
    check(memcmp(y1, y4, sizeof(double) * n) == 0, "prologue threads give the same results");
    for (int r = 0; r < B * H * S; ++r) {
        double ms_x = 0.0, ms_y = 0.0;
        for (int d = 0; d < D; ++d) {
            double a = bf16_val(x[r * D + d]);
            ms_x += a * a / D;
            ms_y += y1[r * D + d] * y1[r * D + d] / D;
        }
        check(fabs(ms_y - ms_x / (ms_x + eps)) <= 1e-12, "identity rotary: mean square of the RMSNorm row");
    }
    check(oracle_qk_norm_rope(x, w, cs, sn, eps, B, H, S, D - 1, y1, 1) == -1, "odd D rejected");
    free(x);
    free(y1);
    free(y4);
}

static void test_merge(void)
{
    enum { R = 3, D = 4 };
    double oa[R * D], ob[R * D], o[R * D];
    double la[R] = {0.5, -INFINITY, -INFINITY}, lb[R] = {-INFINITY, 1.25, -INFINITY}, l[R];
    for (int i = 0; i < R * D; ++i) {
        oa[i] = i * 0.25;
        ob[i] = -i * 0.5;
    }
    oa[D] = NAN;   /* row 1, side a is empty: its values must not matter */
    check(oracle_merge(oa, la, ob, lb, R, D, o, l) == 0, "merge");
    for (int d = 0; d < D; ++d) {
        check(o[d] == oa[d] && o[D + d] == ob[D + d] && o[2 * D + d] == 0.0, "merge with an empty side");
    }
    check(l[0] == la[0] && l[1] == lb[1] && l[2] == -INFINITY, "merged LSE with an empty side");
    check(oracle_merge(NULL, la, ob, lb, R, D, o, l) == -1, "merge NULL rejected");
}

int main(void)
{
    test_attention();
    test_prologue();
    test_merge();
    if (failures) {
        fprintf(stderr, "%d check(s) failed\n", failures);
        return 1;
    }
    printf("oracle sanitize checks passed\n");
    return 0;
}
