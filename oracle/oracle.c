/*
 * oracle.c -- plain, slow, fp64 CPU reference for the DiT attention hot path.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may call, link or
 * load this file; only the tests, the smoke check and the CPU-baseline leg of
 * the benchmark do.  It shares no code, header, table or helper with the GPU
 * library: it decodes bf16 itself, and it computes every result straight from
 * its definition in double precision, with no blocking, no fusion and no
 * online softmax.
 *
 * Sources (the pages the method is taken from):
 *  [COSMOS]  "Cosmos 昇腾 NPU 多卡并行优化说明" (Cosmos on Ascend NPU),
 *            §3.1 Flash Attention replacement, §3.2 RMSNorm, §3.3 Rotary.
 *  [WAN]     "NPU Wan2.2-I2V模型推理优化实践" (Wan2.2-I2V inference on NPU),
 *            sections on npu_fused_infer_attention_score, rotary_mul,
 *            rms_norm and Ring Attention Overlap.
 *  [PR274]   "feat: support Ascend NPU backend (torch_npu) for Qwen-Image
 *            pipelines - #274", change list item 2 (models/basic/attention.py)
 *            and the verification table.
 *
 * Pins: every function here is checked against closed forms, invariants and
 * torch CPU library routines by the CPU test suite (tests/test_oracle_*.py).
 *
 * Build: gcc -O2 -shared -fPIC -pthread oracle.c -lm  (no -ffast-math: the
 * summation order is the plain left-to-right order written below).
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* bf16 is the top half of an IEEE binary32; every bf16 value is exact in
 * double. */
static double bf16_value(uint16_t bits)
{
    uint32_t u = ((uint32_t)bits) << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* ------------------------------------------------------------------------ */
/* Row-parallel driver: splits [0, n) over nthreads plain pthreads.          */

typedef void (*row_fn)(void *ctx, int64_t first, int64_t last, double *scratch);

typedef struct {
    row_fn fn;
    void *ctx;
    int64_t first, last;
    size_t scratch_len;
    int failed;
} worker_arg;

static void *worker_main(void *p)
{
    worker_arg *a = (worker_arg *)p;
    double *scratch = NULL;
    if (a->scratch_len) {
        scratch = (double *)malloc(a->scratch_len * sizeof(double));
        if (!scratch) {
            a->failed = 1;
            return NULL;
        }
    }
    a->fn(a->ctx, a->first, a->last, scratch);
    free(scratch);
    return NULL;
}

static int run_rows(row_fn fn, void *ctx, int64_t n, size_t scratch_len, int nthreads)
{
    if (n <= 0)
        return 0;
    if (nthreads < 1)
        nthreads = 1;
    if (nthreads > 256)
        nthreads = 256;
    if ((int64_t)nthreads > n)
        nthreads = (int)n;
    pthread_t tid[256];
    worker_arg args[256];
    int started[256];
    int64_t per = n / nthreads, extra = n % nthreads, at = 0;
    int rc = 0;
    for (int t = 0; t < nthreads; ++t) {
        int64_t cnt = per + (t < extra ? 1 : 0);
        args[t].fn = fn;
        args[t].ctx = ctx;
        args[t].first = at;
        args[t].last = at + cnt;
        args[t].scratch_len = scratch_len;
        args[t].failed = 0;
        at += cnt;
        started[t] = (pthread_create(&tid[t], NULL, worker_main, &args[t]) == 0);
        if (!started[t])
            worker_main(&args[t]); /* run inline if a thread cannot start */
    }
    for (int t = 0; t < nthreads; ++t) {
        if (started[t])
            pthread_join(tid[t], NULL);
        if (args[t].failed)
            rc = -1;
    }
    return rc;
}

/* ------------------------------------------------------------------------ */
/* Attention: O_i = softmax_j(scale * q_i . k_j) V, LSE_i = ln sum_j exp(.)   */
/*
 * [COSMOS] §3.1 and [WAN] (npu_fused_infer_attention_score) call the fused
 * attention on BNSD tensors with an explicit softmax scale, no dropout, and a
 * switch between full (non-causal) attention and a causal mask; the Cosmos
 * SDPA form fixes the causal mask as key j visible to query i iff j <= i
 * (top-left aligned).  [WAN] "Ring Attention Overlap" and [PR274] item 2
 * (update_out_and_lse) rely on the per-row log-sum-exp of the scaled logits;
 * it is returned in natural-log units.
 *
 * Two passes per row, straight from the definition:
 *   s_j   = scale * sum_d q_d k_jd              for j in J(i)
 *   m     = max_j s_j
 *   l     = sum_j exp(s_j - m)
 *   O_d   = (1/l) sum_j exp(s_j - m) v_jd
 *   LSE   = m + ln l
 * with J(i) = {0..Skv-1}, or {j : j <= i} when causal.
 */
typedef struct {
    const uint16_t *q, *k, *v;
    int H, Sq, Skv, D, causal;
    double scale;
    const int64_t *rows;
    double *out, *lse;
} attn_ctx;

static void attn_rows(void *p, int64_t first, int64_t last, double *s)
{
    const attn_ctx *c = (const attn_ctx *)p;
    const int D = c->D;
    for (int64_t r = first; r < last; ++r) {
        int64_t row = c->rows ? c->rows[r] : r;         /* (b*H + h)*Sq + i */
        int64_t bh = row / c->Sq;
        int64_t i = row % c->Sq;
        const uint16_t *qi = c->q + row * (int64_t)D;
        const uint16_t *kb = c->k + bh * (int64_t)c->Skv * D;
        const uint16_t *vb = c->v + bh * (int64_t)c->Skv * D;
        int64_t nkeys = c->Skv;
        if (c->causal && i + 1 < nkeys)
            nkeys = i + 1;

        /* pass 1: logits and their maximum */
        double m = -INFINITY;
        for (int64_t j = 0; j < nkeys; ++j) {
            double dot = 0.0;
            for (int d = 0; d < D; ++d)
                dot += bf16_value(qi[d]) * bf16_value(kb[j * D + d]);
            s[j] = c->scale * dot;
            if (s[j] > m)
                m = s[j];
        }
        /* pass 2: softmax denominator, then the weighted sum of values */
        double l = 0.0;
        for (int64_t j = 0; j < nkeys; ++j) {
            s[j] = exp(s[j] - m);
            l += s[j];
        }
        double *o = c->out + r * (int64_t)D;
        for (int d = 0; d < D; ++d)
            o[d] = 0.0;
        for (int64_t j = 0; j < nkeys; ++j)
            for (int d = 0; d < D; ++d)
                o[d] += s[j] * bf16_value(vb[j * D + d]);
        for (int d = 0; d < D; ++d)
            o[d] /= l;
        if (c->lse)
            c->lse[r] = m + log(l);
    }
}

/*
 * q: [B,H,Sq,D] bf16 bits; k, v: [B,H,Skv,D] bf16 bits (contiguous BNSD).
 * rows: n_rows flat query-row ids (b*H + h)*Sq + i, or NULL for every row
 * (then n_rows must be B*H*Sq).  out: [n_rows, D] fp64; lse: [n_rows] fp64 or
 * NULL.  Returns 0, or -1 on a bad argument or allocation failure.
 */
int oracle_attn(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                int B, int H, int Sq, int Skv, int D, double scale, int causal,
                const int64_t *rows, int64_t n_rows,
                double *out, double *lse, int nthreads)
{
    if (!q || !k || !v || !out || B < 1 || H < 1 || Sq < 1 || Skv < 1 || D < 1)
        return -1;
    if (!rows && n_rows != (int64_t)B * H * Sq)
        return -1;
    if (rows)
        for (int64_t r = 0; r < n_rows; ++r)
            if (rows[r] < 0 || rows[r] >= (int64_t)B * H * Sq)
                return -1;
    attn_ctx c = {q, k, v, H, Sq, Skv, D, causal ? 1 : 0, scale, rows, out, lse};
    return run_rows(attn_rows, &c, n_rows, (size_t)Skv, nthreads);
}

/* ------------------------------------------------------------------------ */
/* Prologue: per-head RMSNorm, then interleaved rotary embedding.            */
/*
 * RMSNorm ([COSMOS] §3.2, [WAN] rms_norm section): over the head dimension D
 * of each (b,h,s) row,  r = sqrt(mean_d x_d^2 + eps),  y_d = (x_d / r) * w_d.
 * Interleaved rotary ([COSMOS] §3.3, [WAN] rotary_mul section, interleave
 * mode): adjacent pairs (2i, 2i+1) are rotated with the cos/sin tables taken
 * elementwise at the same (s, d):
 *   z_{2i}   = y_{2i}   cos[s,2i]   - y_{2i+1} sin[s,2i]
 *   z_{2i+1} = y_{2i+1} cos[s,2i+1] + y_{2i}   sin[s,2i+1]
 * No intermediate rounding: the result is left in fp64.
 */
typedef struct {
    const uint16_t *x;
    const float *w, *cs, *sn;
    double eps;
    int S, D;
    double *out;
} rope_ctx;

static void rope_rows(void *p, int64_t first, int64_t last, double *y)
{
    const rope_ctx *c = (const rope_ctx *)p;
    const int D = c->D;
    for (int64_t row = first; row < last; ++row) {
        int64_t s = row % c->S;
        const uint16_t *x = c->x + row * (int64_t)D;
        double ss = 0.0;
        for (int d = 0; d < D; ++d) {
            double xd = bf16_value(x[d]);
            ss += xd * xd;
        }
        double r = sqrt(ss / (double)D + c->eps);
        for (int d = 0; d < D; ++d)
            y[d] = bf16_value(x[d]) / r * (double)c->w[d];
        const float *cs = c->cs + s * (int64_t)D;
        const float *sn = c->sn + s * (int64_t)D;
        double *z = c->out + row * (int64_t)D;
        for (int i = 0; i < D / 2; ++i) {
            double a = y[2 * i], b = y[2 * i + 1];
            z[2 * i] = a * (double)cs[2 * i] - b * (double)sn[2 * i];
            z[2 * i + 1] = b * (double)cs[2 * i + 1] + a * (double)sn[2 * i + 1];
        }
    }
}

/*
 * x: [B,H,S,D] bf16 bits; w: [D] fp32; cos, sin: [S,D] fp32 (broadcast over
 * B and H); out: [B,H,S,D] fp64.  D must be even.  Returns 0 or -1.
 */
int oracle_qk_norm_rope(const uint16_t *x, const float *w, const float *cos_t,
                        const float *sin_t, double eps, int B, int H, int S, int D,
                        double *out, int nthreads)
{
    if (!x || !w || !cos_t || !sin_t || !out || B < 1 || H < 1 || S < 1 || D < 2 || (D & 1))
        return -1;
    rope_ctx c = {x, w, cos_t, sin_t, eps, S, D, out};
    return run_rows(rope_rows, &c, (int64_t)B * H * S, (size_t)D, nthreads);
}

/* ------------------------------------------------------------------------ */
/* Merge of two partial attentions over disjoint key sets.                   */
/*
 * [WAN] "Ring Attention Overlap" merges the local-KV and remote-KV attention
 * outputs with their log-sum-exp values; [PR274] item 2 names the same fold
 * (update_out_and_lse).  With a and b the partial results over key sets A
 * and B:
 *   M = max(la, lb),  L = M + ln(exp(la - M) + exp(lb - M))
 *   O = exp(la - L) O_a + exp(lb - L) O_b
 * which equals the attention over A u B.  A side whose LSE is -inf is the
 * attention over an empty key set (ln of an empty sum): it holds no key, so
 * it adds no term at all, whatever its output values are.  When both la and
 * lb are -inf the row saw no key: O = 0 and L = -inf.
 */
int oracle_merge(const double *out_a, const double *lse_a, const double *out_b,
                 const double *lse_b, int64_t rows, int D, double *out, double *lse)
{
    if (!out_a || !lse_a || !out_b || !lse_b || !out || !lse || rows < 0 || D < 1)
        return -1;
    for (int64_t r = 0; r < rows; ++r) {
        double la = lse_a[r], lb = lse_b[r];
        double M = la > lb ? la : lb;
        const double *oa = out_a + r * (int64_t)D;
        const double *ob = out_b + r * (int64_t)D;
        double *o = out + r * (int64_t)D;
        if (M == -INFINITY) {
            for (int d = 0; d < D; ++d)
                o[d] = 0.0;
            lse[r] = -INFINITY;
            continue;
        }
        int has_a = la != -INFINITY, has_b = lb != -INFINITY;
        double L = M + log(exp(la - M) + exp(lb - M));
        double wa = exp(la - L), wb = exp(lb - L);
        for (int d = 0; d < D; ++d) {
            double x = 0.0;
            if (has_a)
                x += wa * oa[d];
            if (has_b)
                x += wb * ob[d];
            o[d] = x;
        }
        lse[r] = L;
    }
    return 0;
}
