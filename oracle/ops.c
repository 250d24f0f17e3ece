/*
 * ops.c -- the fp64 operations of one Llama decode step.  Test
 * infrastructure only.
 *
 * Source: the ntransformer write-up (GeekNews topic 26894).  "Architecture"
 * lists the engine's GPU kernels (GEMV, RMSNorm, RoPE, SwiGLU, softmax);
 * "Main features" lists the Llama pieces (RoPE, GQA, SwiGLU, RMSNorm, KV
 * cache); "Roadmap" says the KV cache is F16.  The pages give no formulas.
 * Each function below is the usual textbook definition, with the readings
 * where the pages are silent stated at the function.
 */
#include "oracle.h"

#include <math.h>
#include <pthread.h>
#include <stdlib.h>
#include <string.h>

/* ---- GEMV ------------------------------------------------------------------
 * y[r] = sum_c w[r][c] * x[c] over the decoded fp32 weights, in fp64, c in
 * increasing order.  The "Architecture" section's GEMV kernel: batch-1 decode
 * multiplies every weight matrix by one activation vector. */

typedef struct {
    int type;
    const uint8_t *W;
    int64_t cols, row_bytes;
    const double *x;
    const int64_t *ids;    /* NULL: row i is row i                           */
    int64_t lo, hi;        /* output positions [lo, hi)                      */
    double *y;
    int err;
} gemv_job;

static void *gemv_worker(void *arg)
{
    gemv_job *j = (gemv_job *)arg;
    float *w = (float *)malloc(sizeof(float) * (size_t)(j->cols > 0 ? j->cols : 1));
    if (!w) {
        j->err = -3;
        return NULL;
    }
    for (int64_t i = j->lo; i < j->hi; ++i) {
        int64_t r = j->ids ? j->ids[i] : i;
        if (or_dequant(j->type, j->W + r * j->row_bytes, j->cols, w) != 0) {
            j->err = -1;
            break;
        }
        double acc = 0.0;
        for (int64_t c = 0; c < j->cols; ++c)
            acc += (double)w[c] * j->x[c];
        j->y[i] = acc;
    }
    free(w);
    return NULL;
}

static int gemv_common(int type, const uint8_t *W, int64_t rows, int64_t cols,
                       const double *x, const int64_t *ids, int64_t n_out, double *y,
                       int nthreads)
{
    int64_t rb = or_row_bytes(type, cols);
    if (rb < 0 || rows < 0 || n_out < 0)
        return -1;
    if (ids)
        for (int64_t i = 0; i < n_out; ++i)
            if (ids[i] < 0 || ids[i] >= rows)
                return -1;
    if (nthreads < 1)
        nthreads = 1;
    if (nthreads > 256)
        nthreads = 256;
    if ((int64_t)nthreads > n_out)
        nthreads = n_out > 0 ? (int)n_out : 1;
    gemv_job jobs[256];
    pthread_t tid[256];
    for (int t = 0; t < nthreads; ++t) {
        jobs[t] = (gemv_job){type, W, cols, rb, x, ids,
                             n_out * t / nthreads, n_out * (t + 1) / nthreads, y, 0};
    }
    if (nthreads == 1) {
        gemv_worker(&jobs[0]);
    } else {
        for (int t = 0; t < nthreads; ++t)
            pthread_create(&tid[t], NULL, gemv_worker, &jobs[t]);
        for (int t = 0; t < nthreads; ++t)
            pthread_join(tid[t], NULL);
    }
    for (int t = 0; t < nthreads; ++t)
        if (jobs[t].err)
            return jobs[t].err;
    return 0;
}

int or_gemv(int type, const uint8_t *W, int64_t rows, int64_t cols, const double *x,
            double *y, int nthreads)
{
    return gemv_common(type, W, rows, cols, x, NULL, rows, y, nthreads);
}

int or_gemv_rows(int type, const uint8_t *W, int64_t rows, int64_t cols, const double *x,
                 const int64_t *row_ids, int64_t n_ids, double *y, int nthreads)
{
    return gemv_common(type, W, rows, cols, x, row_ids, n_ids, y, nthreads);
}

/* ---- RMSNorm ----------------------------------------------------------------
 * y_i = g_i * x_i / sqrt(mean(x^2) + eps).  Reading: eps inside the root (the
 * Llama convention; the pages only name RMSNorm). */
void or_rmsnorm(const double *x, const double *g, int64_t n, double eps, double *y)
{
    double ss = 0.0;
    for (int64_t i = 0; i < n; ++i)
        ss += x[i] * x[i];
    double inv = 1.0 / sqrt(ss / (double)n + eps);
    for (int64_t i = 0; i < n; ++i)
        y[i] = g[i] * (x[i] * inv);
}

/* ---- RoPE -------------------------------------------------------------------
 * Rotary position embedding.  Reading: adjacent pairs (v[2i], v[2i+1]) of a
 * head are rotated by the angle pos * theta^(-2i/head_dim); no frequency
 * rescaling (the pages only name RoPE; theta comes from the workload). */
void or_rope(double *v, int n_heads, int head_dim, int64_t pos, double theta)
{
    for (int h = 0; h < n_heads; ++h) {
        double *hv = v + (int64_t)h * head_dim;
        for (int i = 0; i < head_dim / 2; ++i) {
            double w = pow(theta, -2.0 * i / head_dim);
            double phi = (double)pos * w;
            double c = cos(phi), s = sin(phi);
            double a = hv[2 * i], b = hv[2 * i + 1];
            hv[2 * i] = a * c - b * s;
            hv[2 * i + 1] = a * s + b * c;
        }
    }
}

/* ---- softmax: p_t = exp(s_t - max s) / sum exp(s - max s) ---------------- */
void or_softmax(const double *s, int64_t n, double *p)
{
    if (n <= 0)
        return;
    double mx = s[0];
    for (int64_t t = 1; t < n; ++t)
        mx = fmax(mx, s[t]);
    double sum = 0.0;
    for (int64_t t = 0; t < n; ++t) {
        p[t] = exp(s[t] - mx);
        sum += p[t];
    }
    for (int64_t t = 0; t < n; ++t)
        p[t] /= sum;
}

/* ---- SwiGLU: silu(g) * u, silu(a) = a / (1 + exp(-a)) --------------------- */
double or_silu(double a) { return a / (1.0 + exp(-a)); }

void or_swiglu(const double *gate, const double *up, int64_t n, double *out)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = or_silu(gate[i]) * up[i];
}

/* ---- greedy pick: argmax, the lowest index wins ties ---------------------- */
int64_t or_argmax(const double *v, int64_t n)
{
    int64_t best = 0;
    for (int64_t i = 1; i < n; ++i)
        if (v[i] > v[best])
            best = i;
    return best;
}

/* ---- GQA decode attention over the fp16 KV cache ---------------------------
 * The current token's k and v are stored first (rounded to fp16), then
 * q head h attends to slots [0, pos] of kv head g = h / (n_q / n_kv):
 * s_t = scale * <q_h, k_{g,t}>, p = softmax(s), o_h = sum_t p_t v_{g,t}.
 * Readings: contiguous head groups; scale 1/sqrt(head_dim); the current token
 * attends to itself. */
int or_attention(const double *q, const double *k_new, const double *v_new,
                 uint16_t *k_cache, uint16_t *v_cache, int n_q_heads, int n_kv_heads,
                 int head_dim, int64_t ctx_cap, int64_t pos, double scale, double *out)
{
    if (n_q_heads <= 0 || n_kv_heads <= 0 || n_q_heads % n_kv_heads != 0 || head_dim <= 0 ||
        pos < 0 || pos >= ctx_cap)
        return -1;
    if (scale <= 0.0)
        scale = 1.0 / sqrt((double)head_dim);
    int group = n_q_heads / n_kv_heads;
    for (int g = 0; g < n_kv_heads; ++g)
        for (int d = 0; d < head_dim; ++d) {
            int64_t at = ((int64_t)g * ctx_cap + pos) * head_dim + d;
            k_cache[at] = or_f64_to_f16_rne(k_new[g * head_dim + d]);
            v_cache[at] = or_f64_to_f16_rne(v_new[g * head_dim + d]);
        }
    int64_t n = pos + 1;
    double *s = (double *)malloc(sizeof(double) * (size_t)n);
    double *p = (double *)malloc(sizeof(double) * (size_t)n);
    if (!s || !p) {
        free(s);
        free(p);
        return -3;
    }
    for (int h = 0; h < n_q_heads; ++h) {
        int g = h / group;
        const double *qh = q + (int64_t)h * head_dim;
        for (int64_t t = 0; t < n; ++t) {
            const uint16_t *kt = k_cache + ((int64_t)g * ctx_cap + t) * head_dim;
            double dot = 0.0;
            for (int d = 0; d < head_dim; ++d)
                dot += qh[d] * or_f16_to_f64(kt[d]);
            s[t] = dot * scale;
        }
        or_softmax(s, n, p);
        for (int d = 0; d < head_dim; ++d) {
            double acc = 0.0;
            for (int64_t t = 0; t < n; ++t)
                acc += p[t] * or_f16_to_f64(v_cache[((int64_t)g * ctx_cap + t) * head_dim + d]);
            out[(int64_t)h * head_dim + d] = acc;
        }
    }
    free(s);
    free(p);
    return 0;
}
