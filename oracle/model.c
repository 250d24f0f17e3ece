/*
 * model.c -- one batch-1 Llama decode step in fp64.  Test infrastructure
 * only.
 *
 * Source: the ntransformer write-up (GeekNews topic 26894).  "Main features"
 * lists the Llama block (RoPE, GQA, SwiGLU, RMSNorm, KV cache);
 * "Architecture" puts the transformer config, attention, FFN and
 * normalization under model/ and the sampler and engine under inference/;
 * "Roadmap" reports batch-1 decode of Llama 8B Q8_0 and the F16 KV cache.
 * Readings where the pages are silent: pre-norm residual blocks in the usual
 * Llama order (below), no biases, greedy argmax sampling, the embedding row
 * decoded from the quantized token-embedding matrix.
 *
 *   x = embedding row `token`
 *   per layer: n = RMSNorm(x, g_attn); q, k, v = Wq n, Wk n, Wv n;
 *              RoPE(q, k, pos); store k, v at slot pos; o = Attn(q)
 *              x += Wo o
 *              m = RMSNorm(x, g_ffn); x += Wdown (silu(Wgate m) * Wup m)
 *   logits = Wout RMSNorm(x, g_out); next = argmax(logits)
 */
#include "oracle.h"

#include <stdlib.h>
#include <string.h>

static void f32_to_f64(const float *a, int64_t n, double *out)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = (double)a[i];
}

int or_decode_step(const or_config *cfg, const or_model *m, uint16_t *kv_k, uint16_t *kv_v,
                   int32_t token, int64_t pos, double *logits, int32_t *next, int nthreads)
{
    const int64_t H = cfg->hidden, D = cfg->head_dim, F = cfg->ffn, V = cfg->vocab;
    const int64_t QD = (int64_t)cfg->n_q_heads * D, KD = (int64_t)cfg->n_kv_heads * D;
    if (token < 0 || token >= V || pos < 0 || pos >= cfg->ctx_cap || cfg->n_kv_heads <= 0 ||
        cfg->n_q_heads % cfg->n_kv_heads != 0)
        return -1;

    double *x = calloc((size_t)H, sizeof(double)), *n = calloc((size_t)H, sizeof(double));
    double *q = calloc((size_t)QD, sizeof(double)), *k = calloc((size_t)KD, sizeof(double));
    double *v = calloc((size_t)KD, sizeof(double)), *o = calloc((size_t)QD, sizeof(double));
    double *g = calloc((size_t)F, sizeof(double)), *u = calloc((size_t)F, sizeof(double));
    double *hmid = calloc((size_t)F, sizeof(double)), *gain = calloc((size_t)H, sizeof(double));
    double *tmp = calloc((size_t)(H > QD ? H : QD), sizeof(double));
    double *lg = logits ? logits : calloc((size_t)V, sizeof(double));
    float *row = calloc((size_t)H, sizeof(float));
    int rc = -3;
    if (!x || !n || !q || !k || !v || !o || !g || !u || !hmid || !gain || !tmp || !lg || !row)
        goto done;

    /* embedding: decode row `token` of the token-embedding matrix */
    int64_t erb = or_row_bytes(m->tok_embd.type, H);
    if (erb < 0 || or_dequant(m->tok_embd.type, m->tok_embd.data + token * erb, H, row) != 0) {
        rc = -1;
        goto done;
    }
    f32_to_f64(row, H, x);

    const int64_t layer_kv = (int64_t)cfg->n_kv_heads * cfg->ctx_cap * D;
    for (int l = 0; l < cfg->n_layers; ++l) {
        const or_layer *L = &m->layers[l];
        /* attention block */
        f32_to_f64(L->attn_norm, H, gain);
        or_rmsnorm(x, gain, H, cfg->rms_eps, n);
        if ((rc = or_gemv(L->wq.type, L->wq.data, QD, H, n, q, nthreads)) != 0 ||
            (rc = or_gemv(L->wk.type, L->wk.data, KD, H, n, k, nthreads)) != 0 ||
            (rc = or_gemv(L->wv.type, L->wv.data, KD, H, n, v, nthreads)) != 0)
            goto done;
        or_rope(q, cfg->n_q_heads, (int)D, pos, cfg->rope_theta);
        or_rope(k, cfg->n_kv_heads, (int)D, pos, cfg->rope_theta);
        if ((rc = or_attention(q, k, v, kv_k + l * layer_kv, kv_v + l * layer_kv, cfg->n_q_heads,
                               cfg->n_kv_heads, (int)D, cfg->ctx_cap, pos, 0.0, o)) != 0)
            goto done;
        if ((rc = or_gemv(L->wo.type, L->wo.data, H, QD, o, tmp, nthreads)) != 0)
            goto done;
        for (int64_t i = 0; i < H; ++i)
            x[i] += tmp[i];
        /* feed-forward block */
        f32_to_f64(L->ffn_norm, H, gain);
        or_rmsnorm(x, gain, H, cfg->rms_eps, n);
        if ((rc = or_gemv(L->w_gate.type, L->w_gate.data, F, H, n, g, nthreads)) != 0 ||
            (rc = or_gemv(L->w_up.type, L->w_up.data, F, H, n, u, nthreads)) != 0)
            goto done;
        or_swiglu(g, u, F, hmid);
        if ((rc = or_gemv(L->w_down.type, L->w_down.data, H, F, hmid, tmp, nthreads)) != 0)
            goto done;
        for (int64_t i = 0; i < H; ++i)
            x[i] += tmp[i];
    }
    /* output head and greedy pick */
    f32_to_f64(m->output_norm, H, gain);
    or_rmsnorm(x, gain, H, cfg->rms_eps, n);
    if ((rc = or_gemv(m->output.type, m->output.data, V, H, n, lg, nthreads)) != 0)
        goto done;
    if (next)
        *next = (int32_t)or_argmax(lg, V);
    rc = 0;
done:
    free(x); free(n); free(q); free(k); free(v); free(o); free(g); free(u);
    free(hmid); free(gain); free(tmp); free(row);
    if (!logits)
        free(lg);
    return rc;
}
