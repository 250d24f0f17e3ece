/*
 * oracle.h -- plain, slow CPU reference for quantized batch-1 Llama decode.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, loads or
 * calls this code; only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg may.  It shares no source with the HIP path.
 *
 * What it follows: the ntransformer write-up (GeekNews topic 26894; the same
 * post in Spanish, Vietnamese and Turkish).  Its "Overview" names the weight
 * formats the engine reads (Q4_0, Q8_0, Q4_K_M, Q5_K, Q6_K, F16, F32 inside
 * GGUF files); its "Main features" list the Llama pieces of one decode step
 * (RoPE, GQA, SwiGLU, RMSNorm, KV cache); its "Architecture" section names
 * the GEMV, RMSNorm, RoPE, SwiGLU and softmax kernels; its "Roadmap" adds the
 * F16 KV cache.  The pages give no byte layouts and no formulas, so every
 * layout and formula below is the plain reading stated beside it (the public
 * GGUF block definitions; the usual Llama formulas), and each such reading is
 * listed in the design notes.
 *
 * Arithmetic: fp64 everywhere except where the definition stores a narrower
 * value (fp16 block scales, the fp16 KV cache, fp32 dequantized weights).
 * All functions are single-threaded except where an nthreads argument says
 * otherwise; threading only splits independent output rows, each row is
 * summed by one thread in a fixed order, so results never depend on nthreads.
 *
 * Errors: functions returning int return 0 on success and a negative value on
 * bad arguments (unknown type, size not a multiple of the block, non-finite
 * quantizer input).
 */
#ifndef NT_ORACLE_H
#define NT_ORACLE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Block type ids (the GGUF type-field numbering). */
enum { OR_F32 = 0, OR_F16 = 1, OR_Q4_0 = 2, OR_Q8_0 = 8, OR_Q4_K = 12, OR_Q5_K = 13, OR_Q6_K = 14 };

/* ---- IEEE binary16 by bit manipulation ---------------------------------- */
double   or_f16_to_f64(uint16_t h);
uint16_t or_f64_to_f16_rne(double v);   /* round to nearest, ties to even   */
uint16_t or_f64_to_f16_up(double v);    /* smallest fp16 >= v, for v >= 0   */

/* ---- block formats ------------------------------------------------------- */
int64_t or_block_elems(int type);       /* 32 or 256; 1 for F32/F16; -1 bad */
int64_t or_block_bytes(int type);       /* 34, 18, 144, 210; 4 / 2          */
int64_t or_row_bytes(int type, int64_t cols);  /* -1 if cols % block != 0   */

/* Decode n elements (n a multiple of the block size) of packed blocks into
 * fp32.  Each value is formed exactly in fp64 and rounded once to fp32. */
int or_dequant(int type, const uint8_t *blocks, int64_t n, float *out);

/* Encode n fp32 values into packed blocks (the oracle's own quantizer). */
int or_quantize(int type, const float *x, int64_t n, uint8_t *blocks);

/* Pack Q8_0 blocks from separate scale bits and int8 codes (layout only). */
int or_pack_q8_0(const uint16_t *d_bits, const int8_t *qs, int64_t nblocks,
                 uint8_t *blocks);

/* ---- ops in fp64 ---------------------------------------------------------- */
/* y[r] = sum_c dequant(W)[r][c] * x[c], rows split over nthreads threads.    */
int or_gemv(int type, const uint8_t *W, int64_t rows, int64_t cols,
            const double *x, double *y, int nthreads);
/* Same, only for the listed rows (row_ids[i] -> y[i]).                       */
int or_gemv_rows(int type, const uint8_t *W, int64_t rows, int64_t cols,
                 const double *x, const int64_t *row_ids, int64_t n_ids,
                 double *y, int nthreads);

void    or_rmsnorm(const double *x, const double *g, int64_t n, double eps,
                   double *y);
/* Rotate adjacent pairs (v[2i], v[2i+1]) of each head in place by pos*w_i,
 * w_i = theta^(-2i/head_dim).  v holds n_heads * head_dim values.            */
void    or_rope(double *v, int n_heads, int head_dim, int64_t pos, double theta);
void    or_softmax(const double *s, int64_t n, double *p);
double  or_silu(double a);
void    or_swiglu(const double *gate, const double *up, int64_t n, double *out);
int64_t or_argmax(const double *v, int64_t n);   /* lowest index on ties */

/* One decode-attention call over an fp16 cache laid out
 * [n_kv_heads][ctx_cap][head_dim] (bits).  Writes k_new, v_new (rounded to
 * fp16) at slot pos, then attends over slots [0, pos].  q head h reads kv
 * head h / (n_q_heads / n_kv_heads).  scale <= 0 means 1/sqrt(head_dim).     */
int or_attention(const double *q, const double *k_new, const double *v_new,
                 uint16_t *k_cache, uint16_t *v_cache, int n_q_heads,
                 int n_kv_heads, int head_dim, int64_t ctx_cap, int64_t pos,
                 double scale, double *out);

/* ---- whole decode step ---------------------------------------------------- */
typedef struct {
    int32_t n_layers, hidden, n_q_heads, n_kv_heads, head_dim, ffn, vocab;
    int64_t ctx_cap;
    double  rms_eps, rope_theta;
} or_config;

typedef struct { int type; const uint8_t *data; } or_tensor;   /* host bytes */

typedef struct {
    const float *attn_norm;                  /* fp32[hidden]                  */
    or_tensor    wq, wk, wv, wo;             /* [q_dim x hidden] ...          */
    const float *ffn_norm;                   /* fp32[hidden]                  */
    or_tensor    w_gate, w_up, w_down;       /* [ffn x hidden] x2, [hidden x ffn] */
} or_layer;

typedef struct {
    or_tensor       tok_embd;                /* [vocab x hidden]              */
    const float    *output_norm;             /* fp32[hidden]                  */
    or_tensor       output;                  /* [vocab x hidden]              */
    const or_layer *layers;                  /* n_layers entries              */
} or_model;

/* kv_k / kv_v: [n_layers][n_kv_heads][ctx_cap][head_dim] fp16 bits, updated
 * in place at slot pos.  logits: double[vocab] (may be NULL).               */
int or_decode_step(const or_config *cfg, const or_model *m, uint16_t *kv_k,
                   uint16_t *kv_v, int32_t token, int64_t pos, double *logits,
                   int32_t *next, int nthreads);

#ifdef __cplusplus
}
#endif
#endif
