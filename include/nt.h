/*
 * nt.h -- C ABI of libnt: quantized batch-1 Llama decode on MI355X (gfx950).
 *
 * The problem these calls solve is the one the ntransformer write-up
 * (GeekNews topic 26894) describes: a Llama decode step over GGUF-style
 * block-quantized weights ("Overview": Q4_0, Q8_0, Q4_K_M, Q5_K, Q6_K, F16,
 * F32), made of GEMV, RMSNorm, RoPE, SwiGLU and softmax kernels
 * ("Architecture") around GQA attention over an F16 KV cache ("Main
 * features", "Roadmap"), with layers either resident in GPU memory or
 * streamed from pinned host RAM ("Performance", 3-tier cache).  The pages
 * plan a public C API ("Roadmap", phase 5) but print no signatures; the
 * signatures here are this library's own.
 *
 * Conventions (every call):
 *  - Pointers marked "device" are device (HBM) addresses, "host" are host
 *    addresses.  All memory is owned by the caller; the library never frees
 *    caller memory and per-call functions allocate nothing.
 *  - Work is enqueued on `stream` (a hipStream_t; NULL = the default stream)
 *    and is complete when that stream is synchronized.  Inputs must stay
 *    alive and unmodified until then.
 *  - Argument errors are reported before anything is enqueued: NT_EINVAL
 *    (null pointer, unknown enum, negative size), NT_ESHAPE (sizes that do
 *    not fit the block format or the kernel's limits), NT_EALIGN (a pointer
 *    that breaks its stated alignment).  A failed launch returns NT_EHIP.
 *    NT_ENODEV means no usable GPU.  nt_last_error() then holds a
 *    thread-local message.  Faults inside a kernel surface at the caller's
 *    synchronization.
 *  - Packed-block buffers: blocks are stored back to back, little-endian, row
 *    after row.  The buffer's start must be 16-byte aligned and it must be
 *    readable up to the next multiple of 4 bytes past its last block (kernels
 *    read whole aligned 32-bit words; every allocator that rounds sizes to 4
 *    bytes or more, including hipMalloc and torch, satisfies this).
 *  - Calls are re-entrant; no global state is written except the
 *    thread-local error message.
 */
#ifndef NT_H
#define NT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define NT_ABI_VERSION 1

typedef enum {
    NT_OK = 0,
    NT_EINVAL = 1,
    NT_ESHAPE = 2,
    NT_EALIGN = 3,
    NT_ENOMEM = 4,
    NT_EHIP = 5,
    NT_ESTATE = 6,
    NT_ENODEV = 7
} nt_status;

/* Weight formats.  Ids are the GGUF type-field numbers.
 *   NT_Q8_0 : 34-byte blocks of 32 values, fp16 scale d + 32 int8 codes; x = d*q
 *   NT_Q4_0 : 18-byte blocks of 32 values, fp16 d + 16 bytes of 4-bit codes
 *             (byte i: value i in the low nibble, value i+16 in the high);
 *             x = d*(q-8)
 *   NT_Q4_K : 144-byte super-blocks of 256 values: fp16 d, fp16 dmin, 12 bytes
 *             of packed 6-bit sub-block scales S_j and mins M_j (j = 0..7),
 *             128 bytes of 4-bit codes; x = (d*S_j)*q - dmin*M_j
 *   NT_Q6_K : 210-byte super-blocks of 256 values: 128 bytes of low 4 bits,
 *             64 bytes of high 2 bits, 16 int8 sub-block scales, fp16 d;
 *             x = d*scale[e/16]*(q-32)
 * (Layouts: the public GGUF block definitions; the write-up's "Overview"
 * names the formats.) */
typedef enum { NT_F32 = 0, NT_F16 = 1, NT_Q4_0 = 2, NT_Q8_0 = 8, NT_Q4_K = 12, NT_Q6_K = 14 } nt_qtype;

typedef void *nt_stream; /* hipStream_t */

int         nt_abi_version(void);
const char *nt_status_str(nt_status s);
const char *nt_last_error(void);     /* thread-local; "" when none */

/* Block geometry; -1 for an unknown type or a column count that is not a
 * whole number of blocks. */
int64_t nt_qtype_block_elems(nt_qtype t);
int64_t nt_qtype_block_bytes(nt_qtype t);
int64_t nt_qtype_row_bytes(nt_qtype t, int64_t cols);

/* ---- dequantize ------------------------------------------------------------
 * out[e] = value of element e, e in [0, n), formed exactly and rounded once
 * to fp32 (every format's products are exact in fp32, so the result is the
 * correctly rounded value).
 * blocks: device, packed blocks (see conventions); out: device fp32[n],
 * 4-byte aligned.  n must be a multiple of the block size (NT_ESHAPE). */
nt_status nt_dequant_q8_0(const void *blocks, float *out, int64_t n, nt_stream stream);
nt_status nt_dequant_q4_0(const void *blocks, float *out, int64_t n, nt_stream stream);
nt_status nt_dequant_q4_k(const void *blocks, float *out, int64_t n, nt_stream stream);
nt_status nt_dequant_q6_k(const void *blocks, float *out, int64_t n, nt_stream stream);
nt_status nt_dequant(nt_qtype t, const void *blocks, float *out, int64_t n, nt_stream stream);

/* ---- fused dequantize-GEMV (the write-up's "Architecture": GEMV kernels) ---
 * y[r] = (accumulate ? y[r] : 0) + sum_c W[r][c] * x[c],  r in [0, rows)
 * W: device, rows x cols packed row-major (row r starts at
 *    W + r * nt_qtype_row_bytes(t, cols)); x: device fp32[cols]; y: device
 *    fp32[rows].  x and y 16-byte aligned; y must not overlap W or x.
 * cols must be a whole number of blocks and at most 65536 (NT_ESHAPE).
 * Arithmetic: weights decoded in registers, fp32 products and fp32 sums in a
 * fixed order (results are deterministic run to run). */
nt_status nt_gemv_q8_0(const void *W, const float *x, float *y, int64_t rows, int64_t cols,
                       int accumulate, nt_stream stream);
nt_status nt_gemv_q4_0(const void *W, const float *x, float *y, int64_t rows, int64_t cols,
                       int accumulate, nt_stream stream);
nt_status nt_gemv_q4_k(const void *W, const float *x, float *y, int64_t rows, int64_t cols,
                       int accumulate, nt_stream stream);
nt_status nt_gemv_q6_k(const void *W, const float *x, float *y, int64_t rows, int64_t cols,
                       int accumulate, nt_stream stream);
nt_status nt_gemv(nt_qtype t, const void *W, const float *x, float *y, int64_t rows, int64_t cols,
                  int accumulate, nt_stream stream);

/* ---- per-token ops ("Architecture": RMSNorm, RoPE, SwiGLU, softmax kernels;
 * "Main features": the Llama block) --------------------------------------
 * All buffers are device fp32 unless stated, 4-byte aligned, and may not
 * overlap unless stated.  Reductions run in a fixed order (deterministic). */

/* y[i] = gain[i] * x[i] / sqrt(sum_j x[j]^2 / n + eps), i in [0, n).  y may equal x. */
nt_status nt_rmsnorm(const float *x, const float *gain, float *y, int64_t n, float eps, nt_stream stream);

/* Rotary embedding in place on q (n_q_heads * head_dim values) and k
 * (n_kv_heads * head_dim; k may be NULL when n_kv_heads == 0): the adjacent
 * pair (v[2i], v[2i+1]) of every head turns by angle pos * theta^(-2i/head_dim),
 * pos = *d_pos (device int32).  head_dim even.  The angle is formed in fp64. */
nt_status nt_rope(float *q, float *k, int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim,
                  const int32_t *d_pos, float theta, nt_stream stream);

/* In place: x[t] <- exp(x[t] - max x) / sum_u exp(x[u] - max x), t in [0, n). */
nt_status nt_softmax(float *x, int64_t n, nt_stream stream);

/* out[i] = silu(gate[i]) * up[i], silu(a) = a / (1 + exp(-a)).  out may equal gate or up. */
nt_status nt_swiglu(const float *gate, const float *up, float *out, int64_t n, nt_stream stream);

/* *out (device int32) = index of the largest x[i], the lowest index on ties;
 * NaNs never win against numbers.  1 <= n < 2^31. */
nt_status nt_argmax(const float *x, int64_t n, int32_t *out, nt_stream stream);

/* out[0, hidden) = decoded row *d_token of the packed [vocab x hidden] table
 * (device, 16-byte aligned, format t).  A token outside [0, vocab) yields NaN
 * values (nothing is read out of bounds). */
nt_status nt_embed(nt_qtype t, const void *table, int64_t vocab, int64_t hidden, const int32_t *d_token,
                   float *out, nt_stream stream);

/* ---- decode attention over the fp16 KV cache ("Main features": GQA, KV cache;
 * "Roadmap": F16 KV cache) ------------------------------------------------
 * One layer's cache: k_cache and v_cache are device fp16 bit patterns laid out
 * [n_kv_heads][ctx_cap][head_dim], 16-byte aligned.  With pos = *d_pos:
 *   1. k_new, v_new (device fp32, n_kv_heads * head_dim) are rounded to fp16
 *      and stored at slot pos (skipped when k_new and v_new are NULL: the
 *      caller has stored them already);
 *   2. q head h (of n_q_heads, q device fp32) attends to slots [0, pos] of kv
 *      head h / (n_q_heads / n_kv_heads):  s_t = scale * <q_h, k_t>,
 *      out_h = sum_t softmax(s)_t * v_t   (out: device fp32, n_q_heads * head_dim).
 * scale <= 0 means 1 / sqrt(head_dim).  head_dim must be 64 or 128 and
 * n_q_heads / n_kv_heads one of 1, 2, 4, 8 (NT_ESHAPE).  workspace: device,
 * 16-byte aligned, at least nt_attn_workspace_bytes(desc) bytes (NT_ENOMEM).
 * A pos outside [0, ctx_cap) makes out NaN and writes nothing to the cache. */
typedef struct {
    int32_t n_q_heads, n_kv_heads, head_dim, ctx_cap;
    float scale;
} nt_attn_desc;
size_t    nt_attn_workspace_bytes(const nt_attn_desc *desc);
nt_status nt_attn_decode(const nt_attn_desc *desc, const float *q, const float *k_new, const float *v_new,
                         uint16_t *k_cache, uint16_t *v_cache, const int32_t *d_pos, float *out,
                         void *workspace, size_t workspace_bytes, nt_stream stream);

/* ---- encode (quantize) -------------------------------------------------------
 * blocks <- encoding of x[0, n) (device fp32, 4-byte aligned) into packed
 * blocks (device, 16-byte aligned, n / block_elems * block_bytes bytes).
 * n must be a multiple of the block size.  The encoder is the plain one with
 * error at most half a quantization step per value, computed in fp64 with
 * every operation rounded as written ("round" = half away from zero):
 *   Q8_0: d = fp16_rne(max|x|/127), q = clamp(round(x/d), -127, 127)
 *   Q4_0: d = fp16_rne(max|x|/7),   q = clamp(round(x/d), -8, 7) + 8
 *   Q4_K: per 32-value sub-block, m = -min(0, min x), dmin = fp16_up(max m/63),
 *         M = ceil(m/dmin), o = dmin*M, s = (max(max x, -o) + o)/15,
 *         d = fp16_up(max s/63), S = ceil(s/d), q = clamp(round((x+o)/(d*S)), 0, 15)
 *   Q6_K: per 16-value sub-block, s = max|x|/31, d = fp16_up(max s/127),
 *         S = ceil(s/d), q = clamp(round(x/(d*S)), -32, 31) + 32
 * (fp16_up(v) = the smallest fp16 >= v.)  The pages read GGUF files encoded
 * offline and give no encoder; this one serves to build synthetic models in
 * device memory.  Non-finite inputs give unspecified (but in-bounds) blocks. */
nt_status nt_quantize(nt_qtype t, const float *x, void *blocks, int64_t n, nt_stream stream);

/* ---- bandwidth calibration (measurement aid, not part of decode) -----------
 * nt_read_bytes: streams `bytes` bytes from `src` (device, 16-byte aligned,
 * bytes a multiple of 16) with 128-bit non-temporal loads and folds them into
 * a value whose (practically never taken) store into `sink` (device, >= 4096
 * floats) keeps the reads from being elided.
 * nt_copy_bytes: plain device-to-device copy of `bytes` bytes (both 16-byte
 * aligned, bytes a multiple of 16).
 * nt_delay: occupies `stream` for `microseconds` (0..1e6) with one spinning
 * wave, so a host can queue work behind it and time kernels back to back. */
nt_status nt_read_bytes(const void *src, int64_t bytes, float *sink, nt_stream stream);
nt_status nt_copy_bytes(void *dst, const void *src, int64_t bytes, nt_stream stream);
nt_status nt_delay(double microseconds, nt_stream stream);

#ifdef __cplusplus
}
#endif
#endif
