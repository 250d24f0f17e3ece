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
 *  - Calls are re-entrant and thread-safe.  Beyond the thread-local error
 *    message, the only global state is per-device launch information
 *    (device attributes, kernel LDS limits), set once under a lock.
 */
#ifndef NT_H
#define NT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define NT_ABI_VERSION 2

typedef enum {
    NT_OK = 0,
    NT_EINVAL = 1,
    NT_ESHAPE = 2,
    NT_EALIGN = 3,
    NT_ENOMEM = 4,
    NT_EHIP = 5,
    NT_ESTATE = 6,
    NT_ENODEV = 7,
    NT_EIO = 8
} nt_status;

/* Weight formats.  Ids are the GGUF type-field numbers.
 *   NT_Q8_0 : 34-byte blocks of 32 values, fp16 scale d + 32 int8 codes; x = d*q
 *   NT_Q4_0 : 18-byte blocks of 32 values, fp16 d + 16 bytes of 4-bit codes
 *             (byte i: value i in the low nibble, value i+16 in the high);
 *             x = d*(q-8)
 *   NT_Q4_K : 144-byte super-blocks of 256 values: fp16 d, fp16 dmin, 12 bytes
 *             of packed 6-bit sub-block scales S_j and mins M_j (j = 0..7),
 *             128 bytes of 4-bit codes; x = (d*S_j)*q - dmin*M_j
 *   NT_Q5_K : 176-byte super-blocks of 256 values: fp16 d, fp16 dmin, the
 *             same 12 scale/min bytes as Q4_K, 32 bytes qh, 128 bytes of
 *             low 4 bits laid out as in Q4_K; bit j of qh[l] is the fifth bit
 *             of value 32j + l, q in [0, 31]; x = (d*S_j)*q - dmin*M_j
 *   NT_Q6_K : 210-byte super-blocks of 256 values: 128 bytes of low 4 bits,
 *             64 bytes of high 2 bits, 16 int8 sub-block scales, fp16 d;
 *             x = d*scale[e/16]*(q-32)
 * (Layouts: the public GGUF block definitions; the write-up's "Overview"
 * names the formats.) */
typedef enum { NT_F32 = 0, NT_F16 = 1, NT_Q4_0 = 2, NT_Q8_0 = 8, NT_Q4_K = 12, NT_Q5_K = 13, NT_Q6_K = 14 } nt_qtype;

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
nt_status nt_dequant_q5_k(const void *blocks, float *out, int64_t n, nt_stream stream);
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
nt_status nt_gemv_q5_k(const void *W, const float *x, float *y, int64_t rows, int64_t cols,
                       int accumulate, nt_stream stream);
nt_status nt_gemv_q6_k(const void *W, const float *x, float *y, int64_t rows, int64_t cols,
                       int accumulate, nt_stream stream);
nt_status nt_gemv(nt_qtype t, const void *W, const float *x, float *y, int64_t rows, int64_t cols,
                  int accumulate, nt_stream stream);
/* The launch the GEMV calls above would use for this shape (no GPU needed):
 * info[0] = kernel family (2 = LDS-ring path copying 16-byte pieces, 1 = the
 * same with 4-byte pieces (rows only word-aligned), 0 = generic path),
 * info[1] = largest number of rows one workgroup reduces, info[2] =
 * workgroups, info[3] = threads per workgroup.  The LDS-ring path takes rows
 * whose byte length is a multiple of 4, cols % 64 == 0, cols <= 32768 and
 * rows * row_bytes below 2^32. */
nt_status nt_gemv_launch_info(nt_qtype t, int64_t rows, int64_t cols, int32_t info[4]);

/* Fused variants for the decode step (one launch where the step would make
 * several; each needs a shape the LDS-ring path takes, else NT_ESHAPE):
 *
 * nt_gemv_multi: for s in [0, nseg), nseg in 1..3, matrices of one format
 * and width,  y_s[r] = (accumulate ? y_s[r] : 0) + sum_c W_s[r][c] * n[c]
 * with n = x, or n = RMSNorm(x, gain, eps) as nt_rmsnorm defines it when gain
 * is not NULL (each workgroup forms 1/rms itself; nothing is written back).
 * W, rows, y are host arrays of nseg device pointers / row counts.  This is
 * the Llama block's q/k/v projection from the normalized residual.
 *
 * nt_gemv_swiglu: h[r] = silu(W_gate[r] . n) * (W_up[r] . n), r in [0, rows),
 * n as above: the block's gate and up projections with the SwiGLU
 * activation applied to the two row sums before they leave the kernel.
 *
 * x, gain, every W_s and y_s (h) 16-byte aligned device memory; outputs must
 * not overlap inputs. */
nt_status nt_gemv_multi(nt_qtype t, int32_t nseg, const void *const *W, const int64_t *rows, float *const *y,
                        int64_t cols, const float *x, const float *gain, float eps, int accumulate,
                        nt_stream stream);
nt_status nt_gemv_swiglu(nt_qtype t, const void *W_gate, const void *W_up, int64_t rows, int64_t cols,
                         const float *x, const float *gain, float eps, float *h, nt_stream stream);

/* ---- batched verify pass ("Overview": self-speculative decoding, where the
 * resident layers draft tokens and the whole model checks them in one pass) --
 * Y_n[r] = (Y_n[r] +) sum_c W[r, c] * X_n[c] for n in [0, k), r in [0, rows),
 * 1 <= k <= 8: every weight is read once for the k vectors.  X is k vectors of
 * cols fp32 back to back (X_n at X + n * cols), Y is k vectors of rows fp32
 * (Y_n at Y + n * rows); W is as for nt_gemv.  Types: the five block
 * formats (others: NT_EINVAL); cols a whole number of blocks, at most 65536;
 * rows below 2^31.  The products run on the matrix cores with each x split
 * into two fp16 parts (about 2^-22 relative error per element); weights are
 * not rounded.  Where a part would overflow fp16 (|x| near 65504 or above,
 * or, for the K-quant mins, a sum of 32 activations that large) the vectors
 * of that 256-column step are split scaled by an exact power of two and
 * their sums scaled back, so any finite X is valid.  The call runs one or
 * two kernels: for Q4_K, Q5_K and Q6_K on most shapes the main kernel forms
 * each step's split activations in on-chip memory itself; otherwise a first
 * kernel writes them to the workspace (8224 bytes per 256 columns, 8736 for
 * Q4_K and Q5_K) and the main one reads them.  When the columns are split
 * between workgroups (few rows), the partial sums also go to the workspace
 * and, per set of rows, the last wave to finish adds them in a fixed order
 * (results are deterministic; no wave waits for another), counted by the
 * counters in the workspace's first 16384 bytes.  workspace: device memory
 * of at least nt_gemm_batch_workspace_bytes(t, rows, cols) bytes (never 0
 * for valid arguments; 0 means the arguments are invalid), 16-byte
 * aligned, whose first 16384 bytes are zero before the first call that
 * uses it: every call leaves them zero again, the rest of the workspace
 * is used only during the call (stream order), so one zero-filled
 * workspace serves any sequence of calls (any shapes, graph replays) as
 * long as nothing else writes its first 16384 bytes.  Calls that share a
 * workspace must not overlap.  W, X and the workspace 16-byte aligned, Y
 * 4-byte aligned; Y must not overlap X, W or the workspace. */
size_t nt_gemm_batch_workspace_bytes(nt_qtype t, int64_t rows, int64_t cols);
nt_status nt_gemm_batch(nt_qtype t, const void *W, const float *X, float *Y, int64_t rows, int64_t cols,
                        int32_t k, int32_t accumulate, void *workspace, size_t workspace_bytes, nt_stream stream);

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
 * scale <= 0 means 1 / sqrt(head_dim).  rope_theta > 0 first rotates q and
 * k_new by RoPE at pos exactly as nt_rope would (q itself is not modified);
 * 0 uses them as given.  head_dim must be 64 or 128 and n_q_heads /
 * n_kv_heads one of 1, 2, 4, 8 (NT_ESHAPE).  workspace: device, 16-byte
 * aligned, at least nt_attn_workspace_bytes(desc) bytes (NT_ENOMEM).  q and
 * out 16-byte aligned.  A pos outside [0, ctx_cap) makes out NaN and writes
 * nothing to the cache. */
typedef struct {
    int32_t n_q_heads, n_kv_heads, head_dim, ctx_cap;
    float scale;
    float rope_theta;
} nt_attn_desc;
size_t    nt_attn_workspace_bytes(const nt_attn_desc *desc);
nt_status nt_attn_decode(const nt_attn_desc *desc, const float *q, const float *k_new, const float *v_new,
                         uint16_t *k_cache, uint16_t *v_cache, const int32_t *d_pos, float *out,
                         void *workspace, size_t workspace_bytes, nt_stream stream);

/* The same attention without a caller workspace, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation.  Arguments, results and errors as for
 * nt_attn_decode.  The partial results live in a fixed array of
 * NT_ATTN_NOALLOC_SCRATCH_BYTES bytes that the library keeps in each device's
 * memory until the process ends; its address is looked up (not allocated) on
 * the first call on a device, and no call allocates memory.  A shape whose
 * nt_attn_workspace_bytes exceeds the array returns NT_ENOMEM (use
 * nt_attn_decode).  Every call on one device shares that device's array:
 * calls ordered on one stream are safe, calls that overlap in time on one
 * device (other streams, other threads) race and give undefined results.
 * Nothing in the array needs to start at zero. */
#define NT_ATTN_NOALLOC_SCRATCH_BYTES (8u << 20)
nt_status nt_attn_decode_noalloc(const nt_attn_desc *desc, const float *q, const float *k_new,
                                 const float *v_new, uint16_t *k_cache, uint16_t *v_cache, const int32_t *d_pos,
                                 float *out, nt_stream stream);

/* ---- one batch-1 Llama decode step ("Main features": RoPE, GQA, SwiGLU,
 * RMSNorm, KV cache; "Architecture": engine, sampler) ------------------------
 * Per token, with pos = *d_pos and x the residual stream:
 *   x = row *d_token of tok_embd
 *   per layer: n = RMSNorm(x, attn_norm); q = Wq n, k = Wk n, v = Wv n;
 *              RoPE(q, k, pos); store k, v (fp16) at slot pos; o = Attn(q);
 *              x += Wo o; m = RMSNorm(x, ffn_norm); x += Wdown (silu(Wgate m) * Wup m)
 *   logits = Woutput RMSNorm(x, output_norm); *d_next = argmax(logits); ++*d_pos
 * Weight matrices are packed row-major blocks (any of the four formats, per
 * tensor); norm gains are fp32.  All pointers are device memory owned by the
 * caller and must outlive the model.  The model holds only host state, HIP
 * events and (when enabled) a captured HIP graph. */
typedef struct {
    int32_t n_layers, hidden, n_q_heads, n_kv_heads, head_dim, ffn, vocab, ctx_cap;
    float rms_eps, rope_theta;
} nt_model_config;

typedef struct {
    int32_t type;          /* nt_qtype */
    const void *data;      /* device, 16-byte aligned packed blocks */
} nt_tensor_ref;

typedef struct {
    const float *attn_norm;                    /* fp32[hidden] */
    nt_tensor_ref wq, wk, wv;                  /* [n_q_heads*head_dim | n_kv_heads*head_dim] x hidden */
    nt_tensor_ref wo;                          /* hidden x n_q_heads*head_dim */
    const float *ffn_norm;                     /* fp32[hidden] */
    nt_tensor_ref w_gate, w_up;                /* ffn x hidden */
    nt_tensor_ref w_down;                      /* hidden x ffn */
} nt_layer_weights;

typedef struct {
    nt_tensor_ref tok_embd;                    /* vocab x hidden */
    const float *output_norm;                  /* fp32[hidden] */
    nt_tensor_ref output;                      /* vocab x hidden */
    const nt_layer_weights *layers;            /* host array of n_layers entries, copied */
    uint16_t *k_cache, *v_cache;               /* fp16 bits [n_layers][n_kv_heads][ctx_cap][head_dim] */
    void *workspace;                           /* >= nt_model_workspace_bytes(cfg), 256-byte aligned */
    size_t workspace_bytes;
} nt_model_weights;

typedef struct nt_model nt_model;

/* Scratch the step needs (activations and attention partials); 0 if cfg is invalid. */
size_t nt_model_workspace_bytes(const nt_model_config *cfg);
/* Validates shapes (head_dim 64 or 128; n_q_heads / n_kv_heads in {1,2,4,8};
 * every matrix's column count a whole number of its blocks) and pointers.
 * Layer matrices may be NULL only for layers later served by nt_stream_layers. */
nt_status nt_model_create(const nt_model_config *cfg, const nt_model_weights *w, nt_model **out);
void      nt_model_destroy(nt_model *m);
/* enable != 0 (the default): the first resident step on a stream is captured
 * into a HIP graph that later steps replay (re-captured when the pointer
 * arguments change).  Steps on the NULL stream always run eagerly. */
nt_status nt_model_set_graph(nt_model *m, int enable);
/* Enqueues one decode step on `stream`.  d_token, d_pos: device int32
 * (d_next may equal d_token); logits: device fp32[vocab].  With token =
 * *d_token and pos = *d_pos read on the device: embed row `token`, run every
 * layer (k and v of this token stored at slot pos of each layer's cache,
 * attention over slots [0, pos]), the output RMSNorm and head into logits,
 * then *d_next = argmax(logits) (lowest index on ties, a NaN never wins, 0
 * when every logit is NaN) and *d_pos = pos + 1.  Out-of-range values live on
 * the device, so no status reports them: a token outside [0, vocab) gives
 * NaN logits and token 0 (slot pos then holds NaN k and v); a pos outside
 * [0, ctx_cap) gives NaN logits and token 0 and writes nothing to the cache.
 * In both cases the position still advances. */
nt_status nt_decode_step(nt_model *m, const int32_t *d_token, int32_t *d_pos, float *logits,
                         int32_t *d_next, nt_stream stream);

/* ---- host-streamed layers ("Performance": 3-tier cache with VRAM-resident
 * layers and pinned-RAM layers copied host-to-device; "Main features":
 * double-buffered streaming that overlaps transfer and compute) -------------
 * A layer blob packs one layer's seven matrices back to back in the order
 * wq, wk, wv, wo, w_gate, w_up, w_down, each starting on a 256-byte boundary;
 * types[7] gives their formats. */
nt_status nt_layer_blob_layout(const nt_model_config *cfg, const int32_t types[7], size_t offsets[7],
                               size_t *blob_bytes);
typedef struct {
    int32_t first_streamed_layer;              /* layers [first, n_layers) are streamed */
    const void *const *h_layer_blobs;          /* host array: one pinned blob per streamed layer */
    void *d_buf[2];                            /* device staging buffers, each >= buf_bytes */
    size_t buf_bytes;                          /* >= the blob size */
    nt_stream copy_stream;                     /* side stream for host-to-device copies */
} nt_stream_desc;
/* Streamed layers take their matrix types from the model's layer weights of
 * the first streamed layer (all streamed layers must share them).  Each step
 * then copies blob j into d_buf[j % 2] on copy_stream, and layer j waits for
 * its copy while the next blob is already in flight.  desc == NULL returns
 * to fully resident operation (all layer matrices must then be set). */
nt_status nt_stream_layers(nt_model *m, const nt_stream_desc *desc);
typedef struct {
    uint64_t steps, layers_streamed, h2d_bytes;  /* totals since streaming was enabled */
    double copy_ms, compute_ms, wall_ms;         /* last step: copy-stream busy time, time
                                                    of the streamed layers' compute, step wall */
} nt_stream_stats;
/* Waits for the last step, then reports. */
nt_status nt_stream_stats_get(nt_model *m, nt_stream_stats *out);

/* ---- the third tier: layers read from a file ("Performance": a 3-tier
 * cache of VRAM-resident layers, pinned-RAM layers copied host-to-device, and
 * an NVMe/mmap fallback; "Main features": the data path is chosen VRAM, then
 * pinned host RAM, then the fallback; "NVMe direct streaming": the data
 * flows disk -> pinned staging -> host-to-device copy -> GPU buffer ->
 * compute) ---------------------------------------------------------------
 * As nt_stream_layers, with the streamed layers split in two: layers
 * [first_streamed_layer, first_file_layer) come from desc->h_layer_blobs
 * (first_file_layer - first_streamed_layer pinned blobs), layers
 * [first_file_layer, n_layers) from the file: the blob of layer
 * first_file_layer + j (nt_layer_blob_layout order) starts at byte
 * offset + j * stride of `path`.  Every step reads each file blob into
 * h_staging[j % 2] on a reader thread of the library and only once that
 * read has finished enqueues its host-to-device copy into d_buf and its
 * layer's compute: the GPU never waits on the host, so a failed read cannot
 * stall the device.  With `direct` set and a file system that allows it the
 * file is opened with O_DIRECT (reads bypass the page cache); since a direct
 * read cannot target HIP-pinned memory, each 32 MiB chunk lands in one of two
 * library-owned bounce buffers (64 MiB of ordinary host memory, allocated
 * here and freed with the tier) and is copied into the staging buffer while
 * the next chunk is read.  Otherwise reads go through the page cache
 * straight into the staging buffer.  nt_decode_step then
 * returns after the last file read of the step has finished (it blocks on
 * the reads), and a failed or short read makes it return NT_EIO: the step's
 * later layers, the head and the position update are not enqueued, so
 * logits, *d_next and *d_pos are not valid for that step.
 * Requirements: offset and stride multiples of 4096, stride >= the blob
 * size; the file at least offset + (count - 1) * stride + blob bytes long
 * (NT_EINVAL otherwise; a file that cannot be opened is NT_EIO); h_staging
 * two pinned host buffers (hipHostMalloc), 4096-byte aligned, each at least
 * staging_bytes >= the blob size rounded up to 4096 (each read is that long;
 * the bytes past the blob are ignored).  file == NULL is nt_stream_layers. */
typedef struct {
    const char *path;
    int32_t first_file_layer;
    uint64_t offset, stride;
    void *h_staging[2];
    size_t staging_bytes;
    int32_t direct;
} nt_file_tier;
nt_status nt_stream_layers_tiered(nt_model *m, const nt_stream_desc *desc, const nt_file_tier *file);
typedef struct {
    uint64_t reads, read_bytes;   /* totals since the file tier was enabled */
    double read_ms;               /* last step: summed duration of its file reads */
    double read_span_ms;          /* last step: first read's start to last read's end */
    int32_t direct;               /* 1: the file was opened with O_DIRECT (reads bypass the page cache) */
    int32_t file_layers;
} nt_file_stats;
/* Reports the file reads of the last step (complete once nt_decode_step returned). */
nt_status nt_file_stats_get(nt_model *m, nt_file_stats *out);
/* The data-path choice as plain arithmetic: with every layer's blob the size
 * nt_layer_blob_layout gives for `types`, the first floor(vram_bytes / blob)
 * layers stay resident, the next floor(pinned_bytes / blob) are pinned, the
 * rest come from the file (each count capped by the layers left). */
nt_status nt_tier_plan(const nt_model_config *cfg, const int32_t types[7], uint64_t vram_bytes,
                       uint64_t pinned_bytes, int32_t *first_streamed, int32_t *first_file);

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
 *   Q5_K: as Q4_K with 31 in place of 15 (q in [0, 31])
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
 * aligned, bytes a multiple of 16). */
nt_status nt_read_bytes(const void *src, int64_t bytes, float *sink, nt_stream stream);
nt_status nt_copy_bytes(void *dst, const void *src, int64_t bytes, nt_stream stream);

/* ---- GGUF model files ("Overview": the engine loads GGUF models) -----------
 * Host-side reader of the GGUF v2/v3 container: the file is mapped read-only
 * and parsed with every read bounds-checked (a truncated or malformed file
 * returns NT_EINVAL with a message, never reads past the mapping).  Tensor
 * data stays in the mapping: `data` pointers are host addresses valid until
 * nt_gguf_close; copy them to the device to build an nt_model (the Llama
 * tensor names are token_embd.weight, output_norm.weight, output.weight and
 * blk.<i>.{attn_norm, attn_q, attn_k, attn_v, attn_output, ffn_norm,
 * ffn_gate, ffn_up, ffn_down}.weight).  No GGUF file from another tool is
 * available to this library's tests, so compatibility with such files is
 * checked against the published format only. */
typedef struct nt_gguf nt_gguf;
nt_status nt_gguf_open(const char *path, nt_gguf **out);
void      nt_gguf_close(nt_gguf *g);
int64_t   nt_gguf_tensor_count(const nt_gguf *g);            /* -1 for NULL */
int64_t   nt_gguf_find_tensor(const nt_gguf *g, const char *name);   /* index or -1 */
/* Tensor i: name (valid until close), type (the GGUF/ggml type id; the
 * nt_qtype values are the same ids), rows x cols (cols = the fastest
 * dimension, rows = the product of the others), host data and its size.
 * NT_ESHAPE (data NULL) for a type whose size this library does not know. */
nt_status nt_gguf_tensor_info(const nt_gguf *g, int64_t i, const char **name, int32_t *type, int64_t *rows,
                              int64_t *cols, const void **data, size_t *bytes);
/* The decode configuration of a Llama model file from its llama.* keys and
 * token_embd.weight (vocab = its rows); ctx_cap > 0 sets the KV capacity,
 * 0 takes llama.context_length.  head_dim = llama.attention.key_length, or
 * hidden / head_count when that key is absent (llama.attention.value_length,
 * when stored, must equal it: NT_ESHAPE otherwise); rope_theta defaults to
 * 10000 and head_count_kv to head_count. */
nt_status nt_gguf_llama_config(const nt_gguf *g, int32_t ctx_cap, nt_model_config *cfg);

#ifdef __cplusplus
}
#endif
#endif
