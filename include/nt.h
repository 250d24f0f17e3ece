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
