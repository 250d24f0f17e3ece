// abi.cpp -- the C-ABI entry points of libnt: argument validation, error
// reporting and dispatch to the HIP launchers.  Validation happens before any
// HIP call, so argument errors are reported the same way with or without a
// GPU.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <string>

#include "nt_internal.h"

namespace nt {

static thread_local std::string g_last_error;

void set_error(const std::string &msg) { g_last_error = msg; }

nt_status fail(nt_status s, const std::string &msg) {
    set_error(msg);
    return s;
}

nt_status check_launch(const char *what) {
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(NT_EHIP, std::string(what) + ": " + hipGetErrorString(e));
    return NT_OK;
}

int64_t block_elems(nt_qtype t) {
    switch (t) {
    case NT_F32: case NT_F16: return 1;
    case NT_Q8_0: case NT_Q4_0: return 32;
    case NT_Q4_K: case NT_Q5_K: case NT_Q6_K: return 256;
    }
    return -1;
}

int64_t block_bytes(nt_qtype t) {
    switch (t) {
    case NT_F32: return 4;
    case NT_F16: return 2;
    case NT_Q8_0: return 34;
    case NT_Q4_0: return 18;
    case NT_Q4_K: return 144;
    case NT_Q5_K: return 176;
    case NT_Q6_K: return 210;
    }
    return -1;
}

bool is_quant(nt_qtype t) {
    return t == NT_Q8_0 || t == NT_Q4_0 || t == NT_Q4_K || t == NT_Q5_K || t == NT_Q6_K;
}

// Device presence, checked after argument validation.
static nt_status need_device() {
    int n = 0;
    hipError_t e = hipGetDeviceCount(&n);
    if (e != hipSuccess || n <= 0) {
        (void)hipGetLastError();
        return fail(NT_ENODEV, "no HIP device available");
    }
    return NT_OK;
}

static nt_status finish(hipError_t e, const char *what) {
    if (e != hipSuccess) {
        (void)hipGetLastError();
        return fail(NT_EHIP, std::string(what) + ": " + hipGetErrorString(e));
    }
    return check_launch(what);
}

static const char *qname(nt_qtype t) {
    switch (t) {
    case NT_Q8_0: return "q8_0";
    case NT_Q4_0: return "q4_0";
    case NT_Q4_K: return "q4_k";
    case NT_Q5_K: return "q5_k";
    case NT_Q6_K: return "q6_k";
    case NT_F32: return "f32";
    case NT_F16: return "f16";
    }
    return "?";
}

}  // namespace nt

using namespace nt;

extern "C" {

int nt_abi_version(void) { return NT_ABI_VERSION; }

const char *nt_status_str(nt_status s) {
    switch (s) {
    case NT_OK: return "NT_OK";
    case NT_EINVAL: return "NT_EINVAL: invalid argument";
    case NT_ESHAPE: return "NT_ESHAPE: size does not fit the format or kernel limits";
    case NT_EALIGN: return "NT_EALIGN: misaligned pointer";
    case NT_ENOMEM: return "NT_ENOMEM: buffer too small";
    case NT_EHIP: return "NT_EHIP: HIP runtime error";
    case NT_ESTATE: return "NT_ESTATE: call not valid in the current state";
    case NT_ENODEV: return "NT_ENODEV: no GPU device";
    case NT_EIO: return "NT_EIO: file read failed";
    }
    return "unknown nt_status";
}

const char *nt_last_error(void) { return g_last_error.c_str(); }

int64_t nt_qtype_block_elems(nt_qtype t) { return block_elems(t); }
int64_t nt_qtype_block_bytes(nt_qtype t) { return block_bytes(t); }

int64_t nt_qtype_row_bytes(nt_qtype t, int64_t cols) {
    int64_t be = block_elems(t);
    if (be <= 0 || cols < 0 || cols % be != 0) return -1;
    return cols / be * block_bytes(t);
}

// ---- dequant ------------------------------------------------------------------
nt_status nt_dequant(nt_qtype t, const void *blocks, float *out, int64_t n, nt_stream stream) {
    set_error("");
    if (!is_quant(t)) return fail(NT_EINVAL, "nt_dequant: unsupported type");
    if (n < 0) return fail(NT_EINVAL, "nt_dequant: negative n");
    if (n % block_elems(t) != 0)
        return fail(NT_ESHAPE, std::string("nt_dequant_") + qname(t) + ": n is not a multiple of the block size");
    if (n == 0) return NT_OK;
    if (!blocks || !out) return fail(NT_EINVAL, "nt_dequant: null pointer");
    if (!aligned(blocks, 16)) return fail(NT_EALIGN, "nt_dequant: blocks not 16-byte aligned");
    if (!aligned(out, 4)) return fail(NT_EALIGN, "nt_dequant: out not 4-byte aligned");
    if (nt_status s = need_device()) return s;
    return finish(launch_dequant(t, blocks, out, n, as_stream(stream)), "nt_dequant");
}

nt_status nt_dequant_q8_0(const void *b, float *o, int64_t n, nt_stream s) { return nt_dequant(NT_Q8_0, b, o, n, s); }
nt_status nt_dequant_q4_0(const void *b, float *o, int64_t n, nt_stream s) { return nt_dequant(NT_Q4_0, b, o, n, s); }
nt_status nt_dequant_q4_k(const void *b, float *o, int64_t n, nt_stream s) { return nt_dequant(NT_Q4_K, b, o, n, s); }
nt_status nt_dequant_q5_k(const void *b, float *o, int64_t n, nt_stream s) { return nt_dequant(NT_Q5_K, b, o, n, s); }
nt_status nt_dequant_q6_k(const void *b, float *o, int64_t n, nt_stream s) { return nt_dequant(NT_Q6_K, b, o, n, s); }

// ---- GEMV ------------------------------------------------------------------------
nt_status nt_gemv(nt_qtype t, const void *W, const float *x, float *y, int64_t rows, int64_t cols,
                  int accumulate, nt_stream stream) {
    set_error("");
    if (!is_quant(t)) return fail(NT_EINVAL, "nt_gemv: unsupported type");
    if (rows < 0 || cols < 0) return fail(NT_EINVAL, "nt_gemv: negative size");
    if (cols % block_elems(t) != 0)
        return fail(NT_ESHAPE, std::string("nt_gemv_") + qname(t) + ": cols is not a multiple of the block size");
    if (cols > kMaxGemvCols) return fail(NT_ESHAPE, "nt_gemv: cols above 65536");
    if (rows > (int64_t)1 << 31) return fail(NT_ESHAPE, "nt_gemv: rows above 2^31");
    if (rows == 0) return NT_OK;
    if (!W || !x || !y) return fail(NT_EINVAL, "nt_gemv: null pointer");
    if (!aligned(W, 16) || !aligned(x, 16) || !aligned(y, 16))
        return fail(NT_EALIGN, "nt_gemv: W, x and y must be 16-byte aligned");
    if (nt_status s = need_device()) return s;
    return finish(launch_gemv(t, W, x, y, rows, cols, accumulate, as_stream(stream)), "nt_gemv");
}

nt_status nt_gemv_launch_info(nt_qtype t, int64_t rows, int64_t cols, int32_t info[4]) {
    set_error("");
    if (!info) return fail(NT_EINVAL, "nt_gemv_launch_info: null pointer");
    if (!is_quant(t)) return fail(NT_EINVAL, "nt_gemv_launch_info: unsupported type");
    if (rows <= 0 || cols <= 0 || cols % block_elems(t) != 0 || cols > kMaxGemvCols)
        return fail(NT_ESHAPE, "nt_gemv_launch_info: bad shape");
    gemv_launch_info(t, rows, cols, info);
    return NT_OK;
}

nt_status nt_gemv_multi(nt_qtype t, int32_t nseg, const void *const *W, const int64_t *rows, float *const *y,
                        int64_t cols, const float *x, const float *gain, float eps, int accumulate,
                        nt_stream stream) {
    set_error("");
    if (!is_quant(t)) return fail(NT_EINVAL, "nt_gemv_multi: unsupported type");
    if (nseg < 1 || nseg > 3) return fail(NT_EINVAL, "nt_gemv_multi: nseg must be 1, 2 or 3");
    if (!W || !rows || !y) return fail(NT_EINVAL, "nt_gemv_multi: null array");
    if (cols <= 0 || cols % block_elems(t) != 0) return fail(NT_ESHAPE, "nt_gemv_multi: cols not a whole number of blocks");
    if (!(eps >= 0.f)) return fail(NT_EINVAL, "nt_gemv_multi: negative eps");
    int64_t total = 0;
    for (int s = 0; s < nseg; ++s) {
        if (rows[s] < 0) return fail(NT_EINVAL, "nt_gemv_multi: negative rows");
        total += rows[s];
        if (!W[s] || !y[s]) return fail(NT_EINVAL, "nt_gemv_multi: null pointer");
        if (!aligned(W[s], 16) || !aligned(y[s], 16)) return fail(NT_EALIGN, "nt_gemv_multi: W and y must be 16-byte aligned");
        if (rows[s] > 0 && !gemv_fast_ok(t, rows[s], cols))
            return fail(NT_ESHAPE, "nt_gemv_multi: shape not taken by the fused kernels (word-aligned rows, "
                                   "cols % 64 == 0, cols <= 32768, rows * row_bytes < 2^32)");
    }
    if (total > (int64_t(1) << 31) - 1) return fail(NT_ESHAPE, "nt_gemv_multi: more than 2^31 rows");
    if (!x) return fail(NT_EINVAL, "nt_gemv_multi: null x");
    if (!aligned(x, 16) || !aligned(gain, 16)) return fail(NT_EALIGN, "nt_gemv_multi: x and gain must be 16-byte aligned");
    if (total == 0) return NT_OK;
    if (nt_status s = need_device()) return s;
    // drop empty matrices (the kernel assumes every listed matrix has rows)
    const void *Wk[3];
    int64_t rk[3];
    float *yk[3];
    int k = 0;
    for (int s = 0; s < nseg; ++s)
        if (rows[s] > 0) { Wk[k] = W[s]; rk[k] = rows[s]; yk[k] = y[s]; ++k; }
    return finish(launch_gemv_multi(t, k, Wk, rk, yk, cols, x, gain, eps, accumulate, as_stream(stream)),
                  "nt_gemv_multi");
}

nt_status nt_gemv_swiglu(nt_qtype t, const void *W_gate, const void *W_up, int64_t rows, int64_t cols,
                         const float *x, const float *gain, float eps, float *h, nt_stream stream) {
    set_error("");
    if (!is_quant(t)) return fail(NT_EINVAL, "nt_gemv_swiglu: unsupported type");
    if (rows < 0) return fail(NT_EINVAL, "nt_gemv_swiglu: negative rows");
    if (cols <= 0 || cols % block_elems(t) != 0) return fail(NT_ESHAPE, "nt_gemv_swiglu: cols not a whole number of blocks");
    if (!(eps >= 0.f)) return fail(NT_EINVAL, "nt_gemv_swiglu: negative eps");
    if (rows > (int64_t(1) << 30)) return fail(NT_ESHAPE, "nt_gemv_swiglu: more than 2^30 rows");
    if (rows > 0 && !gemv_fast_ok(t, rows, cols))
        return fail(NT_ESHAPE, "nt_gemv_swiglu: shape not taken by the fused kernels (word-aligned rows, "
                               "cols % 64 == 0, cols <= 32768, rows * row_bytes < 2^32)");
    if (!W_gate || !W_up || !x || !h) return fail(NT_EINVAL, "nt_gemv_swiglu: null pointer");
    if (!aligned(W_gate, 16) || !aligned(W_up, 16) || !aligned(x, 16) || !aligned(gain, 16) || !aligned(h, 16))
        return fail(NT_EALIGN, "nt_gemv_swiglu: W_gate, W_up, x, gain and h must be 16-byte aligned");
    if (rows == 0) return NT_OK;
    if (nt_status s = need_device()) return s;
    return finish(launch_gemv_swiglu(t, W_gate, W_up, rows, cols, x, gain, eps, h, as_stream(stream)),
                  "nt_gemv_swiglu");
}

#define NT_GEMV_FN(name, T)                                                                       \
    nt_status name(const void *W, const float *x, float *y, int64_t rows, int64_t cols, int acc,  \
                   nt_stream s) {                                                                 \
        return nt_gemv(T, W, x, y, rows, cols, acc, s);                                           \
    }
NT_GEMV_FN(nt_gemv_q8_0, NT_Q8_0)
NT_GEMV_FN(nt_gemv_q4_0, NT_Q4_0)
NT_GEMV_FN(nt_gemv_q4_k, NT_Q4_K)
NT_GEMV_FN(nt_gemv_q5_k, NT_Q5_K)
NT_GEMV_FN(nt_gemv_q6_k, NT_Q6_K)

// ---- batched verify pass ------------------------------------------------------------
size_t nt_gemm_batch_workspace_bytes(nt_qtype t, int64_t rows, int64_t cols) {
    if (!gemm_batch_type_ok(t) || rows < 0 || rows > (int64_t(1) << 31) - 1 || cols <= 0 || cols > kMaxGemvCols ||
        cols % block_elems(t) != 0)
        return 0;
    return gemm_batch_workspace_bytes(t, rows, cols);
}

nt_status nt_gemm_batch(nt_qtype t, const void *W, const float *X, float *Y, int64_t rows, int64_t cols,
                        int32_t k, int32_t accumulate, void *workspace, size_t workspace_bytes, nt_stream stream) {
    set_error("");
    if (!gemm_batch_type_ok(t)) return fail(NT_EINVAL, "nt_gemm_batch: not a block-quantized type");
    if (k < 1 || k > 8) return fail(NT_EINVAL, "nt_gemm_batch: k must be 1..8");
    if (rows < 0 || cols <= 0) return fail(NT_EINVAL, "nt_gemm_batch: rows < 0 or cols <= 0");
    if (cols % block_elems(t) != 0) return fail(NT_ESHAPE, "nt_gemm_batch: cols not a whole number of blocks");
    if (cols > kMaxGemvCols) return fail(NT_ESHAPE, "nt_gemm_batch: cols above 65536");
    if (rows > (int64_t(1) << 31) - 1) return fail(NT_ESHAPE, "nt_gemm_batch: rows above 2^31 - 1");
    if (rows == 0) return NT_OK;
    const size_t need = gemm_batch_workspace_bytes(t, rows, cols);
    if (!W || !X || !Y || (need > 0 && !workspace)) return fail(NT_EINVAL, "nt_gemm_batch: null pointer");
    if (!aligned(W, 16) || !aligned(X, 16) || !aligned(workspace, 16) || !aligned(Y, 4))
        return fail(NT_EALIGN, "nt_gemm_batch: W, X and workspace 16-byte aligned, Y 4-byte aligned");
    if (workspace_bytes < need)
        return fail(NT_ENOMEM, "nt_gemm_batch: workspace smaller than nt_gemm_batch_workspace_bytes");
    if (nt_status s = need_device()) return s;
    return finish(launch_gemm_batch(t, W, rows, cols, X, k, Y, accumulate, workspace, as_stream(stream)),
                  "nt_gemm_batch");
}
#undef NT_GEMV_FN

// ---- per-token ops ---------------------------------------------------------------
#define NT_REQ(cond, st, msg) \
    do {                      \
        if (!(cond)) return fail(st, msg); \
    } while (0)

nt_status nt_rmsnorm(const float *x, const float *gain, float *y, int64_t n, float eps, nt_stream stream) {
    set_error("");
    NT_REQ(n >= 0, NT_EINVAL, "nt_rmsnorm: negative n");
    if (n == 0) return NT_OK;
    NT_REQ(x && gain && y, NT_EINVAL, "nt_rmsnorm: null pointer");
    NT_REQ(aligned(x, 4) && aligned(gain, 4) && aligned(y, 4), NT_EALIGN, "nt_rmsnorm: misaligned");
    NT_REQ(eps >= 0.f, NT_EINVAL, "nt_rmsnorm: negative eps");
    if (nt_status s = need_device()) return s;
    return finish(launch_rmsnorm(x, gain, y, n, eps, as_stream(stream)), "nt_rmsnorm");
}

nt_status nt_rope(float *q, float *k, int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim,
                  const int32_t *d_pos, float theta, nt_stream stream) {
    set_error("");
    NT_REQ(n_q_heads >= 0 && n_kv_heads >= 0 && head_dim > 0, NT_EINVAL, "nt_rope: bad sizes");
    NT_REQ(head_dim % 2 == 0, NT_ESHAPE, "nt_rope: head_dim must be even");
    NT_REQ(theta > 0.f, NT_EINVAL, "nt_rope: theta must be positive");
    if (n_q_heads + n_kv_heads == 0) return NT_OK;
    NT_REQ(d_pos && (q || n_q_heads == 0) && (k || n_kv_heads == 0), NT_EINVAL, "nt_rope: null pointer");
    NT_REQ(aligned(q, 4) && aligned(k, 4) && aligned(d_pos, 4), NT_EALIGN, "nt_rope: misaligned");
    if (nt_status s = need_device()) return s;
    return finish(launch_rope(q, k, n_q_heads, n_kv_heads, head_dim, d_pos, theta, as_stream(stream)), "nt_rope");
}

nt_status nt_softmax(float *x, int64_t n, nt_stream stream) {
    set_error("");
    NT_REQ(n >= 0, NT_EINVAL, "nt_softmax: negative n");
    if (n == 0) return NT_OK;
    NT_REQ(x, NT_EINVAL, "nt_softmax: null pointer");
    NT_REQ(aligned(x, 4), NT_EALIGN, "nt_softmax: misaligned");
    if (nt_status s = need_device()) return s;
    return finish(launch_softmax(x, n, as_stream(stream)), "nt_softmax");
}

nt_status nt_swiglu(const float *gate, const float *up, float *out, int64_t n, nt_stream stream) {
    set_error("");
    NT_REQ(n >= 0, NT_EINVAL, "nt_swiglu: negative n");
    if (n == 0) return NT_OK;
    NT_REQ(gate && up && out, NT_EINVAL, "nt_swiglu: null pointer");
    NT_REQ(aligned(gate, 4) && aligned(up, 4) && aligned(out, 4), NT_EALIGN, "nt_swiglu: misaligned");
    if (nt_status s = need_device()) return s;
    return finish(launch_swiglu(gate, up, out, n, as_stream(stream)), "nt_swiglu");
}

nt_status nt_argmax(const float *x, int64_t n, int32_t *out, nt_stream stream) {
    set_error("");
    NT_REQ(n >= 1 && n < (int64_t(1) << 31), NT_EINVAL, "nt_argmax: need 1 <= n < 2^31");
    NT_REQ(x && out, NT_EINVAL, "nt_argmax: null pointer");
    NT_REQ(aligned(x, 4) && aligned(out, 4), NT_EALIGN, "nt_argmax: misaligned");
    if (nt_status s = need_device()) return s;
    return finish(launch_argmax(x, n, out, nullptr, as_stream(stream)), "nt_argmax");
}

nt_status nt_embed(nt_qtype t, const void *table, int64_t vocab, int64_t hidden, const int32_t *d_token,
                   float *out, nt_stream stream) {
    set_error("");
    NT_REQ(is_quant(t), NT_EINVAL, "nt_embed: unsupported type");
    NT_REQ(vocab > 0 && hidden >= 0 && vocab < (int64_t(1) << 31), NT_EINVAL, "nt_embed: bad sizes");
    NT_REQ(hidden % block_elems(t) == 0, NT_ESHAPE, "nt_embed: hidden is not a multiple of the block size");
    if (hidden == 0) return NT_OK;
    NT_REQ(table && d_token && out, NT_EINVAL, "nt_embed: null pointer");
    NT_REQ(aligned(table, 16) && aligned(d_token, 4) && aligned(out, 4), NT_EALIGN, "nt_embed: misaligned");
    if (nt_status s = need_device()) return s;
    return finish(launch_embed(t, table, vocab, hidden, d_token, out, as_stream(stream)), "nt_embed");
}

size_t nt_attn_workspace_bytes(const nt_attn_desc *desc) {
    if (!desc || !attn_shape_ok(*desc)) return 0;
    return attn_workspace_bytes(*desc);
}

nt_status nt_attn_decode(const nt_attn_desc *desc, const float *q, const float *k_new, const float *v_new,
                         uint16_t *k_cache, uint16_t *v_cache, const int32_t *d_pos, float *out,
                         void *workspace, size_t workspace_bytes, nt_stream stream) {
    set_error("");
    NT_REQ(desc, NT_EINVAL, "nt_attn_decode: null descriptor");
    NT_REQ(desc->n_q_heads > 0 && desc->n_kv_heads > 0 && desc->head_dim > 0 && desc->ctx_cap > 0,
           NT_EINVAL, "nt_attn_decode: sizes must be positive");
    NT_REQ(attn_shape_ok(*desc), NT_ESHAPE,
           "nt_attn_decode: need head_dim 64 or 128 and n_q_heads / n_kv_heads in {1, 2, 4, 8}");
    NT_REQ(q && k_cache && v_cache && d_pos && out && workspace, NT_EINVAL, "nt_attn_decode: null pointer");
    NT_REQ((k_new == nullptr) == (v_new == nullptr), NT_EINVAL, "nt_attn_decode: k_new and v_new must both be set or both NULL");
    NT_REQ(desc->rope_theta >= 0.f, NT_EINVAL, "nt_attn_decode: rope_theta must be >= 0");
    NT_REQ(aligned(k_cache, 16) && aligned(v_cache, 16) && aligned(workspace, 16) && aligned(q, 16) &&
               aligned(out, 4) && aligned(d_pos, 4) && aligned(k_new, 4) && aligned(v_new, 4),
           NT_EALIGN, "nt_attn_decode: misaligned pointer");
    NT_REQ(workspace_bytes >= attn_workspace_bytes(*desc), NT_ENOMEM, "nt_attn_decode: workspace too small");
    if (nt_status s = need_device()) return s;
    return finish(launch_attn(*desc, q, k_new, v_new, k_cache, v_cache, d_pos, out, workspace, as_stream(stream)),
                  "nt_attn_decode");
}

// ---- encode -------------------------------------------------------------------------
nt_status nt_quantize(nt_qtype t, const float *x, void *blocks, int64_t n, nt_stream stream) {
    set_error("");
    if (!is_quant(t)) return fail(NT_EINVAL, "nt_quantize: unsupported type");
    if (n < 0) return fail(NT_EINVAL, "nt_quantize: negative n");
    if (n % block_elems(t) != 0) return fail(NT_ESHAPE, "nt_quantize: n is not a multiple of the block size");
    if (n == 0) return NT_OK;
    if (!x || !blocks) return fail(NT_EINVAL, "nt_quantize: null pointer");
    if (!aligned(x, 4) || !aligned(blocks, 16)) return fail(NT_EALIGN, "nt_quantize: misaligned pointer");
    if (nt_status s = need_device()) return s;
    return finish(launch_quantize(t, x, blocks, n, as_stream(stream)), "nt_quantize");
}

// ---- calibration kernels -----------------------------------------------------------
nt_status nt_read_bytes(const void *src, int64_t bytes, float *sink, nt_stream stream) {
    set_error("");
    if (bytes < 0) return fail(NT_EINVAL, "nt_read_bytes: negative size");
    if (bytes % 16 != 0) return fail(NT_ESHAPE, "nt_read_bytes: size not a multiple of 16");
    if (bytes == 0) return NT_OK;
    if (!src || !sink) return fail(NT_EINVAL, "nt_read_bytes: null pointer");
    if (!aligned(src, 16) || !aligned(sink, 4)) return fail(NT_EALIGN, "nt_read_bytes: misaligned");
    if (nt_status s = need_device()) return s;
    return finish(launch_read_bytes(src, bytes, sink, as_stream(stream)), "nt_read_bytes");
}


nt_status nt_copy_bytes(void *dst, const void *src, int64_t bytes, nt_stream stream) {
    set_error("");
    if (bytes < 0) return fail(NT_EINVAL, "nt_copy_bytes: negative size");
    if (bytes % 16 != 0) return fail(NT_ESHAPE, "nt_copy_bytes: size not a multiple of 16");
    if (bytes == 0) return NT_OK;
    if (!src || !dst) return fail(NT_EINVAL, "nt_copy_bytes: null pointer");
    if (!aligned(src, 16) || !aligned(dst, 16)) return fail(NT_EALIGN, "nt_copy_bytes: misaligned");
    if (nt_status s = need_device()) return s;
    return finish(launch_copy_bytes(dst, src, bytes, as_stream(stream)), "nt_copy_bytes");
}

}  // extern "C"
