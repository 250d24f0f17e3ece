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
    case NT_Q4_K: case NT_Q6_K: return 256;
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
    case NT_Q6_K: return 210;
    }
    return -1;
}

bool is_quant(nt_qtype t) { return t == NT_Q8_0 || t == NT_Q4_0 || t == NT_Q4_K || t == NT_Q6_K; }

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

#define NT_GEMV_FN(name, T)                                                                       \
    nt_status name(const void *W, const float *x, float *y, int64_t rows, int64_t cols, int acc,  \
                   nt_stream s) {                                                                 \
        return nt_gemv(T, W, x, y, rows, cols, acc, s);                                           \
    }
NT_GEMV_FN(nt_gemv_q8_0, NT_Q8_0)
NT_GEMV_FN(nt_gemv_q4_0, NT_Q4_0)
NT_GEMV_FN(nt_gemv_q4_k, NT_Q4_K)
NT_GEMV_FN(nt_gemv_q6_k, NT_Q6_K)
#undef NT_GEMV_FN

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

nt_status nt_delay(double microseconds, nt_stream stream) {
    set_error("");
    if (!(microseconds >= 0.0) || microseconds > 1e6) return fail(NT_EINVAL, "nt_delay: need 0 <= us <= 1e6");
    if (nt_status s = need_device()) return s;
    return finish(launch_delay(microseconds, as_stream(stream)), "nt_delay");
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
