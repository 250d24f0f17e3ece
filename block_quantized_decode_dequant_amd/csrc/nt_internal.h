// nt_internal.h -- shared between the C-ABI layer and the HIP kernel files of
// libnt.  Not installed; the public interface is include/nt.h.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>
#include <string>

#include "nt.h"

namespace nt {

// Thread-local message behind nt_last_error().
void set_error(const std::string &msg);
nt_status fail(nt_status s, const std::string &msg);
nt_status check_launch(const char *what);

inline hipStream_t as_stream(nt_stream s) { return reinterpret_cast<hipStream_t>(s); }

inline bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Block geometry, shared by validation and launchers.
int64_t block_elems(nt_qtype t);
int64_t block_bytes(nt_qtype t);
bool is_quant(nt_qtype t);

// ---- launchers (defined in the .hip files; arguments already validated) ----
hipError_t launch_dequant(nt_qtype t, const void *blocks, float *out, int64_t n, hipStream_t st);
hipError_t launch_gemv(nt_qtype t, const void *W, const float *x, float *y, int64_t rows,
                       int64_t cols, int accumulate, hipStream_t st);
void gemv_launch_info(nt_qtype t, int64_t rows, int64_t cols, int32_t info[4]);
int64_t gemv_row_bytes(nt_qtype t, int64_t cols);
// shapes the LDS-ring kernels take (and with them the fused variants below)
bool gemv_fast_ok(nt_qtype t, int64_t rows, int64_t cols);
hipError_t launch_gemv_multi(nt_qtype t, int nseg, const void *const *W, const int64_t *rows, float *const *y,
                             int64_t cols, const float *x, const float *gain, float eps, int accumulate,
                             hipStream_t st);
hipError_t launch_gemv_swiglu(nt_qtype t, const void *Wg, const void *Wu, int64_t rows, int64_t cols,
                              const float *x, const float *gain, float eps, float *h, hipStream_t st);
// Two groups of matrices of different formats (each group one format, up to
// three matrices) over the same RMSNorm-ed activations in one launch; both
// groups must satisfy gemv_pair_ok (16-byte rows, at most 8192 columns).
bool gemv_pair_ok(nt_qtype t, int64_t rows, int64_t cols);
hipError_t launch_gemv_pair(nt_qtype ta, int na, const void *const *Wa, const int64_t *rows_a, float *const *ya,
                            nt_qtype tb, int nb, const void *const *Wb, const int64_t *rows_b, float *const *yb,
                            int64_t cols, const float *x, const float *gain, float eps, hipStream_t st);
hipError_t launch_quantize(nt_qtype t, const float *x, void *blocks, int64_t n, hipStream_t st);
hipError_t launch_rmsnorm(const float *x, const float *g, float *y, int64_t n, float eps, hipStream_t st);
hipError_t launch_rope(float *q, float *k, int n_q_heads, int n_kv_heads, int head_dim, const int32_t *d_pos,
                       float theta, hipStream_t st);
hipError_t launch_softmax(float *x, int64_t n, hipStream_t st);
hipError_t launch_swiglu(const float *g, const float *u, float *out, int64_t n, hipStream_t st);
hipError_t launch_argmax(const float *x, int64_t n, int32_t *out, int32_t *pos_inc, hipStream_t st);
// The same over many workgroups; scratch: 16 device bytes, zero before the
// first call, left zero by every call (x 16-byte aligned).
hipError_t launch_argmax_multi(const float *x, int64_t n, void *scratch, int32_t *out, int32_t *pos_inc,
                               hipStream_t st);
hipError_t launch_embed(nt_qtype t, const void *table, int64_t vocab, int64_t hidden, const int32_t *d_token,
                        float *out, hipStream_t st);
int attn_chunk(const nt_attn_desc &a);
size_t attn_workspace_bytes(const nt_attn_desc &a);
bool attn_shape_ok(const nt_attn_desc &a);
hipError_t launch_attn(const nt_attn_desc &a, const float *q, const float *k_new, const float *v_new, uint16_t *kc,
                       uint16_t *vc, const int32_t *d_pos, float *out, void *ws, hipStream_t st);
hipError_t launch_read_bytes(const void *src, int64_t bytes, float *sink, hipStream_t st);
hipError_t launch_copy_bytes(void *dst, const void *src, int64_t bytes, hipStream_t st);

// k <= 8 activation vectors against one matrix on the matrix cores
// (all five block formats); ws: gemm_batch_workspace_bytes, 16-byte aligned.
bool gemm_batch_type_ok(nt_qtype t);
size_t gemm_batch_workspace_bytes(nt_qtype t, int64_t rows, int64_t cols);
hipError_t launch_gemm_batch(nt_qtype t, const void *W, int64_t rows, int64_t cols, const float *X, int k, float *Y,
                             int accumulate, void *ws, hipStream_t st);

constexpr int64_t kMaxGemvCols = 65536;

}  // namespace nt
