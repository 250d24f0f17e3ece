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
hipError_t launch_quantize(nt_qtype t, const float *x, void *blocks, int64_t n, hipStream_t st);
hipError_t launch_delay(double us, hipStream_t st);
hipError_t launch_read_bytes(const void *src, int64_t bytes, float *sink, hipStream_t st);
hipError_t launch_copy_bytes(void *dst, const void *src, int64_t bytes, hipStream_t st);

constexpr int64_t kMaxGemvCols = 65536;

}  // namespace nt
