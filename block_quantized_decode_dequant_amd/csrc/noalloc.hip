// noalloc.hip -- decode attention with library-held scratch memory, for
// callers that cannot allocate device memory (code under HIP graph capture,
// tight serving loops, harnesses that forbid allocation).
//
// The attention kernels keep per-chunk partial results between their two
// phases.  nt_attn_decode takes that scratch from the caller; the entry
// point here takes it from a fixed array in device memory instead.  The
// array is a file-scope __device__ object, so every device the library runs
// on holds its own copy until the process ends.  In host code the array's
// name is only a host-side stand-in: its device address is looked up once
// per device with hipGetSymbolAddress, and only that address is ever passed
// to kernels.
#include <hip/hip_runtime.h>

#include <mutex>

#include "nt_internal.h"

namespace nt {
namespace {

static_assert(NT_ATTN_NOALLOC_SCRATCH_BYTES % 256 == 0, "scratch size is a multiple of its alignment");

__device__ __align__(256) uint8_t scratch[NT_ATTN_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;

// The device address of `scratch` on the current device, looked up on the
// first call on that device (with that device current) and kept.
hipError_t scratch_ptr(void **out) {
    static std::mutex mu;
    static void *ptrs[kMaxDevices] = {};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (!ptrs[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        ptrs[dev] = p;
    }
    *out = ptrs[dev];
    return hipSuccess;
}

}  // namespace
}  // namespace nt

using namespace nt;

extern "C" nt_status nt_attn_decode_noalloc(const nt_attn_desc *desc, const float *q, const float *k_new,
                                            const float *v_new, uint16_t *k_cache, uint16_t *v_cache,
                                            const int32_t *d_pos, float *out, nt_stream stream) {
    set_error("");
    if (!desc) return fail(NT_EINVAL, "nt_attn_decode_noalloc: null descriptor");
    if (!(desc->n_q_heads > 0 && desc->n_kv_heads > 0 && desc->head_dim > 0 && desc->ctx_cap > 0))
        return fail(NT_EINVAL, "nt_attn_decode_noalloc: sizes must be positive");
    if (!attn_shape_ok(*desc))
        return fail(NT_ESHAPE, "nt_attn_decode_noalloc: need head_dim 64 or 128 and n_q_heads / n_kv_heads in "
                               "{1, 2, 4, 8}");
    if (!q || !k_cache || !v_cache || !d_pos || !out)
        return fail(NT_EINVAL, "nt_attn_decode_noalloc: null pointer");
    if ((k_new == nullptr) != (v_new == nullptr))
        return fail(NT_EINVAL, "nt_attn_decode_noalloc: k_new and v_new must both be set or both NULL");
    if (!(desc->rope_theta >= 0.f)) return fail(NT_EINVAL, "nt_attn_decode_noalloc: rope_theta must be >= 0");
    if (!(aligned(k_cache, 16) && aligned(v_cache, 16) && aligned(q, 16) && aligned(out, 4) && aligned(d_pos, 4) &&
          aligned(k_new, 4) && aligned(v_new, 4)))
        return fail(NT_EALIGN, "nt_attn_decode_noalloc: misaligned pointer");
    const size_t need = attn_workspace_bytes(*desc);
    if (need > size_t(NT_ATTN_NOALLOC_SCRATCH_BYTES))
        return fail(NT_ENOMEM, "nt_attn_decode_noalloc: this shape needs " + std::to_string(need) +
                                   " bytes of scratch, above the fixed " +
                                   std::to_string(NT_ATTN_NOALLOC_SCRATCH_BYTES) + " (use nt_attn_decode)");
    int n = 0;
    if (hipGetDeviceCount(&n) != hipSuccess || n <= 0) {
        (void)hipGetLastError();
        return fail(NT_ENODEV, "nt_attn_decode_noalloc: no HIP device available");
    }
    void *ws = nullptr;
    hipError_t e = scratch_ptr(&ws);
    if (e != hipSuccess) {
        (void)hipGetLastError();
        return fail(NT_EHIP, std::string("nt_attn_decode_noalloc: scratch address: ") + hipGetErrorString(e));
    }
    e = launch_attn(*desc, q, k_new, v_new, k_cache, v_cache, d_pos, out, ws, as_stream(stream));
    if (e != hipSuccess) {
        (void)hipGetLastError();
        return fail(NT_EHIP, std::string("nt_attn_decode_noalloc: ") + hipGetErrorString(e));
    }
    return NT_OK;
}
