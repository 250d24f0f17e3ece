// calib.hip -- plain streaming read and copy kernels of known size.  They are
// the yardstick for the GEMV kernels: the same 128-bit loads, no decode work,
// so their bandwidth is the practical read ceiling of the chip and their
// counter readings calibrate the HBM-traffic counters.
#include "device_util.h"
#include "nt_internal.h"

namespace nt {
namespace {

__global__ void __launch_bounds__(256) read_kernel(const u32x4 *__restrict__ src, int64_t n16,
                                                  float *__restrict__ sink) {
    const int64_t stride = int64_t(gridDim.x) * blockDim.x;
    uint32_t acc = 0;
    int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
    for (; i + 3 * stride < n16; i += 4 * stride) {
        u32x4 a = __builtin_nontemporal_load(src + i);
        u32x4 b = __builtin_nontemporal_load(src + i + stride);
        u32x4 c = __builtin_nontemporal_load(src + i + 2 * stride);
        u32x4 d = __builtin_nontemporal_load(src + i + 3 * stride);
        acc ^= (a.x ^ a.y ^ a.z ^ a.w) + (b.x ^ b.y ^ b.z ^ b.w) + (c.x ^ c.y ^ c.z ^ c.w) +
               (d.x ^ d.y ^ d.z ^ d.w);
    }
    for (; i < n16; i += stride) {
        u32x4 a = __builtin_nontemporal_load(src + i);
        acc ^= a.x ^ a.y ^ a.z ^ a.w;
    }
    // a store that depends on every thread's loads keeps them alive; it
    // practically never fires
    if (acc == 0x9e3779b9u) sink[(blockIdx.x + threadIdx.x) & 4095] = 1.0f;
}

__global__ void __launch_bounds__(256) copy_kernel(u32x4 *__restrict__ dst, const u32x4 *__restrict__ src,
                                                  int64_t n16) {
    const int64_t stride = int64_t(gridDim.x) * blockDim.x;
    for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n16; i += stride)
        dst[i] = __builtin_nontemporal_load(src + i);
}

int calib_grid(int64_t n16) {
    int64_t want = (n16 + 255) / 256;
    return int(want < 8192 ? want : 8192);
}

}  // namespace

hipError_t launch_read_bytes(const void *src, int64_t bytes, float *sink, hipStream_t st) {
    const int64_t n16 = bytes / 16;
    read_kernel<<<calib_grid(n16), 256, 0, st>>>(static_cast<const u32x4 *>(src), n16, sink);
    return hipGetLastError();
}

hipError_t launch_copy_bytes(void *dst, const void *src, int64_t bytes, hipStream_t st) {
    const int64_t n16 = bytes / 16;
    copy_kernel<<<calib_grid(n16), 256, 0, st>>>(static_cast<u32x4 *>(dst), static_cast<const u32x4 *>(src), n16);
    return hipGetLastError();
}

}  // namespace nt
