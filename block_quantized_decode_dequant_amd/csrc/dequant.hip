// dequant.hip -- packed blocks -> fp32, one thread per output value.
//
// Formats: the GGUF quantizations the ntransformer write-up lists in its
// "Overview" (block layouts in include/nt.h).  Every value is a product of
// fp16 scale bits, small integer sub-scales and a small integer code, at most
// 24 significant bits in all, so the fp32 arithmetic below is exact and the
// result is the correctly rounded value of the definition.  In Q4_K the two
// exact terms (d*S)*q and dmin*M are combined with one rounding.
#include "device_util.h"
#include "nt_internal.h"

namespace nt {
namespace {

__device__ __forceinline__ uint32_t rd16(const uint8_t *p) { return p[0] | (uint32_t(p[1]) << 8); }

__device__ __forceinline__ float dq_q8_0(const uint8_t *blk, int e) {
    return h2f(rd16(blk)) * static_cast<float>(static_cast<int8_t>(blk[2 + e]));
}

__device__ __forceinline__ float dq_q4_0(const uint8_t *blk, int e) {
    uint32_t byte = blk[2 + (e & 15)];
    int q = (e < 16) ? (byte & 15) : (byte >> 4);
    return h2f(rd16(blk)) * static_cast<float>(q - 8);
}

__device__ __forceinline__ float dq_q4_k(const uint8_t *blk, int e) {
    const float d = h2f(rd16(blk)), dmin = h2f(rd16(blk + 2));
    const uint8_t *b = blk + 4;
    const int j = e >> 5;
    int S, M;
    if (j < 4) {
        S = b[j] & 63;
        M = b[j + 4] & 63;
    } else {
        S = (b[j + 4] & 15) | ((b[j - 4] >> 6) << 4);
        M = (b[j + 4] >> 4) | ((b[j] >> 6) << 4);
    }
    uint32_t byte = blk[16 + 32 * (j >> 1) + (e & 31)];
    int q = (j & 1) ? (byte >> 4) : (byte & 15);
    const float ds = d * static_cast<float>(S);     // exact
    const float dm = dmin * static_cast<float>(M);  // exact
    return ds * static_cast<float>(q) - dm;         // one rounding
}

// Q5_K: Q4_K's header and nibbles (qs after 32 bytes of qh) plus bit j of
// qh[l] as the fifth bit of value 32j + l; (d*S)*q has at most 22 bits.
__device__ __forceinline__ float dq_q5_k(const uint8_t *blk, int e) {
    const float d = h2f(rd16(blk)), dmin = h2f(rd16(blk + 2));
    const uint8_t *b = blk + 4;
    const int j = e >> 5, l = e & 31;
    int S, M;
    if (j < 4) {
        S = b[j] & 63;
        M = b[j + 4] & 63;
    } else {
        S = (b[j + 4] & 15) | ((b[j - 4] >> 6) << 4);
        M = (b[j + 4] >> 4) | ((b[j] >> 6) << 4);
    }
    uint32_t byte = blk[48 + 32 * (j >> 1) + l];
    int q = int((j & 1) ? (byte >> 4) : (byte & 15)) | (((blk[16 + l] >> j) & 1) << 4);
    const float ds = d * static_cast<float>(S);     // exact
    const float dm = dmin * static_cast<float>(M);  // exact
    return ds * static_cast<float>(q) - dm;         // one rounding
}

__device__ __forceinline__ float dq_q6_k(const uint8_t *blk, int e) {
    const int h = e >> 7, r = e & 127, k = r >> 5, l = r & 31;
    uint32_t lob = blk[64 * h + 32 * (k & 1) + l];
    int lo = (k < 2) ? (lob & 15) : (lob >> 4);
    int hi = (blk[128 + 32 * h + l] >> (2 * k)) & 3;
    int q = lo | (hi << 4);
    const float d = h2f(rd16(blk + 208));
    const float sc = static_cast<float>(static_cast<int8_t>(blk[192 + (e >> 4)]));
    return (d * sc) * static_cast<float>(q - 32);   // each product exact
}

template <nt_qtype T>
__global__ void __launch_bounds__(256) dequant_kernel(const uint8_t *__restrict__ blocks,
                                                       float *__restrict__ out, int64_t n) {
    constexpr int BE = (T == NT_Q8_0 || T == NT_Q4_0) ? 32 : 256;
    constexpr int BB = T == NT_Q8_0 ? 34 : T == NT_Q4_0 ? 18 : T == NT_Q4_K ? 144 : T == NT_Q5_K ? 176 : 210;
    const int64_t stride = int64_t(gridDim.x) * blockDim.x;
    for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n; i += stride) {
        const uint8_t *blk = blocks + (i / BE) * BB;
        const int e = int(i % BE);
        float v;
        if constexpr (T == NT_Q8_0) v = dq_q8_0(blk, e);
        else if constexpr (T == NT_Q4_0) v = dq_q4_0(blk, e);
        else if constexpr (T == NT_Q4_K) v = dq_q4_k(blk, e);
        else if constexpr (T == NT_Q5_K) v = dq_q5_k(blk, e);
        else v = dq_q6_k(blk, e);
        out[i] = v;
    }
}

}  // namespace

hipError_t launch_dequant(nt_qtype t, const void *blocks, float *out, int64_t n, hipStream_t st) {
    const int threads = 256;
    int64_t want = (n + threads - 1) / threads;
    const int grid = int(want < 65536 ? want : 65536);
    const uint8_t *b = static_cast<const uint8_t *>(blocks);
    switch (t) {
    case NT_Q8_0: dequant_kernel<NT_Q8_0><<<grid, threads, 0, st>>>(b, out, n); break;
    case NT_Q4_0: dequant_kernel<NT_Q4_0><<<grid, threads, 0, st>>>(b, out, n); break;
    case NT_Q4_K: dequant_kernel<NT_Q4_K><<<grid, threads, 0, st>>>(b, out, n); break;
    case NT_Q5_K: dequant_kernel<NT_Q5_K><<<grid, threads, 0, st>>>(b, out, n); break;
    case NT_Q6_K: dequant_kernel<NT_Q6_K><<<grid, threads, 0, st>>>(b, out, n); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace nt
