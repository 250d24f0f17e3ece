// dequant.hip -- packed blocks -> fp32.
//
// The output (4 bytes per value against 0.56-1.06 bytes read) dominates the
// traffic, so the main kernel is laid out for the stores: a wave takes a
// window of 256 values (one K-quant super-block, or eight Q8_0 / Q4_0
// blocks), lane i forms values 4i .. 4i + 3 and writes them with one 16-byte
// store, so each store instruction writes 1 KB contiguously; the lane reads
// only the code bytes of its four values (one word, or two half-words where
// blocks are only 2-byte aligned) and the window's scales.  An output that is
// not 16-byte aligned takes the one-value-per-thread kernel.
//
// Formats: the GGUF quantizations the ntransformer write-up lists in its
// "Overview" (block layouts in include/nt.h).  Every value is a product of
// fp16 scale bits, small integer sub-scales and a small integer code, at most
// 24 significant bits in all, so the fp32 arithmetic below is exact and the
// result is the correctly rounded value of the definition.  In Q4_K the two
// exact terms (d*S)*q and dmin*M are combined with one rounding.
#include <algorithm>

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

__device__ __forceinline__ uint32_t rd32_2(const uint8_t *p) {   // 4 bytes from a 2-byte-aligned address
    const uint16_t *q = reinterpret_cast<const uint16_t *>(p);
    return uint32_t(q[0]) | (uint32_t(q[1]) << 16);
}

// Values 4i .. 4i + 3 of 256-value window w: the same arithmetic, value by
// value, as the dq_* functions above, so the results are bit-identical.
template <nt_qtype T>
__device__ __forceinline__ bool window_values(const uint8_t *__restrict__ blocks, int64_t w, int i, int64_t nblk,
                                              float4 &o) {
    float v[4];
    if constexpr (T == NT_Q8_0 || T == NT_Q4_0) {
        constexpr int BB = T == NT_Q8_0 ? 34 : 18;
        const int64_t b = 8 * w + (i >> 3);            // block of these values
        if (b >= nblk) return false;
        const uint8_t *blk = blocks + b * BB;
        const float d = h2f(*reinterpret_cast<const uint16_t *>(blk));
        const int e0 = 4 * (i & 7);                    // first value in the block
        if constexpr (T == NT_Q8_0) {
            const uint32_t c = rd32_2(blk + 2 + e0);
#pragma unroll
            for (int t = 0; t < 4; ++t) v[t] = d * static_cast<float>(static_cast<int8_t>((c >> (8 * t)) & 0xffu));
        } else {
            const uint32_t c = rd32_2(blk + 2 + (e0 & 15)) >> (e0 < 16 ? 0 : 4);
#pragma unroll
            for (int t = 0; t < 4; ++t) v[t] = d * static_cast<float>(int((c >> (8 * t)) & 15u) - 8);
        }
    } else if constexpr (T == NT_Q4_K || T == NT_Q5_K) {
        constexpr int BB = T == NT_Q4_K ? 144 : 176, QS = T == NT_Q4_K ? 16 : 48;
        const uint8_t *blk = blocks + w * BB;          // 16-byte aligned
        const u32x4 h = ld4(blk);
        const float d = h2f(h.x & 0xffffu), dmin = h2f(h.x >> 16);
        const int j = i >> 3, l0 = 4 * (i & 7);        // sub-block, first value in it
        const uint32_t sc[3] = {h.y, h.z, h.w};
        auto byte = [&](int k) { return int((sc[k >> 2] >> (8 * (k & 3))) & 0xffu); };
        int S, M;
        if (j < 4) {
            S = byte(j) & 63;
            M = byte(j + 4) & 63;
        } else {
            S = (byte(j + 4) & 15) | ((byte(j - 4) >> 6) << 4);
            M = (byte(j + 4) >> 4) | ((byte(j) >> 6) << 4);
        }
        const uint32_t c = ld1(blk + QS + 32 * (j >> 1) + l0) >> (4 * (j & 1));
        uint32_t hb = 0;
        if constexpr (T == NT_Q5_K) hb = ld1(blk + 16 + l0) >> j;
        const float ds = d * static_cast<float>(S);     // exact
        const float dm = dmin * static_cast<float>(M);  // exact
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const int q = int((c >> (8 * t)) & 15u) | (T == NT_Q5_K ? int(((hb >> (8 * t)) & 1u) << 4) : 0);
            v[t] = ds * static_cast<float>(q) - dm;     // one rounding
        }
    } else {
        const uint8_t *blk = blocks + w * 210;         // 2-byte aligned
        const int h = i >> 5, k = (i >> 3) & 3, l0 = 4 * (i & 7);
        const uint32_t lob = rd32_2(blk + 64 * h + 32 * (k & 1) + l0) >> (k < 2 ? 0 : 4);
        const uint32_t hib = rd32_2(blk + 128 + 32 * h + l0) >> (2 * k);
        const float d = h2f(*reinterpret_cast<const uint16_t *>(blk + 208));
        const float sc = static_cast<float>(static_cast<int8_t>(blk[192 + (i >> 2)]));
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const int q = int((lob >> (8 * t)) & 15u) | int(((hib >> (8 * t)) & 3u) << 4);
            v[t] = (d * sc) * static_cast<float>(q - 32);   // each product exact
        }
    }
    o = float4{v[0], v[1], v[2], v[3]};
    return true;
}

typedef float f4v __attribute__((ext_vector_type(4)));

// Each wave takes windows w, w + nw, ..., four per iteration, so the loads
// of four windows are in flight together.  The stores are non-temporal
// (streamed past the caches, which the output would only evict): 268 MB of
// Q4_K output from cached blocks took 83 us with ordinary stores and 51 us
// so.  (Issuing the next four windows' loads before this iteration's stores
// was measured too: Q8_0 faster, Q4_K the same, Q6_K a third slower.)
template <nt_qtype T>
__global__ void __launch_bounds__(256) dequant_windows(const uint8_t *__restrict__ blocks, float *__restrict__ out,
                                                        int64_t nwin, int64_t nblk) {
    constexpr int U = 4;
    const int lane = threadIdx.x & 63;
    const int64_t nw = int64_t(gridDim.x) * (blockDim.x >> 6);
    for (int64_t w = int64_t(blockIdx.x) * (blockDim.x >> 6) + (threadIdx.x >> 6); w < nwin; w += U * nw) {
        float4 o[U];
        bool live[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t wu = w + u * nw;
            live[u] = wu < nwin && window_values<T>(blocks, wu, lane, nblk, o[u]);
        }
#pragma unroll
        for (int u = 0; u < U; ++u)
            if (live[u])
                __builtin_nontemporal_store(f4v{o[u].x, o[u].y, o[u].z, o[u].w},
                                            reinterpret_cast<f4v *>(out + 256 * (w + u * nw)) + lane);
    }
}

}  // namespace

hipError_t launch_dequant(nt_qtype t, const void *blocks, float *out, int64_t n, hipStream_t st) {
    const uint8_t *b = static_cast<const uint8_t *>(blocks);
    if ((reinterpret_cast<uintptr_t>(out) & 15) == 0) {
        const int64_t be = (t == NT_Q8_0 || t == NT_Q4_0) ? 32 : 256;
        const int64_t nblk = n / be, nwin = (n + 255) / 256;
        // four waves per workgroup, eight workgroups per CU
        const int grid = int(std::min<int64_t>((nwin + 3) / 4, 256 * 8));
        switch (t) {
        case NT_Q8_0: dequant_windows<NT_Q8_0><<<grid, 256, 0, st>>>(b, out, nwin, nblk); break;
        case NT_Q4_0: dequant_windows<NT_Q4_0><<<grid, 256, 0, st>>>(b, out, nwin, nblk); break;
        case NT_Q4_K: dequant_windows<NT_Q4_K><<<grid, 256, 0, st>>>(b, out, nwin, nblk); break;
        case NT_Q5_K: dequant_windows<NT_Q5_K><<<grid, 256, 0, st>>>(b, out, nwin, nblk); break;
        case NT_Q6_K: dequant_windows<NT_Q6_K><<<grid, 256, 0, st>>>(b, out, nwin, nblk); break;
        default: return hipErrorInvalidValue;
        }
        return hipGetLastError();
    }
    const int threads = 256;
    int64_t want = (n + threads - 1) / threads;
    const int grid = int(want < 65536 ? want : 65536);
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
