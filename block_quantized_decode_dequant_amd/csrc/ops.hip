// ops.hip -- the small per-token kernels around the GEMVs: RMSNorm, RoPE,
// softmax, SwiGLU, greedy argmax and the embedding-row lookup.
//
// The ntransformer write-up lists RMSNorm, RoPE, SwiGLU and softmax among its
// GPU kernels ("Architecture") and RoPE, GQA, SwiGLU, RMSNorm and the KV cache
// as the Llama pieces it supports ("Main features"); the sampler lives under
// inference/.  Formulas (the pages give none; the usual Llama ones):
//   RMSNorm  y_i = g_i * x_i / sqrt(mean(x^2) + eps)
//   RoPE     pair (v[2i], v[2i+1]) of each head turns by pos * theta^(-2i/D)
//   softmax  p_t = exp(s_t - max s) / sum exp(s - max s)
//   SwiGLU   silu(g) * u, silu(a) = a / (1 + exp(-a))
//   greedy   index of the largest logit, lowest index on ties
// Each is tiny next to the GEMVs (a few KB per token); they are latency-bound,
// so they run as single workgroups or flat grids with fixed-order reductions
// (deterministic results).
#include "device_util.h"
#include "nt_internal.h"

namespace nt {
namespace {

constexpr int kBlock = 1024;

// Sum of one value per thread over a 1024-thread block, in a fixed order;
// every thread gets the result.
__device__ float block_sum(float v, float *red) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
    v = wave_sum_to_lane63(v);
    __syncthreads();
    if (lane == 63) red[wave] = v;
    __syncthreads();
    float s = 0.f;
    for (int w = 0; w < nw; ++w) s += red[w];
    return s;
}

__device__ float block_max(float v, float *red) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
    v = wave_max(v);
    __syncthreads();
    if (lane == 0) red[wave] = v;
    __syncthreads();
    float m = red[0];
    for (int w = 1; w < nw; ++w) m = fmaxf(m, red[w]);
    return m;
}

__global__ void __launch_bounds__(kBlock) rmsnorm_kernel(const float *__restrict__ x, const float *__restrict__ g,
                                                         float *__restrict__ y, int64_t n, float eps) {
    __shared__ float red[16];
    float ss = 0.f;
    for (int64_t i = threadIdx.x; i < n; i += blockDim.x) ss = fmaf(x[i], x[i], ss);
    const float tot = block_sum(ss, red);
    const float inv = 1.0f / sqrtf(tot / float(n) + eps);
    for (int64_t i = threadIdx.x; i < n; i += blockDim.x) y[i] = g[i] * (x[i] * inv);
}

__global__ void __launch_bounds__(256) rope_kernel(float *__restrict__ q, float *__restrict__ k, int n_q_heads,
                                                   int n_kv_heads, int head_dim, const int32_t *__restrict__ d_pos,
                                                   float theta) {
    const int half = head_dim / 2;
    const int idx = blockIdx.x * blockDim.x + threadIdx.x;
    const int total = (n_q_heads + n_kv_heads) * half;
    if (idx >= total) return;
    const int head = idx / half, i = idx % half;
    float *v = head < n_q_heads ? q + int64_t(head) * head_dim : k + int64_t(head - n_q_heads) * head_dim;
    const double pos = double(*d_pos);
    // angle in fp64: pos * theta^(-2i/D)
    const double w = pow(double(theta), -2.0 * double(i) / double(head_dim));
    double s, c;
    sincos(pos * w, &s, &c);
    const float cf = float(c), sf = float(s);
    const float a = v[2 * i], b = v[2 * i + 1];
    v[2 * i] = a * cf - b * sf;
    v[2 * i + 1] = a * sf + b * cf;
}

__global__ void __launch_bounds__(kBlock) softmax_kernel(float *__restrict__ x, int64_t n) {
    __shared__ float red[16];
    float m = -INFINITY;
    for (int64_t i = threadIdx.x; i < n; i += blockDim.x) m = fmaxf(m, x[i]);
    const float mx = block_max(m, red);
    float s = 0.f;
    for (int64_t i = threadIdx.x; i < n; i += blockDim.x) s += expf(x[i] - mx);
    const float tot = block_sum(s, red);
    const float inv = 1.0f / tot;
    for (int64_t i = threadIdx.x; i < n; i += blockDim.x) x[i] = expf(x[i] - mx) * inv;
}

__global__ void __launch_bounds__(256) swiglu_kernel(const float *__restrict__ g, const float *__restrict__ u,
                                                     float *__restrict__ out, int64_t n) {
    const int64_t stride = int64_t(gridDim.x) * blockDim.x;
    for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n; i += stride) {
        const float a = g[i];
        out[i] = a / (1.0f + expf(-a)) * u[i];
    }
}

// (value, index) pair order: larger value wins, lower index on ties.  NaNs
// never win against a number.
__device__ __forceinline__ bool better(float v, int i, float bv, int bi) {
    return v > bv || (v == bv && i < bi) || (bv != bv && v == v);
}

// Writes the index of the largest of x[0, n) to *out; when `pos` is given,
// also increments *pos (the decode step's position) after the pick.
__global__ void __launch_bounds__(kBlock) argmax_kernel(const float *__restrict__ x, int64_t n,
                                                        int32_t *__restrict__ out, int32_t *__restrict__ pos) {
    __shared__ float rv[16];
    __shared__ int ri[16];
    float bv = -INFINITY;
    int bi = 0x7fffffff;
    int64_t i0 = 0;
    if ((reinterpret_cast<uintptr_t>(x) & 15) == 0) {
        // 16-byte loads, several in flight per thread
        const float4 *x4 = reinterpret_cast<const float4 *>(x);
        const int64_t n4 = n / 4;
#pragma unroll 8
        for (int64_t i = threadIdx.x; i < n4; i += blockDim.x) {
            const float4 v = x4[i];
            const int b = int(4 * i);
            if (better(v.x, b, bv, bi)) { bv = v.x; bi = b; }
            if (better(v.y, b + 1, bv, bi)) { bv = v.y; bi = b + 1; }
            if (better(v.z, b + 2, bv, bi)) { bv = v.z; bi = b + 2; }
            if (better(v.w, b + 3, bv, bi)) { bv = v.w; bi = b + 3; }
        }
        i0 = 4 * n4;
    }
#pragma unroll 8
    for (int64_t i = i0 + threadIdx.x; i < n; i += blockDim.x) {
        const float v = x[i];
        if (better(v, int(i), bv, bi)) { bv = v; bi = int(i); }
    }
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) {
        const float ov = __shfl_xor(bv, m, 64);
        const int oi = __shfl_xor(bi, m, 64);
        if (better(ov, oi, bv, bi)) { bv = ov; bi = oi; }
    }
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
    if (lane == 0) { rv[wave] = bv; ri[wave] = bi; }
    __syncthreads();
    if (threadIdx.x == 0) {
        float v = rv[0];
        int id = ri[0];
        for (int w = 1; w < nw; ++w)
            if (better(rv[w], ri[w], v, id)) { v = rv[w]; id = ri[w]; }
        *out = (id == 0x7fffffff) ? 0 : id;
        if (pos) *pos += 1;
    }
}

// The same pick spread over many workgroups (the decode step's head: 128K
// logits are too many for one workgroup's memory bandwidth).  Each
// workgroup reduces its contiguous range, then folds its best (value, index)
// into one 64-bit key with a device-scope atomic max; the key orders values
// like better() (NaN lowest, -0 as +0, lower index first on ties).  A ticket
// counter tells the last workgroup that every other fold is done (each
// workgroup waits for its max to return before taking a ticket); that one
// writes the index, bumps the position and clears key and ticket for the
// next call.  Key and ticket start at zero (the model clears them once).
__device__ __forceinline__ unsigned long long pick_key(float v, int i) {
    if (v != v || i == 0x7fffffff) return 0ull;
    uint32_t b = __float_as_uint(v == 0.f ? 0.f : v);
    b = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
    return (static_cast<unsigned long long>(b) << 32) | (0xffffffffu - uint32_t(i));
}

constexpr int kPickBlock = 256;

__global__ void __launch_bounds__(kPickBlock) argmax_multi_kernel(const float *__restrict__ x, int64_t n,
                                                                  unsigned long long *key, unsigned int *ticket,
                                                                  int32_t *__restrict__ out, int32_t *__restrict__ pos) {
    __shared__ float rv[kPickBlock / 64];
    __shared__ int ri[kPickBlock / 64];
    // contiguous ranges, multiples of 4 values (x is 16-byte aligned)
    const int64_t per = ((n + gridDim.x - 1) / gridDim.x + 3) / 4 * 4;
    const int64_t lo = int64_t(blockIdx.x) * per, hi = lo + per < n ? lo + per : n;
    float bv = -INFINITY;
    int bi = 0x7fffffff;
    const int64_t hi4 = lo + (hi > lo ? (hi - lo) / 4 * 4 : 0);
    for (int64_t i = lo + 4 * threadIdx.x; i < hi4; i += 4 * kPickBlock) {
        const float4 v = *reinterpret_cast<const float4 *>(x + i);
        const int b = int(i);
        if (better(v.x, b, bv, bi)) { bv = v.x; bi = b; }
        if (better(v.y, b + 1, bv, bi)) { bv = v.y; bi = b + 1; }
        if (better(v.z, b + 2, bv, bi)) { bv = v.z; bi = b + 2; }
        if (better(v.w, b + 3, bv, bi)) { bv = v.w; bi = b + 3; }
    }
    for (int64_t i = hi4 + threadIdx.x; i < hi; i += kPickBlock) {
        const float v = x[i];
        if (better(v, int(i), bv, bi)) { bv = v; bi = int(i); }
    }
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) {
        const float ov = __shfl_xor(bv, m, 64);
        const int oi = __shfl_xor(bi, m, 64);
        if (better(ov, oi, bv, bi)) { bv = ov; bi = oi; }
    }
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (lane == 0) { rv[wave] = bv; ri[wave] = bi; }
    __syncthreads();
    if (threadIdx.x == 0) {
        float v = rv[0];
        int id = ri[0];
        for (int w = 1; w < kPickBlock / 64; ++w)
            if (better(rv[w], ri[w], v, id)) { v = rv[w]; id = ri[w]; }
        const unsigned long long prev =
            __hip_atomic_fetch_max(key, pick_key(v, id), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        // the ticket is taken only once the max has returned: the increment
        // depends on its result (a key is never all ones, so it is always 1)
        const unsigned int t = __hip_atomic_fetch_add(ticket, prev == ~0ull ? 2u : 1u, __ATOMIC_RELAXED,
                                                      __HIP_MEMORY_SCOPE_AGENT);
        if (t == gridDim.x - 1) {
            const unsigned long long k = __hip_atomic_exchange(key, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(ticket, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            *out = k == 0ull ? 0 : int(0xffffffffu - uint32_t(k));
            if (pos) *pos += 1;
        }
    }
}

// Decodes row *d_token of a packed [vocab x hidden] table into out[hidden]; a
// token outside [0, vocab) yields NaNs instead of an out-of-bounds read.
template <int T>
__global__ void __launch_bounds__(256) embed_kernel(const uint8_t *__restrict__ table, int64_t vocab,
                                                    int64_t hidden, const int32_t *__restrict__ d_token,
                                                    float *__restrict__ out);

__device__ __forceinline__ uint32_t rd16(const uint8_t *p) { return p[0] | (uint32_t(p[1]) << 8); }

template <int T>
__device__ float decode_one(const uint8_t *row, int64_t e) {
    if constexpr (T == NT_Q8_0) {
        const uint8_t *blk = row + (e / 32) * 34;
        return h2f(rd16(blk)) * float(int8_t(blk[2 + e % 32]));
    } else if constexpr (T == NT_Q4_0) {
        const uint8_t *blk = row + (e / 32) * 18;
        const int i = int(e % 32);
        const uint32_t byte = blk[2 + (i & 15)];
        return h2f(rd16(blk)) * float(int((i < 16) ? (byte & 15) : (byte >> 4)) - 8);
    } else if constexpr (T == NT_Q4_K) {
        const uint8_t *blk = row + (e / 256) * 144;
        const int i = int(e % 256), j = i >> 5;
        const uint8_t *b = blk + 4;
        int S, M;
        if (j < 4) { S = b[j] & 63; M = b[j + 4] & 63; }
        else { S = (b[j + 4] & 15) | ((b[j - 4] >> 6) << 4); M = (b[j + 4] >> 4) | ((b[j] >> 6) << 4); }
        const uint32_t byte = blk[16 + 32 * (j >> 1) + (i & 31)];
        const int q = (j & 1) ? (byte >> 4) : (byte & 15);
        return (h2f(rd16(blk)) * float(S)) * float(q) - h2f(rd16(blk + 2)) * float(M);
    } else if constexpr (T == NT_Q5_K) {
        const uint8_t *blk = row + (e / 256) * 176;
        const int i = int(e % 256), j = i >> 5, l = i & 31;
        const uint8_t *b = blk + 4;
        int S, M;
        if (j < 4) { S = b[j] & 63; M = b[j + 4] & 63; }
        else { S = (b[j + 4] & 15) | ((b[j - 4] >> 6) << 4); M = (b[j + 4] >> 4) | ((b[j] >> 6) << 4); }
        const uint32_t byte = blk[48 + 32 * (j >> 1) + l];
        const int q = int((j & 1) ? (byte >> 4) : (byte & 15)) | (((blk[16 + l] >> j) & 1) << 4);
        return (h2f(rd16(blk)) * float(S)) * float(q) - h2f(rd16(blk + 2)) * float(M);
    } else {
        const uint8_t *blk = row + (e / 256) * 210;
        const int i = int(e % 256), h = i >> 7, r = i & 127, k = r >> 5, l = r & 31;
        const uint32_t lob = blk[64 * h + 32 * (k & 1) + l];
        const int q = int((k < 2) ? (lob & 15) : (lob >> 4)) | (((blk[128 + 32 * h + l] >> (2 * k)) & 3) << 4);
        return (h2f(rd16(blk + 208)) * float(int8_t(blk[192 + (i >> 4)]))) * float(q - 32);
    }
}

template <int T>
__global__ void __launch_bounds__(256) embed_kernel(const uint8_t *__restrict__ table, int64_t vocab,
                                                    int64_t hidden, const int32_t *__restrict__ d_token,
                                                    float *__restrict__ out) {
    const int64_t e = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
    if (e >= hidden) return;
    const int32_t tok = *d_token;
    if (tok < 0 || tok >= vocab) {
        out[e] = __int_as_float(0x7fc00000);
        return;
    }
    constexpr int BE = (T == NT_Q8_0 || T == NT_Q4_0) ? 32 : 256;
    constexpr int BB = T == NT_Q8_0 ? 34 : T == NT_Q4_0 ? 18 : T == NT_Q4_K ? 144 : T == NT_Q5_K ? 176 : 210;
    const uint8_t *row = table + int64_t(tok) * (hidden / BE) * BB;
    out[e] = decode_one<T>(row, e);
}

}  // namespace

hipError_t launch_rmsnorm(const float *x, const float *g, float *y, int64_t n, float eps, hipStream_t st) {
    rmsnorm_kernel<<<1, kBlock, 0, st>>>(x, g, y, n, eps);
    return hipGetLastError();
}

hipError_t launch_rope(float *q, float *k, int n_q_heads, int n_kv_heads, int head_dim, const int32_t *d_pos,
                       float theta, hipStream_t st) {
    const int total = (n_q_heads + n_kv_heads) * (head_dim / 2);
    rope_kernel<<<(total + 255) / 256, 256, 0, st>>>(q, k, n_q_heads, n_kv_heads, head_dim, d_pos, theta);
    return hipGetLastError();
}

hipError_t launch_softmax(float *x, int64_t n, hipStream_t st) {
    softmax_kernel<<<1, kBlock, 0, st>>>(x, n);
    return hipGetLastError();
}

hipError_t launch_swiglu(const float *g, const float *u, float *out, int64_t n, hipStream_t st) {
    int64_t want = (n + 255) / 256;
    const int grid = int(want < 4096 ? want : 4096);
    swiglu_kernel<<<grid, 256, 0, st>>>(g, u, out, n);
    return hipGetLastError();
}

hipError_t launch_argmax(const float *x, int64_t n, int32_t *out, int32_t *pos_inc, hipStream_t st) {
    argmax_kernel<<<1, kBlock, 0, st>>>(x, n, out, pos_inc);
    return hipGetLastError();
}

hipError_t launch_argmax_multi(const float *x, int64_t n, void *scratch, int32_t *out, int32_t *pos_inc,
                               hipStream_t st) {
    // about 4 KB of logits per workgroup, at most 512 workgroups
    int64_t want = (n + 1023) / 1024;
    const int grid = int(want < 1 ? 1 : (want > 512 ? 512 : want));
    unsigned long long *key = static_cast<unsigned long long *>(scratch);
    unsigned int *ticket = reinterpret_cast<unsigned int *>(key + 1);
    argmax_multi_kernel<<<grid, kPickBlock, 0, st>>>(x, n, key, ticket, out, pos_inc);
    return hipGetLastError();
}

hipError_t launch_embed(nt_qtype t, const void *table, int64_t vocab, int64_t hidden, const int32_t *d_token,
                        float *out, hipStream_t st) {
    const uint8_t *tb = static_cast<const uint8_t *>(table);
    const int grid = int((hidden + 255) / 256);
    switch (t) {
    case NT_Q8_0: embed_kernel<NT_Q8_0><<<grid, 256, 0, st>>>(tb, vocab, hidden, d_token, out); break;
    case NT_Q4_0: embed_kernel<NT_Q4_0><<<grid, 256, 0, st>>>(tb, vocab, hidden, d_token, out); break;
    case NT_Q4_K: embed_kernel<NT_Q4_K><<<grid, 256, 0, st>>>(tb, vocab, hidden, d_token, out); break;
    case NT_Q5_K: embed_kernel<NT_Q5_K><<<grid, 256, 0, st>>>(tb, vocab, hidden, d_token, out); break;
    case NT_Q6_K: embed_kernel<NT_Q6_K><<<grid, 256, 0, st>>>(tb, vocab, hidden, d_token, out); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace nt
