// attn.hip -- grouped-query attention for one decode token over an fp16 KV
// cache (the write-up's "Main features": GQA and the KV cache; "Roadmap":
// F16 KV cache; softmax among the "Architecture" kernels).
//
// For q head h in kv group g = h / G (G = n_q_heads / n_kv_heads):
//   s_t = scale * <q_h, k_{g,t}>,  p = softmax(s over t = 0..pos),
//   o_h = sum_t p_t v_{g,t}
// The context is split into chunks of C positions so that n_kv_heads x chunks
// workgroups fill the chip; each workgroup reads its chunk of K and V once for
// all G query heads of the group and leaves (max, sum, unnormalized o) per
// head; a merge kernel combines the chunks with the log-sum-exp rule in a
// fixed order.  The current token's k and v are stored at slot pos (rounded to
// fp16) by the workgroup that owns that slot, which attends to the rounded
// values, so the cache and the attention agree.  A position outside
// [0, ctx_cap) writes NaN outputs and touches no memory out of bounds.
#include "device_util.h"
#include "nt_internal.h"

namespace nt {
namespace {

constexpr int kAttnThreads = 256;

__device__ __forceinline__ uint16_t f2h_bits(float v) { return __half_as_ushort(__float2half_rn(v)); }
__device__ __forceinline__ float hb2f(uint16_t b) { return __half2float(__ushort_as_half(b)); }

// Sum over aligned groups of 16 lanes (every lane of the group gets it).
__device__ __forceinline__ float sum16(float v) {
    v += dpp<0xb1>(v);    // xor 1
    v += dpp<0x4e>(v);    // xor 2
    v += dpp<0x141>(v);   // half-row mirror
    v += dpp<0x140>(v);   // row mirror
    return v;
}

// grid (max_chunks, n_kv_heads); D = head_dim, G = q heads per kv head.
template <int D, int G>
__global__ void __launch_bounds__(kAttnThreads) attn_split_kernel(
    const float *__restrict__ q, const float *__restrict__ k_new, const float *__restrict__ v_new,
    uint16_t *__restrict__ kc, uint16_t *__restrict__ vc, const int32_t *__restrict__ d_pos, int ctx_cap,
    int chunk, float scale, float *__restrict__ part) {
    constexpr int DL = D / 16;          // dims per lane in the score phase
    extern __shared__ float sm[];       // p[G][chunk] | knew[D] | vnew[D]
    float *p = sm;
    float *knew = sm + G * chunk;
    float *vnew = knew + D;

    const int pos = *d_pos;
    if (pos < 0 || pos >= ctx_cap) return;          // the merge kernel writes NaNs
    const int c = blockIdx.x, g = blockIdx.y;
    const int t0 = c * chunk;
    if (t0 > pos) return;                           // chunk not reached yet
    const int tn = min(chunk, pos + 1 - t0);        // positions in this chunk
    const int64_t head_base = int64_t(g) * ctx_cap * D;
    const bool owns_new = k_new && pos < t0 + chunk;

    if (owns_new) {
        for (int d = threadIdx.x; d < D; d += blockDim.x) {
            const uint16_t kb = f2h_bits(k_new[g * D + d]), vb = f2h_bits(v_new[g * D + d]);
            kc[head_base + int64_t(pos) * D + d] = kb;
            vc[head_base + int64_t(pos) * D + d] = vb;
            knew[d] = hb2f(kb);
            vnew[d] = hb2f(vb);
        }
    }

    // ---- scores: 16 lanes per position, DL dims per lane ----
    const int grp = threadIdx.x >> 4, l16 = threadIdx.x & 15;
    float qr[G][DL];
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
        for (int i = 0; i < DL; ++i) qr[h][i] = q[(g * G + h) * D + l16 * DL + i] * scale;
    __syncthreads();
    const int ngrp = blockDim.x >> 4;
    for (int tt = grp; tt < ((tn + ngrp - 1) / ngrp) * ngrp; tt += ngrp) {
        const bool live = tt < tn;
        const int t = t0 + tt;
        float kv[DL];
        if (live && owns_new && t == pos) {
#pragma unroll
            for (int i = 0; i < DL; ++i) kv[i] = knew[l16 * DL + i];
        } else if (live) {
            // DL fp16 values = 16 (D = 128) or 8 (D = 64) contiguous bytes
            const uint16_t *kp = kc + head_base + int64_t(t) * D + l16 * DL;
            uint32_t wv[DL / 2];
            if constexpr (DL == 8) {
                const uint4 w4 = *reinterpret_cast<const uint4 *>(kp);
                wv[0] = w4.x; wv[1] = w4.y; wv[2] = w4.z; wv[3] = w4.w;
            } else {
                const uint2 w2 = *reinterpret_cast<const uint2 *>(kp);
                wv[0] = w2.x; wv[1] = w2.y;
            }
#pragma unroll
            for (int i = 0; i < DL / 2; ++i) {
                kv[2 * i] = hb2f(uint16_t(wv[i]));
                kv[2 * i + 1] = hb2f(uint16_t(wv[i] >> 16));
            }
        } else {
#pragma unroll
            for (int i = 0; i < DL; ++i) kv[i] = 0.f;
        }
#pragma unroll
        for (int h = 0; h < G; ++h) {
            float s = 0.f;
#pragma unroll
            for (int i = 0; i < DL; ++i) s = fmaf(qr[h][i], kv[i], s);
            s = sum16(s);
            if (live && l16 == 0) p[h * chunk + tt] = s;
        }
    }
    __syncthreads();

    // ---- chunk softmax statistics per head (one wave per head) ----
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nwave = blockDim.x >> 6;
    float *stat = vnew + D;             // [G][2]: max, sum
    for (int h = wave; h < G; h += nwave) {
        float m = -INFINITY;
        for (int tt = lane; tt < tn; tt += 64) m = fmaxf(m, p[h * chunk + tt]);
        m = wave_max(m);
        float l = 0.f;
        for (int tt = lane; tt < tn; tt += 64) {
            const float e = expf(p[h * chunk + tt] - m);
            p[h * chunk + tt] = e;
            l += e;
        }
        l = wave_sum(l);
        if (lane == 0) { stat[2 * h] = m; stat[2 * h + 1] = l; }
    }
    __syncthreads();

    // ---- unnormalized o = sum_t p_t v_t: threads over (dim pair, head set) ----
    constexpr int NP = D / 2;                       // dim pairs
    const int dp = threadIdx.x % NP, hs = threadIdx.x / NP, nhs = blockDim.x / NP;
    float o0[G], o1[G];
#pragma unroll
    for (int h = 0; h < G; ++h) { o0[h] = 0.f; o1[h] = 0.f; }
    for (int tt = 0; tt < tn; ++tt) {
        const int t = t0 + tt;
        float v0, v1;
        if (owns_new && t == pos) {
            v0 = vnew[2 * dp]; v1 = vnew[2 * dp + 1];
        } else {
            const uint32_t w = *reinterpret_cast<const uint32_t *>(vc + head_base + int64_t(t) * D + 2 * dp);
            v0 = hb2f(uint16_t(w)); v1 = hb2f(uint16_t(w >> 16));
        }
#pragma unroll
        for (int h = 0; h < G; ++h)
            if (h % nhs == hs) {
                const float pt = p[h * chunk + tt];
                o0[h] = fmaf(pt, v0, o0[h]);
                o1[h] = fmaf(pt, v1, o1[h]);
            }
    }
    // partial record per (g, c, h): [max, sum, o[0..D)]
    const int nchunks = gridDim.x;
#pragma unroll
    for (int h = 0; h < G; ++h)
        if (h % nhs == hs) {
            float *rec = part + ((int64_t(g) * G + h) * nchunks + c) * (D + 2);
            rec[2 + 2 * dp] = o0[h];
            rec[2 + 2 * dp + 1] = o1[h];
            if (dp == 0) { rec[0] = stat[2 * h]; rec[1] = stat[2 * h + 1]; }
        }
}

// grid n_q_heads, block D: combines the chunks of head h in chunk order.
template <int D>
__global__ void __launch_bounds__(256) attn_merge_kernel(const float *__restrict__ part, const int32_t *__restrict__ d_pos,
                                                        int ctx_cap, int chunk, int nchunks, float *__restrict__ out) {
    const int h = blockIdx.x, d = threadIdx.x;
    const int pos = *d_pos;
    if (pos < 0 || pos >= ctx_cap) {
        out[h * D + d] = __int_as_float(0x7fc00000);
        return;
    }
    const int nact = pos / chunk + 1;
    const float *base = part + int64_t(h) * nchunks * (D + 2);
    float M = -INFINITY;
    for (int c = 0; c < nact; ++c) M = fmaxf(M, base[c * (D + 2)]);
    float L = 0.f, o = 0.f;
    for (int c = 0; c < nact; ++c) {
        const float *rec = base + c * (D + 2);
        const float w = expf(rec[0] - M);
        L = fmaf(rec[1], w, L);
        o = fmaf(rec[2 + d], w, o);
    }
    out[h * D + d] = o / L;
}

template <int D, int G>
hipError_t launch_dg(const nt_attn_desc &a, int chunk, int nchunks, const float *q, const float *k_new,
                     const float *v_new, uint16_t *kc, uint16_t *vc, const int32_t *d_pos, float *out,
                     float *part, hipStream_t st) {
    const float scale = a.scale > 0.f ? a.scale : 1.0f / sqrtf(float(D));
    const size_t lds = (size_t(G) * chunk + 2 * D + 2 * G) * sizeof(float);
    attn_split_kernel<D, G><<<dim3(nchunks, a.n_kv_heads), kAttnThreads, lds, st>>>(
        q, k_new, v_new, kc, vc, d_pos, a.ctx_cap, chunk, scale, part);
    attn_merge_kernel<D><<<a.n_q_heads, D, 0, st>>>(part, d_pos, a.ctx_cap, chunk, nchunks, out);
    return hipGetLastError();
}

template <int D>
hipError_t launch_d(const nt_attn_desc &a, int chunk, int nchunks, const float *q, const float *k_new,
                    const float *v_new, uint16_t *kc, uint16_t *vc, const int32_t *d_pos, float *out, float *part,
                    hipStream_t st) {
    switch (a.n_q_heads / a.n_kv_heads) {
    case 1: return launch_dg<D, 1>(a, chunk, nchunks, q, k_new, v_new, kc, vc, d_pos, out, part, st);
    case 2: return launch_dg<D, 2>(a, chunk, nchunks, q, k_new, v_new, kc, vc, d_pos, out, part, st);
    case 4: return launch_dg<D, 4>(a, chunk, nchunks, q, k_new, v_new, kc, vc, d_pos, out, part, st);
    case 8: return launch_dg<D, 8>(a, chunk, nchunks, q, k_new, v_new, kc, vc, d_pos, out, part, st);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace

int attn_chunk(const nt_attn_desc &a) {
    // the largest power-of-two chunk (16..256 positions) that still gives at
    // least 256 (kv head, chunk) workgroups at full context
    const int64_t want = int64_t(a.ctx_cap) * a.n_kv_heads / 256;
    int c = 16;
    while (2 * c <= want && c < 256) c *= 2;
    return c;
}

size_t attn_workspace_bytes(const nt_attn_desc &a) {
    const int chunk = attn_chunk(a);
    const int64_t nchunks = (a.ctx_cap + chunk - 1) / chunk;
    return size_t(a.n_q_heads) * size_t(nchunks) * size_t(a.head_dim + 2) * sizeof(float);
}

bool attn_shape_ok(const nt_attn_desc &a) {
    if (a.n_kv_heads <= 0 || a.n_q_heads <= 0 || a.n_q_heads % a.n_kv_heads != 0) return false;
    const int G = a.n_q_heads / a.n_kv_heads;
    return (a.head_dim == 64 || a.head_dim == 128) && (G == 1 || G == 2 || G == 4 || G == 8) && a.ctx_cap > 0;
}

hipError_t launch_attn(const nt_attn_desc &a, const float *q, const float *k_new, const float *v_new, uint16_t *kc,
                       uint16_t *vc, const int32_t *d_pos, float *out, void *ws, hipStream_t st) {
    const int chunk = attn_chunk(a);
    const int nchunks = (a.ctx_cap + chunk - 1) / chunk;
    float *part = static_cast<float *>(ws);
    if (a.head_dim == 128) return launch_d<128>(a, chunk, nchunks, q, k_new, v_new, kc, vc, d_pos, out, part, st);
    return launch_d<64>(a, chunk, nchunks, q, k_new, v_new, kc, vc, d_pos, out, part, st);
}

}  // namespace nt
