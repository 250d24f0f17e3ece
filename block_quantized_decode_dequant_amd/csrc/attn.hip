// attn.hip -- grouped-query attention for one decode token over an fp16 KV
// cache (the write-up's "Main features": GQA, RoPE and the KV cache;
// "Roadmap": F16 KV cache; softmax among the "Architecture" kernels).
//
// For q head h in kv group g = h / G (G = n_q_heads / n_kv_heads):
//   s_t = scale * <q_h, k_{g,t}>,  p = softmax(s over t = 0..pos),
//   o_h = sum_t p_t v_{g,t}
// Optionally q and the new k are first rotated by RoPE (adjacent pairs, angle
// pos * theta^(-2i/D) formed in fp64), so the decode step needs no separate
// rotation kernel.
//
// The context is split into chunks of C positions so that n_kv_heads x chunks
// workgroups fill the chip.  A workgroup first issues every load of its
// chunk's K and V (each thread holds its share in registers), then computes
// the G heads' scores, their chunk-local softmax statistics and the
// unnormalized weighted sum of V, and leaves (max, sum, o[D]) per head.  A
// merge kernel combines the chunks with the log-sum-exp rule in a fixed order
// (deterministic).  The current token's k and v are stored at slot pos
// (rounded to fp16) by the workgroup that owns that slot, which attends to the
// rounded values, so the cache and the attention agree.  A position outside
// [0, ctx_cap) writes NaN outputs and touches no memory out of bounds.
#include <algorithm>
#include <cmath>

#include "device_util.h"
#include "nt_internal.h"

namespace nt {
namespace {

constexpr int kAttnThreads = 256;
constexpr int kMaxChunk = 128;
constexpr int kMergeThreads = 512;

// RoPE frequencies theta^(-2i/D), i < D/2, formed in fp64 on the host and
// passed by value (the angle pos * w_i is formed in fp64 on the device).
struct RopeFreq {
    double w[64];
};

__device__ __forceinline__ uint16_t f2h_bits(float v) { return __half_as_ushort(__float2half_rn(v)); }

// Sum over aligned groups of N (8 or 16) lanes; every lane of a group gets it.
template <int N>
__device__ __forceinline__ float group_sum(float v) {
    v += dpp<0xb1>(v);    // xor 1
    v += dpp<0x4e>(v);    // xor 2
    v += dpp<0x141>(v);   // half-row mirror: the other quad of the 8
    if constexpr (N == 16) v += dpp<0x140>(v);   // row mirror: the other 8 of the 16
    return v;
}

// grid (chunks, n_kv_heads), 256 threads; D = head_dim, G = q heads per kv head.
template <int D, int G>
__global__ void __launch_bounds__(kAttnThreads) attn_split_kernel(
    const float *__restrict__ q, const float *__restrict__ k_new, const float *__restrict__ v_new,
    uint16_t *__restrict__ kc, uint16_t *__restrict__ vc, const int32_t *__restrict__ d_pos, int ctx_cap,
    int chunk, float scale, bool rope, const RopeFreq freq, float *__restrict__ part) {
    constexpr int LPP = D / 8;                   // score phase: lanes per position (8 dims each)
    constexpr int NPS = kAttnThreads / LPP;      // position subsets
    constexpr int NIK = kMaxChunk / NPS;         // positions per thread, at most
    constexpr int NDQ = D / 4;                   // value phase: dim quads (8 bytes of V)
    constexpr int NVS = kAttnThreads / NDQ;      // position subsets
    constexpr int NIV = kMaxChunk / NVS;
    __shared__ __attribute__((aligned(16))) float p[G][kMaxChunk];
    __shared__ __attribute__((aligned(16))) float qs[G * D];   // the G heads' q, rotated and scaled
    __shared__ float kn[D], vn[D];
    __shared__ float stat[G][2];
    __shared__ __attribute__((aligned(16))) float red[NVS][G][D];

    const int c = blockIdx.x, g = blockIdx.y, tid = threadIdx.x;
    // the G heads' q, 4 values per thread (needs no position: load first)
    constexpr int NQ = G * D / 4;                // threads holding q values
    static_assert(NQ <= kAttnThreads, "one float4 of q per thread");
    float4 q4 = make_float4(0.f, 0.f, 0.f, 0.f);
    if (tid < NQ) q4 = reinterpret_cast<const float4 *>(q + g * G * D)[tid];
    // the new token's k and v pair of this thread, loaded by every workgroup
    // with q (1 KB): only the one that owns slot pos uses them, but it then
    // needs no second memory round trip after reading the position
    // (k_new and v_new are only 4-byte aligned: two float loads each)
    float2 kn2 = make_float2(0.f, 0.f), vn2 = make_float2(0.f, 0.f);
    if (k_new && tid < D / 2) {
        kn2 = make_float2(k_new[g * D + 2 * tid], k_new[g * D + 2 * tid + 1]);
        vn2 = make_float2(v_new[g * D + 2 * tid], v_new[g * D + 2 * tid + 1]);
    }
    const int oc = tid % LPP, ps = tid / LPP;
    // ---- every K and V load of the chunk, issued before the position is
    // known (rows past the cache end re-read its last row), so the cache
    // reads overlap the read of *d_pos; rows past pos are loaded and ignored
    const int t0 = c * chunk;
    const int64_t head_base = int64_t(g) * ctx_cap * D;
    // K: thread (oc, ps) holds dims 8oc..8oc+7 of positions ps*nik + i (a
    // chunk that is not a multiple of NPS leaves the last subsets short)
    const int nik = (chunk + NPS - 1) / NPS;
    uint4 kr[NIK];
#pragma unroll
    for (int i = 0; i < NIK; ++i) {
        const int t = min(t0 + ps * nik + i, ctx_cap - 1);
        if (i < nik) kr[i] = *reinterpret_cast<const uint4 *>(kc + head_base + int64_t(t) * D + 8 * oc);
    }
    // V: thread (dq, vs) holds dims 4dq..4dq+3 of positions vs*niv + i
    const int dq = tid % NDQ, vs = tid / NDQ, niv = (chunk + NVS - 1) / NVS;
    uint2 vr[NIV];
#pragma unroll
    for (int i = 0; i < NIV; ++i) {
        const int t = min(t0 + vs * niv + i, ctx_cap - 1);
        if (i < niv) vr[i] = *reinterpret_cast<const uint2 *>(vc + head_base + int64_t(t) * D + 4 * dq);
    }

    const int pos = *d_pos;
    if (pos < 0 || pos >= ctx_cap || t0 > pos) {    // invalid (the merge writes NaNs) or chunk not reached
        __builtin_amdgcn_s_waitcnt(0);              // leave with no load outstanding
        return;
    }
    const int tn = min(chunk, pos + 1 - t0);        // positions in this chunk
    const bool owns_new = k_new && pos < t0 + chunk;

    // ---- RoPE angle of pair i: pos * w_i in fp64, reduced to [-pi, pi] in
    // fp64, then an fp32 sincos (the reduced angle is exact to ~1e-7 rad) ----
    const auto angle = [&](int i, float &cn, float &sn) {
        const double ph = double(pos) * freq.w[i];
        const double r = fma(-6.283185307179586, rint(ph * 0.15915494309189535), ph);
        sincosf(float(r), &sn, &cn);
    };
    // the q values, rotated and scaled, into LDS (values 4 tid .. 4 tid + 3:
    // two pairs of one head)
    if (tid < NQ) {
        float x[4] = {q4.x, q4.y, q4.z, q4.w};
        if (rope) {
            const int i0 = (4 * tid % D) / 2;
#pragma unroll
            for (int m = 0; m < 2; ++m) {
                float cs, sn;
                angle(i0 + m, cs, sn);
                const float x0 = x[2 * m], x1 = x[2 * m + 1];
                x[2 * m] = x0 * cs - x1 * sn;
                x[2 * m + 1] = x0 * sn + x1 * cs;
            }
        }
        *reinterpret_cast<float4 *>(&qs[4 * tid]) = make_float4(x[0] * scale, x[1] * scale, x[2] * scale, x[3] * scale);
    }
    if (owns_new && tid < D / 2) {
        float k0 = kn2.x, k1 = kn2.y;
        if (rope) {
            float cs, sn;
            angle(tid, cs, sn);
            const float a = k0, b = k1;
            k0 = a * cs - b * sn;
            k1 = a * sn + b * cs;
        }
        const uint16_t kb0 = f2h_bits(k0), kb1 = f2h_bits(k1);
        const uint16_t vb0 = f2h_bits(vn2.x), vb1 = f2h_bits(vn2.y);
        const int64_t at = head_base + int64_t(pos) * D + 2 * tid;
        *reinterpret_cast<uint32_t *>(kc + at) = uint32_t(kb0) | (uint32_t(kb1) << 16);
        *reinterpret_cast<uint32_t *>(vc + at) = uint32_t(vb0) | (uint32_t(vb1) << 16);
        kn[2 * tid] = h2f(kb0);
        kn[2 * tid + 1] = h2f(kb1);
        vn[2 * tid] = h2f(vb0);
        vn[2 * tid + 1] = h2f(vb1);
    }

    __syncthreads();                               // qs, kn, vn visible
    // ---- this thread's q octet of each head ----
    float qr[G][8];
#pragma unroll
    for (int h = 0; h < G; ++h) {
        const float4 a = *reinterpret_cast<const float4 *>(&qs[h * D + 8 * oc]);
        const float4 b = *reinterpret_cast<const float4 *>(&qs[h * D + 8 * oc + 4]);
        qr[h][0] = a.x; qr[h][1] = a.y; qr[h][2] = a.z; qr[h][3] = a.w;
        qr[h][4] = b.x; qr[h][5] = b.y; qr[h][6] = b.z; qr[h][7] = b.w;
    }

    // ---- scores ----
#pragma unroll
    for (int i = 0; i < NIK; ++i) {
        const int tt = ps * nik + i;
        if (i < nik && tt < tn) {                  // uniform over the LPP lanes of a position
            float kv[8];
            if (owns_new && t0 + tt == pos) {
#pragma unroll
                for (int e = 0; e < 8; ++e) kv[e] = kn[8 * oc + e];
            } else {
                const uint32_t w[4] = {kr[i].x, kr[i].y, kr[i].z, kr[i].w};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    kv[2 * e] = h_lo(w[e]);
                    kv[2 * e + 1] = h_hi(w[e]);
                }
            }
#pragma unroll
            for (int h = 0; h < G; ++h) {
                float s = 0.f;
#pragma unroll
                for (int e = 0; e < 8; ++e) s = fmaf(qr[h][e], kv[e], s);
                s = group_sum<LPP>(s);
                if (oc == 0) p[h][tt] = s;
            }
        }
    }
    __syncthreads();

    // ---- chunk softmax statistics, one wave per head ----
    const int lane = tid & 63, wave = tid >> 6;
    for (int h = wave; h < G; h += kAttnThreads / 64) {
        float m = -INFINITY;
        for (int tt = lane; tt < tn; tt += 64) m = fmaxf(m, p[h][tt]);
        m = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wave_max_to_lane63(m)), 63));
        float l = 0.f;
        for (int tt = lane; tt < tn; tt += 64) {
            const float e = expf(p[h][tt] - m);
            p[h][tt] = e;
            l += e;
        }
        l = wave_sum_to_lane63(l);
        if (lane == 63) {
            stat[h][0] = m;
            stat[h][1] = l;
        }
    }
    __syncthreads();

    // ---- unnormalized o = sum_t p_t v_t over this thread's positions ----
    float o[G][4];
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
        for (int e = 0; e < 4; ++e) o[h][e] = 0.f;
#pragma unroll
    for (int i = 0; i < NIV; ++i) {
        const int tt = vs * niv + i;
        if (i < niv && tt < tn) {
            float v[4];
            if (owns_new && t0 + tt == pos) {
#pragma unroll
                for (int e = 0; e < 4; ++e) v[e] = vn[4 * dq + e];
            } else {
                v[0] = h_lo(vr[i].x);
                v[1] = h_hi(vr[i].x);
                v[2] = h_lo(vr[i].y);
                v[3] = h_hi(vr[i].y);
            }
#pragma unroll
            for (int h = 0; h < G; ++h) {
                const float pt = p[h][tt];
#pragma unroll
                for (int e = 0; e < 4; ++e) o[h][e] = fmaf(pt, v[e], o[h][e]);
            }
        }
    }
#pragma unroll
    for (int h = 0; h < G; ++h)
        *reinterpret_cast<float4 *>(&red[vs][h][4 * dq]) = make_float4(o[h][0], o[h][1], o[h][2], o[h][3]);
    __syncthreads();

    // partial record per (g, h, c): [max, sum, o[0..D)], subsets added in order
    const int nchunks = gridDim.x;
    for (int k = tid; k < G * D; k += kAttnThreads) {
        const int h = k / D, d = k % D;
        float s = 0.f;
#pragma unroll
        for (int j = 0; j < NVS; ++j) s += red[j][h][d];
        float *rec = part + ((int64_t(g) * G + h) * nchunks + c) * (D + 2);
        rec[2 + d] = s;
        if (d == 0) {
            rec[0] = stat[h][0];
            rec[1] = stat[h][1];
        }
    }
}

// grid n_q_heads, 512 threads: thread (d, grp) adds the chunks c = grp mod NG
// of head h; the groups are then added in order.
template <int D>
__global__ void __launch_bounds__(kMergeThreads) attn_merge_kernel(const float *__restrict__ part,
                                                                   const int32_t *__restrict__ d_pos, int ctx_cap,
                                                                   int chunk, int nchunks, float *__restrict__ out) {
    constexpr int NG = kMergeThreads / D;
    extern __shared__ float msm[];               // w[nchunks] | ored[NG][D] | scal[2]
    float *w = msm;
    float *ored = w + nchunks;
    float *scal = ored + NG * D;
    const int h = blockIdx.x, tid = threadIdx.x, d = tid % D, grp = tid / D;
    const int pos = *d_pos;
    if (pos < 0 || pos >= ctx_cap) {
        if (grp == 0) out[h * D + d] = __int_as_float(0x7fc00000);
        return;
    }
    const int nact = pos / chunk + 1;
    const float *base = part + int64_t(h) * nchunks * (D + 2);
    // chunk maxima -> weights (wave 0, lanes strided over the chunks)
    if (tid < 64) {
        float m = -INFINITY;
        for (int c = tid; c < nact; c += 64) m = fmaxf(m, base[int64_t(c) * (D + 2)]);
        m = wave_max(m);
        float l = 0.f;
        for (int c = tid; c < nact; c += 64) {
            const float e = expf(base[int64_t(c) * (D + 2)] - m);
            w[c] = e;
            l = fmaf(base[int64_t(c) * (D + 2) + 1], e, l);
        }
        l = wave_sum(l);
        if (tid == 0) scal[0] = l;
    }
    __syncthreads();
    float o = 0.f;
#pragma unroll 8
    for (int c = grp; c < nact; c += NG) o = fmaf(base[int64_t(c) * (D + 2) + 2 + d], w[c], o);
    ored[grp * D + d] = o;
    __syncthreads();
    if (grp == 0) {
        float s = 0.f;
#pragma unroll
        for (int j = 0; j < NG; ++j) s += ored[j * D + d];
        out[h * D + d] = s / scal[0];
    }
}

template <int D, int G>
hipError_t launch_dg(const nt_attn_desc &a, int chunk, int nchunks, const float *q, const float *k_new,
                     const float *v_new, uint16_t *kc, uint16_t *vc, const int32_t *d_pos, float *out,
                     float *part, hipStream_t st) {
    const float scale = a.scale > 0.f ? a.scale : 1.0f / sqrtf(float(D));
    RopeFreq f{};
    const bool rope = a.rope_theta > 0.f;
    if (rope)
        for (int i = 0; i < D / 2; ++i) f.w[i] = std::pow(double(a.rope_theta), -2.0 * double(i) / double(D));
    attn_split_kernel<D, G><<<dim3(nchunks, a.n_kv_heads), kAttnThreads, 0, st>>>(
        q, k_new, v_new, kc, vc, d_pos, a.ctx_cap, chunk, scale, rope, f, part);
    const size_t lds = (size_t(nchunks) + size_t(kMergeThreads) + 2) * sizeof(float);
    attn_merge_kernel<D><<<a.n_q_heads, kMergeThreads, lds, st>>>(part, d_pos, a.ctx_cap, chunk, nchunks, out);
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
    // Positions per workgroup: the split kernel is bound by its arithmetic
    // and latency, not by bandwidth, so the chunk is chosen for the busiest
    // CU: at full context the (kv head, chunk) workgroups come to a whole
    // number per CU of a 256-CU part: two, e.g. 65 positions for 8 kv heads
    // at 4160 (512 workgroups instead of 520 at 64, where 8 CUs ran a third
    // one), or one where two would leave a workgroup fewer than 128
    // (position, q head) pairs, e.g. 36 positions of 4 heads at 1152, where
    // the fixed cost per workgroup dominates (measured: 8 kv heads of 8 q
    // heads at 4160, 65 vs 64: -1.0 % decode time; of 4 q heads at 1152, 36
    // vs 18 and 32: -0.8 %).
    const int kv = std::max(1, a.n_kv_heads), G = std::max(1, a.n_q_heads / kv);
    int per_head = std::max(1, 512 / kv);
    int c = (a.ctx_cap + per_head - 1) / per_head;
    if (c * G < 128) {
        per_head = std::max(1, 256 / kv);
        c = (a.ctx_cap + per_head - 1) / per_head;
    }
    return std::min(kMaxChunk, std::max(8, c));
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
