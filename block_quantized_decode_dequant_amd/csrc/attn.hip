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
// workgroups fill the chip.  A workgroup first issues asynchronous copies of
// its chunk's K and V rows into LDS, then computes the G heads' scores, their
// chunk-local softmax statistics and the unnormalized weighted sum of V (both
// products on the matrix cores), and leaves (max, sum, o[D]) per head.  A
// merge kernel combines the chunks with the log-sum-exp rule in a fixed order
// (deterministic).  The current token's k and v are stored at slot pos
// (rounded to fp16) by the workgroup that owns that slot, which attends to the
// rounded values, so the cache and the attention agree.  A position outside
// [0, ctx_cap) writes NaN outputs and touches no memory out of bounds.
#include <algorithm>
#include <atomic>
#include <cmath>

#include "device_util.h"
#include "nt_internal.h"

namespace nt {
namespace {

constexpr int kAttnThreads = 256;
constexpr int kMaxChunk = 128;
constexpr int kMergeThreads = 512;

// RoPE frequency of pair i, theta^(-2i/D) = 2^(i * c) with c = -2 log2(theta) / D
// formed in fp64 on the host: computed in registers, so the rotation needs
// no memory access (a table indexed per lane would be read from memory, one
// round trip behind every K and V load of the chunk).
__device__ __forceinline__ double rope_freq(int i, double c) { return exp2(double(i) * c); }

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

typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef uint32_t w2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ h4 as_h4(uint32_t lo, uint32_t hi) { return __builtin_bit_cast(h4, w2{lo, hi}); }

// s_waitcnt vmcnt(n) for a wave-uniform n in [0, 16] (the immediate must be
// a constant, so a uniform branch picks it).
__device__ __forceinline__ void wait_vm(int n) {
    switch (n) {
    case 0: __builtin_amdgcn_s_waitcnt(vmcnt_imm(0)); break;
    case 1: __builtin_amdgcn_s_waitcnt(vmcnt_imm(1)); break;
    case 2: __builtin_amdgcn_s_waitcnt(vmcnt_imm(2)); break;
    case 3: __builtin_amdgcn_s_waitcnt(vmcnt_imm(3)); break;
    case 4: __builtin_amdgcn_s_waitcnt(vmcnt_imm(4)); break;
    case 5: __builtin_amdgcn_s_waitcnt(vmcnt_imm(5)); break;
    case 6: __builtin_amdgcn_s_waitcnt(vmcnt_imm(6)); break;
    case 7: __builtin_amdgcn_s_waitcnt(vmcnt_imm(7)); break;
    case 8: __builtin_amdgcn_s_waitcnt(vmcnt_imm(8)); break;
    case 9: __builtin_amdgcn_s_waitcnt(vmcnt_imm(9)); break;
    case 10: __builtin_amdgcn_s_waitcnt(vmcnt_imm(10)); break;
    case 11: __builtin_amdgcn_s_waitcnt(vmcnt_imm(11)); break;
    case 12: __builtin_amdgcn_s_waitcnt(vmcnt_imm(12)); break;
    case 13: __builtin_amdgcn_s_waitcnt(vmcnt_imm(13)); break;
    case 14: __builtin_amdgcn_s_waitcnt(vmcnt_imm(14)); break;
    case 15: __builtin_amdgcn_s_waitcnt(vmcnt_imm(15)); break;
    default: __builtin_amdgcn_s_waitcnt(vmcnt_imm(16)); break;
    }
    __builtin_amdgcn_sched_barrier(0);
}

// Max / sum over the 16 lanes of a DPP row (every lane of the row gets it).
__device__ __forceinline__ float row16_max(float v) {
    v = fmaxf(v, dpp_keep<0x128>(v));    // row_ror:8
    v = fmaxf(v, dpp_keep<0x124>(v));    // row_ror:4
    v = fmaxf(v, dpp_keep<0x122>(v));    // row_ror:2
    v = fmaxf(v, dpp_keep<0x121>(v));    // row_ror:1
    return v;
}
__device__ __forceinline__ float row16_sum(float v) {
    v += dpp_keep<0x128>(v);
    v += dpp_keep<0x124>(v);
    v += dpp_keep<0x122>(v);
    v += dpp_keep<0x121>(v);
    return v;
}

// LDS layout of one workgroup (dynamic; cpw = copies per wave of K, and of V,
// 1 KB each, so a chunk of at most 4 * cpw * R rows with R = 1024 / (2 D)):
//   K rows, V rows: [4 cpw KB each] fp16, row t's 16-byte piece c stored at
//     slot c ^ (t mod 8 or 16) (so the 16 lanes of one MFMA row group, which
//     read one piece of 16 different rows, hit different banks);
//   qraw [G D] fp32 (q as loaded), then rotated and scaled in place;
//   knew, vnew [D] fp32 as loaded; knh, vnh [D] fp16 (rotated k, v as stored);
//   p [G][4 cpw R] fp32 softmax weights; stat [2][4 waves][8] fp32.
template <int D> struct AttnLds {
    static constexpr int kRowBytes = 2 * D;
    static constexpr int kRowsPerCopy = 1024 / kRowBytes;
    static constexpr int kPieces = kRowBytes / 16;              // 16 (D 128) or 8 (D 64)
};

// K and V rows
__host__ __device__ constexpr size_t attn_rows_bytes(int D, int G, int cpw) {
    return (void)D, (void)G, size_t(2) * 4 * cpw * 1024;
}

__host__ __device__ constexpr size_t attn_lds_bytes(int D, int G, int cpw) {
    return attn_rows_bytes(D, G, cpw)                            // K, V rows / P V sums
           + size_t(G) * D * 4                                   // qraw
           + size_t(2) * D * 4 + size_t(2) * D * 2               // knew, vnew, knh, vnh
           + size_t(4) * cpw * (1024 / (2 * D)) * G * 4          // p
           + 2 * 4 * 8 * 4;                                      // stat
}

// grid (chunks, n_kv_heads), 256 threads; D = head_dim, G = q heads per kv
// head; chunk <= 4 cpw R positions.  Per workgroup: asynchronous copies of
// the chunk's K and V rows (and of q, k_new, v_new) into LDS; q rotated by
// RoPE and scaled; scores on the matrix cores (v_mfma_f32_16x16x16_f16: M =
// q heads, N = 16 positions, K = 16 dims; q split into fp16 hi + lo parts,
// two MFMAs per step, so the scores carry ~2^-22 relative error; K is fp16
// already); chunk softmax statistics by 16-lane DPP reductions; P V on the
// matrix cores too (M = q heads, N = 16 dims, K = 16 positions, p split into
// fp16 hi + lo parts); the partial record per head.
template <int D, int G>
__global__ void __launch_bounds__(kAttnThreads) attn_split_kernel(
    const float *__restrict__ q, const float *__restrict__ k_new, const float *__restrict__ v_new,
    uint16_t *__restrict__ kc, uint16_t *__restrict__ vc, const int32_t *__restrict__ d_pos, int ctx_cap,
    int chunk, int cpw, float scale, bool rope, double rope_c, float *__restrict__ part) {
    using L = AttnLds<D>;
    constexpr int RPC = L::kRowsPerCopy, NP = L::kPieces, SWZ = NP - 1;
    constexpr int KSTEPS = D / 16;            // MFMA steps over the head dimension
    constexpr int DG = D / 4;                 // dims per lane group (4 groups)
    extern __shared__ __attribute__((aligned(16))) uint8_t sm[];
    const int rows_cap = 4 * cpw * RPC;
    uint8_t *const k_rows = sm;
    uint8_t *const v_rows = sm + 4 * cpw * 1024;
    float *const qraw = reinterpret_cast<float *>(sm + attn_rows_bytes(D, G, cpw));
    float *const knew = qraw + G * D;
    float *const vnew = knew + D;
    uint16_t *const knh = reinterpret_cast<uint16_t *>(vnew + D);
    uint16_t *const vnh = knh + D;
    float *const psh = reinterpret_cast<float *>(vnh + D);            // [G][rows_cap]
    float *const stat = psh + rows_cap * G;                          // [2][4][8]

    const int c = blockIdx.x, g = blockIdx.y, tid = threadIdx.x;
    const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int t0 = c * chunk;
    const int64_t head_base = int64_t(g) * ctx_cap * D;

    // ---- 1. asynchronous copies: wave 0 also fetches q (G D floats) and the
    // new k, v (D floats each); then every wave its cpw pieces of K and V.
    // Copy k covers rows [R k, R k + R) of the chunk; row t of the chunk comes
    // from cache row min(t0 + t, t0 + chunk - 1, ctx_cap - 1) (rows past the
    // chunk repeat its last row: cache hits, never used).
    if (wave == 0) {
        const uint8_t *qg = reinterpret_cast<const uint8_t *>(q + int64_t(g) * G * D);
        constexpr int QB = G * D * 4;                 // bytes of q
#pragma unroll
        for (int k = 0; k < (QB + 1023) / 1024; ++k)
            if (1024 * k + 16 * lane < QB) dma<16>(qg, uint32_t(1024 * k + 16 * lane), lds_addr(qraw) + 1024 * k);
        if (k_new && lane < D / 4) {               // D floats = D / 4 pieces of 16 bytes each
            dma<16>(reinterpret_cast<const uint8_t *>(k_new + int64_t(g) * D), uint32_t(16 * lane), lds_addr(knew));
            dma<16>(reinterpret_cast<const uint8_t *>(v_new + int64_t(g) * D), uint32_t(16 * lane), lds_addr(vnew));
        }
    }
    {
        const int last = min(t0 + chunk, ctx_cap) - 1;
        const uint8_t *kb = reinterpret_cast<const uint8_t *>(kc + head_base);
        const uint8_t *vb = reinterpret_cast<const uint8_t *>(vc + head_base);
        for (int k = 0; k < cpw; ++k) {
            const int cp = wave * cpw + k;                       // copy index, rows [R cp, R cp + R)
            const int rl = cp * RPC + lane / NP;                 // chunk row of this lane's piece
            const int slot = lane % NP;
            const int piece = slot ^ (rl & SWZ);
            const uint32_t off = uint32_t(min(t0 + rl, last)) * uint32_t(2 * D) + uint32_t(piece) * 16u;
            dma<16, true>(kb, off, lds_addr(k_rows) + 1024 * cp);
        }
        for (int k = 0; k < cpw; ++k) {
            const int cp = wave * cpw + k;
            const int rl = cp * RPC + lane / NP;
            const int slot = lane % NP;
            const int piece = slot ^ (rl & SWZ);
            const uint32_t off = uint32_t(min(t0 + rl, last)) * uint32_t(2 * D) + uint32_t(piece) * 16u;
            dma<16, true>(vb, off, lds_addr(v_rows) + 1024 * cp);
        }
    }

    const int pos = *d_pos;
    if (pos < 0 || pos >= ctx_cap || t0 > pos) {    // invalid (the merge writes NaNs) or chunk not reached
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));   // leave with no copy into LDS outstanding
        return;
    }
    const int tn = min(chunk, pos + 1 - t0);        // positions of this chunk to attend
    const bool owns_new = k_new && pos < t0 + chunk;
    const int new_row = pos - t0;                   // chunk row of the new token (when owned)

    // ---- RoPE angle of pair i: pos * w_i in fp64, reduced to [-pi, pi] in
    // fp64, then an fp32 sincos (the reduced angle is exact to ~1e-7 rad) ----
    const auto angle = [&](int i, float &cn, float &sn) {
        const double ph = double(pos) * rope_freq(i, rope_c);
        const double r = fma(-6.283185307179586, rint(ph * 0.15915494309189535), ph);
        sincosf(float(r), &sn, &cn);
    };
    // the angles need only the position: formed while the copies land
    constexpr int QPAIRS = G * D / 2;
    constexpr int QPT = (QPAIRS + kAttnThreads - 1) / kAttnThreads;   // q pairs per thread
    float qc[QPT], qs_[QPT], kcs = 1.f, ksn = 0.f;
#pragma unroll
    for (int m = 0; m < QPT; ++m) {
        qc[m] = 1.f;
        qs_[m] = 0.f;
        const int pr = tid + m * kAttnThreads;
        if (rope && pr < QPAIRS) angle(pr % (D / 2), qc[m], qs_[m]);
    }
    if (rope && owns_new && tid < D / 2) angle(tid, kcs, ksn);

    // ---- 2. q (and k_new, v_new) landed: rotate and scale q in place; the
    // owner rounds the new k, v to fp16, stores them in the cache and keeps
    // them for the substitution of its row below
    if (wave == 0) wait_vm(2 * cpw);
    __syncthreads();
#pragma unroll
    for (int m = 0; m < QPT; ++m) {
        const int pr = tid + m * kAttnThreads;
        if (pr < QPAIRS) {
            const float x0 = qraw[2 * pr], x1 = qraw[2 * pr + 1];
            qraw[2 * pr] = (x0 * qc[m] - x1 * qs_[m]) * scale;
            qraw[2 * pr + 1] = (x0 * qs_[m] + x1 * qc[m]) * scale;
        }
    }
    if (owns_new && tid < D / 2) {
        const float a = knew[2 * tid], b = knew[2 * tid + 1];
        const float k0 = a * kcs - b * ksn, k1 = a * ksn + b * kcs;
        const uint16_t kb0 = f2h_bits(k0), kb1 = f2h_bits(k1);
        const uint16_t vb0 = f2h_bits(vnew[2 * tid]), vb1 = f2h_bits(vnew[2 * tid + 1]);
        const int64_t at = head_base + int64_t(pos) * D + 2 * tid;
        *reinterpret_cast<uint32_t *>(kc + at) = uint32_t(kb0) | (uint32_t(kb1) << 16);
        *reinterpret_cast<uint32_t *>(vc + at) = uint32_t(vb0) | (uint32_t(vb1) << 16);
        knh[2 * tid] = kb0;
        knh[2 * tid + 1] = kb1;
        vnh[2 * tid] = vb0;
        vnh[2 * tid + 1] = vb1;
    }
    __syncthreads();

    // ---- 3. the MFMA A operand: lane (row i = lane % 16, group j = lane / 16)
    // holds q head i's dims [DG j + 4 s, +4) for step s, as fp16 hi and lo
    const int arow = lane & 15, grp = lane >> 4;
    h4 a_hi[KSTEPS], a_lo[KSTEPS];
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) {
        float x[4] = {0.f, 0.f, 0.f, 0.f};
        if (arow < G) {
            const float4 v = *reinterpret_cast<const float4 *>(&qraw[arow * D + DG * grp + 4 * s]);
            x[0] = v.x; x[1] = v.y; x[2] = v.z; x[3] = v.w;
        }
        _Float16 hi[4], lo[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            hi[e] = _Float16(x[e]);
            lo[e] = _Float16(x[e] - float(hi[e]));
        }
        a_hi[s] = h4{hi[0], hi[1], hi[2], hi[3]};
        a_lo[s] = h4{lo[0], lo[1], lo[2], lo[3]};
    }

    // ---- 4. scores: wave w takes the 16-row tiles w, w + 4 of the chunk
    wait_vm(cpw);                                    // this wave's K copies have landed
    __syncthreads();                                 // ... and every wave's
    const int ntiles = (tn + 15) >> 4;
    float sc[2][4];
    float mx[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
    // every B operand of both tiles is read from LDS before the first MFMA
    uint4 kb[2][KSTEPS / 2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int tile = wave + 4 * u;
        const int row = min(16 * tile + arow, rows_cap - 1);   // this lane's position (B column)
        const bool fresh = owns_new && row == new_row;
#pragma unroll
        for (int s2 = 0; s2 < KSTEPS / 2; ++s2) {
            // 8 dims = steps 2 s2 and 2 s2 + 1: one 16-byte piece
            const int piece = (DG * grp + 8 * s2) / 8;
            const uint8_t *src = fresh ? reinterpret_cast<const uint8_t *>(knh) + 16 * piece
                                       : k_rows + row * (2 * D) + 16 * (piece ^ (row & SWZ));
            kb[u][s2] = tile < ntiles ? *reinterpret_cast<const uint4 *>(src) : uint4{0u, 0u, 0u, 0u};
        }
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int tile = wave + 4 * u;
        f4 acc = {0.f, 0.f, 0.f, 0.f};
        if (tile < ntiles) {
#pragma unroll
            for (int s2 = 0; s2 < KSTEPS / 2; ++s2) {
                const h4 b0 = as_h4(kb[u][s2].x, kb[u][s2].y), b1 = as_h4(kb[u][s2].z, kb[u][s2].w);
                acc = __builtin_amdgcn_mfma_f32_16x16x16f16(a_hi[2 * s2], b0, acc, 0, 0, 0);
                acc = __builtin_amdgcn_mfma_f32_16x16x16f16(a_lo[2 * s2], b0, acc, 0, 0, 0);
                acc = __builtin_amdgcn_mfma_f32_16x16x16f16(a_hi[2 * s2 + 1], b1, acc, 0, 0, 0);
                acc = __builtin_amdgcn_mfma_f32_16x16x16f16(a_lo[2 * s2 + 1], b1, acc, 0, 0, 0);
            }
        }
        // lane holds position 16 tile + lane % 16 for heads 4 grp + e
        const bool valid = tile < ntiles && 16 * tile + arow < tn;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            sc[u][e] = valid ? acc[e] : -INFINITY;
            mx[e] = fmaxf(mx[e], sc[u][e]);
        }
    }
    // chunk maxima per head: 16-lane rows, then across the waves through LDS
#pragma unroll
    for (int e = 0; e < 4; ++e) mx[e] = row16_max(mx[e]);
    if (arow == 0 && 4 * grp < G) {
#pragma unroll
        for (int e = 0; e < 4; ++e)
            if (4 * grp + e < G) stat[wave * 8 + 4 * grp + e] = mx[e];
    }
    __syncthreads();
    float M[4], lsum[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int h = min(4 * grp + e, G - 1);
        M[e] = fmaxf(fmaxf(stat[h], stat[8 + h]), fmaxf(stat[16 + h], stat[24 + h]));
        lsum[e] = 0.f;
    }
    // weights p = exp(s - M) into LDS [head][position], and their sums
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int tile = wave + 4 * u;
        const int row = 16 * tile + arow;
        if (tile < ntiles) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float pv = sc[u][e] == -INFINITY ? 0.f : expf(sc[u][e] - M[e]);
                lsum[e] += pv;
                if (4 * grp + e < G) psh[(4 * grp + e) * rows_cap + row] = pv;
            }
        }
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) lsum[e] = row16_sum(lsum[e]);
    if (arow == 0 && 4 * grp < G) {
#pragma unroll
        for (int e = 0; e < 4; ++e)
            if (4 * grp + e < G) stat[32 + wave * 8 + 4 * grp + e] = lsum[e];
    }

    // ---- 5. O = P V on the matrix cores: M = q heads, N = 16 dims, K = 16
    // positions; p split into fp16 hi + lo (two MFMAs per step), V fp16.
    // Wave w owns the dim tiles w, w + 4 (all positions), so every output
    // value is complete in one wave: A (p) lane (head i = lane % 16, group j)
    // holds positions 16 step + 4 j .. + 3, B (V) lane (dim lane % 16, group
    // j) the same positions of its dim; D lane: dim lane % 16, heads 4 j + e.
    wait_vm(0);                                      // this wave's V copies have landed
    __syncthreads();                                 // ... and every wave's; p and sums visible
    constexpr int DT = D / 16;                       // dim tiles
    constexpr int TPW = (DT + 3) / 4;                // dim tiles per wave
    const int nsteps = ntiles;                       // 16-position steps
    f4 oacc[TPW];
#pragma unroll
    for (int u = 0; u < TPW; ++u) oacc[u] = f4{0.f, 0.f, 0.f, 0.f};
    for (int st = 0; st < nsteps; ++st) {
        const int tb = 16 * st + 4 * grp;            // first of this lane's 4 positions
        float pa[4] = {0.f, 0.f, 0.f, 0.f};
        if (arow < G) {
            const float4 pp = *reinterpret_cast<const float4 *>(&psh[arow * rows_cap + tb]);
            pa[0] = pp.x; pa[1] = pp.y; pa[2] = pp.z; pa[3] = pp.w;
        }
        _Float16 phi[4], plo[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            phi[e] = _Float16(pa[e]);
            plo[e] = _Float16(pa[e] - float(phi[e]));
        }
        const h4 ahi = h4{phi[0], phi[1], phi[2], phi[3]}, alo = h4{plo[0], plo[1], plo[2], plo[3]};
#pragma unroll
        for (int u = 0; u < TPW; ++u) {
            const int dt = wave + 4 * u;
            if (dt < DT) {
                const int d = 16 * dt + arow;        // this lane's dim
                _Float16 vb[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int t = tb + e;
                    const bool fresh = owns_new && t == new_row;
                    const uint8_t *src = fresh ? reinterpret_cast<const uint8_t *>(vnh) + 2 * d
                                               : v_rows + t * (2 * D) + 16 * ((d >> 3) ^ (t & SWZ)) + 2 * (d & 7);
                    vb[e] = *reinterpret_cast<const _Float16 *>(src);
                }
                const h4 b = h4{vb[0], vb[1], vb[2], vb[3]};
                oacc[u] = __builtin_amdgcn_mfma_f32_16x16x16f16(ahi, b, oacc[u], 0, 0, 0);
                oacc[u] = __builtin_amdgcn_mfma_f32_16x16x16f16(alo, b, oacc[u], 0, 0, 0);
            }
        }
    }

    // partial record per (g, h, c): [max, sum, o[0..D)] (rows past tn have p = 0)
    const int nchunks = gridDim.x;
#pragma unroll
    for (int u = 0; u < TPW; ++u) {
        const int dt = wave + 4 * u;
        if (dt < DT && 4 * grp < G) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int h = 4 * grp + e;
                if (h < G) part[((int64_t(g) * G + h) * nchunks + c) * (D + 2) + 2 + 16 * dt + arow] = oacc[u][e];
            }
        }
    }
    if (tid < G) {
        const int h = tid;
        float *rec = part + ((int64_t(g) * G + h) * nchunks + c) * (D + 2);
        rec[0] = fmaxf(fmaxf(stat[h], stat[8 + h]), fmaxf(stat[16 + h], stat[24 + h]));
        rec[1] = (stat[32 + h] + stat[40 + h]) + (stat[48 + h] + stat[56 + h]);
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

// K (and V) copies per wave: each copy moves 1 KB, i.e. 1024 / (2 D) rows;
// four waves cover the chunk.
int attn_copies_per_wave(int D, int chunk) {
    const int rows_per_copy = 1024 / (2 * D);
    return (chunk + 4 * rows_per_copy - 1) / (4 * rows_per_copy);
}

template <int D, int G>
hipError_t launch_dg(const nt_attn_desc &a, int chunk, int nchunks, const float *q, const float *k_new,
                     const float *v_new, uint16_t *kc, uint16_t *vc, const int32_t *d_pos, float *out,
                     float *part, hipStream_t st) {
    const float scale = a.scale > 0.f ? a.scale : 1.0f / sqrtf(float(D));
    const bool rope = a.rope_theta > 0.f;
    const double rope_c = rope ? -2.0 * std::log2(double(a.rope_theta)) / double(D) : 0.0;
    const int cpw = attn_copies_per_wave(D, chunk);
    const size_t lds_split = attn_lds_bytes(D, G, cpw);
    if (lds_split > 65536) {
        // the largest chunks need more than 64 KB of dynamic LDS: allowed once
        // per device (a repeated setting is harmless)
        static std::atomic<uint64_t> done{0};
        int dev = 0;
        if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
        if (!((done.load(std::memory_order_acquire) >> dev) & 1)) {
            if (hipFuncSetAttribute(reinterpret_cast<const void *>(&attn_split_kernel<D, G>),
                                    hipFuncAttributeMaxDynamicSharedMemorySize, int(attn_lds_bytes(D, G, 8))) !=
                hipSuccess)
                (void)hipGetLastError();        // a launch that still exceeds the limit reports it
            done.fetch_or(uint64_t(1) << dev, std::memory_order_release);
        }
    }
    attn_split_kernel<D, G><<<dim3(nchunks, a.n_kv_heads), kAttnThreads, lds_split, st>>>(
        q, k_new, v_new, kc, vc, d_pos, a.ctx_cap, chunk, cpw, scale, rope, rope_c, part);
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
