// gemv.hip -- fused dequantize + matrix-vector product for batch-1 decode,
// y = W x (+ y), over GGUF-style block-quantized W.
//
// The ntransformer write-up ("Architecture") names GEMV as the engine's core
// kernel: at batch 1 every weight byte is read once per token, so the
// product is bound by HBM bandwidth, not by arithmetic, and MFMA does not
// apply (there is no reuse to feed a matrix core).  The design is for gfx950:
//
//  * A "unit" is 32 consecutive codes of one row handled by one lane: one
//    Q8_0 / Q4_0 block, or one eighth of a Q4_K / Q6_K super-block.  Lane
//    `l` of wave `w` owns the same units in every row (column-stationary), so
//    the 32 activations of its unit are loaded once into registers, with the
//    per-unit activation sums the offset tricks below need.
//  * Consecutive lanes own consecutive units, so one wave instruction reads a
//    contiguous run of the row: 128-bit loads for the 16-byte-aligned Q4_K
//    chunks, and word-aligned 128/96/32-bit loads plus a per-lane byte
//    funnel (v_perm_b32) for the 2-byte-aligned Q8_0, Q4_0 and Q6_K blocks.
//  * Codes are unpacked in registers (masks and shifts on whole words) and
//    converted with byte-to-float conversions; constant offsets are taken
//    out of the inner loop: sum d*(q-o)*x = d*(sum q*x - o*sum x).
//  * A wave works on R rows at once (R independent load streams in flight),
//    reduces each row over its 64 lanes, and the waves of a workgroup (one
//    per 2048-column slice) combine their partial sums through LDS in a fixed
//    order.  No atomics: results are deterministic.
#include <cstdlib>

#include "device_util.h"
#include "nt_internal.h"

namespace nt {
namespace {

constexpr uint32_t kLo4 = 0x0f0f0f0fu;

// ---- Q8_0: one unit = one 34-byte block ------------------------------------
struct Q80 {
    static constexpr int kBlockElems = 32, kBlockBytes = 34;
    struct Raw { u32x4 a, b; uint32_t c, sh; };
    struct X { float v[32]; float sum; };

    __device__ static void load_x(const float *x, int64_t unit, X &xs) {
        const float4 *p = reinterpret_cast<const float4 *>(x + unit * 32);
        float s = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            float4 v = p[i];
            xs.v[4 * i] = v.x; xs.v[4 * i + 1] = v.y; xs.v[4 * i + 2] = v.z; xs.v[4 * i + 3] = v.w;
            s += (v.x + v.y) + (v.z + v.w);
        }
        xs.sum = s;
    }
    // g: global block index (row * blocks_per_row + unit)
    __device__ static void load(const uint8_t *W, int64_t g, Raw &r) {
        const int64_t off = g * 34;
        r.sh = uint32_t(off & 3);
        const uint8_t *p = W + (off - r.sh);
        r.a = ld4(p); r.b = ld4(p + 16); r.c = ld1(p + 32);
    }
    __device__ static float dot(const Raw &r, const X &xs) {
        const uint32_t w[9] = {r.a.x, r.a.y, r.a.z, r.a.w, r.b.x, r.b.y, r.b.z, r.b.w, r.c};
        const float d = h2f(w[0] >> (8 * r.sh));
        // codes start at byte sh+2 of w: 2 -> bytes 2..5 of w[i+1]:w[i], 4 -> w[i+1]
        const uint32_t sel = r.sh ? 0x07060504u : 0x05040302u;
        float s = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            // flipping the sign bit turns int8 q into unsigned q + 128
            const uint32_t u = funnel(w[i + 1], w[i], sel) ^ 0x80808080u;
            s = fmaf(ubyte<0>(u), xs.v[4 * i + 0], s);
            s = fmaf(ubyte<1>(u), xs.v[4 * i + 1], s);
            s = fmaf(ubyte<2>(u), xs.v[4 * i + 2], s);
            s = fmaf(ubyte<3>(u), xs.v[4 * i + 3], s);
        }
        return d * fmaf(-128.f, xs.sum, s);
    }
};

// ---- Q4_0: one unit = one 18-byte block -------------------------------------
struct Q40 {
    static constexpr int kBlockElems = 32, kBlockBytes = 18;
    struct Raw { u32x4 a; uint32_t c, sh; };
    // v[i]: value i of the block = low nibble of byte i (i < 16) or high
    // nibble of byte i - 16, so the activations load exactly as for Q8_0
    using X = Q80::X;

    __device__ static void load_x(const float *x, int64_t unit, X &xs) { Q80::load_x(x, unit, xs); }
    __device__ static void load(const uint8_t *W, int64_t g, Raw &r) {
        const int64_t off = g * 18;
        r.sh = uint32_t(off & 3);
        const uint8_t *p = W + (off - r.sh);
        r.a = ld4(p); r.c = ld1(p + 16);
    }
    __device__ static float dot(const Raw &r, const X &xs) {
        const uint32_t w[5] = {r.a.x, r.a.y, r.a.z, r.a.w, r.c};
        const float d = h2f(w[0] >> (8 * r.sh));
        const uint32_t sel = r.sh ? 0x07060504u : 0x05040302u;
        float s = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t q = funnel(w[i + 1], w[i], sel);
            const uint32_t lo = q & kLo4, hi = (q >> 4) & kLo4;
            s = fmaf(ubyte<0>(lo), xs.v[4 * i + 0], s);
            s = fmaf(ubyte<1>(lo), xs.v[4 * i + 1], s);
            s = fmaf(ubyte<2>(lo), xs.v[4 * i + 2], s);
            s = fmaf(ubyte<3>(lo), xs.v[4 * i + 3], s);
            s = fmaf(ubyte<0>(hi), xs.v[16 + 4 * i + 0], s);
            s = fmaf(ubyte<1>(hi), xs.v[16 + 4 * i + 1], s);
            s = fmaf(ubyte<2>(hi), xs.v[16 + 4 * i + 2], s);
            s = fmaf(ubyte<3>(hi), xs.v[16 + 4 * i + 3], s);
        }
        return d * fmaf(-8.f, xs.sum, s);
    }
};

// ---- Q4_K: one unit = one 16-byte code chunk of a 144-byte super-block ------
// Chunk t (0..7) of super-block b holds bytes 16t..16t+15 of qs: pair p = t/2,
// half hh = t%2; low nibbles are sub-block 2p, values 64p + 16hh + i, high
// nibbles sub-block 2p+1, values 64p + 32 + 16hh + i (i = 0..15).
struct Q4K {
    static constexpr int kBlockElems = 256, kBlockBytes = 144;
    struct Raw { u32x4 hdr, q; };
    struct X { float lo[16], hi[16]; float slo, shi; uint32_t t; };

    __device__ static void load_x(const float *x, int64_t unit, X &xs) {
        const int64_t b = unit >> 3;
        const uint32_t t = uint32_t(unit & 7), p = t >> 1, hh = t & 1;
        const float4 *pl = reinterpret_cast<const float4 *>(x + b * 256 + 64 * p + 16 * hh);
        const float4 *ph = reinterpret_cast<const float4 *>(x + b * 256 + 64 * p + 32 + 16 * hh);
        float sl = 0.f, sh = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float4 a = pl[i], c = ph[i];
            xs.lo[4 * i] = a.x; xs.lo[4 * i + 1] = a.y; xs.lo[4 * i + 2] = a.z; xs.lo[4 * i + 3] = a.w;
            xs.hi[4 * i] = c.x; xs.hi[4 * i + 1] = c.y; xs.hi[4 * i + 2] = c.z; xs.hi[4 * i + 3] = c.w;
            sl += (a.x + a.y) + (a.z + a.w);
            sh += (c.x + c.y) + (c.z + c.w);
        }
        xs.slo = sl; xs.shi = sh; xs.t = t;
    }
    // g: global super-block index; unit chunk t from xs
    __device__ static void load(const uint8_t *W, int64_t g, uint32_t t, Raw &r) {
        const uint8_t *p = W + g * 144;
        r.hdr = ld4(p);
        r.q = ld4(p + 16 + 16 * t);
    }
    __device__ static float dot(const Raw &r, const X &xs) {
        const uint32_t qw[4] = {r.q.x, r.q.y, r.q.z, r.q.w};
        float s0 = 0.f, s1 = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t lo = qw[i] & kLo4, hi = (qw[i] >> 4) & kLo4;
            s0 = fmaf(ubyte<0>(lo), xs.lo[4 * i + 0], s0);
            s0 = fmaf(ubyte<1>(lo), xs.lo[4 * i + 1], s0);
            s0 = fmaf(ubyte<2>(lo), xs.lo[4 * i + 2], s0);
            s0 = fmaf(ubyte<3>(lo), xs.lo[4 * i + 3], s0);
            s1 = fmaf(ubyte<0>(hi), xs.hi[4 * i + 0], s1);
            s1 = fmaf(ubyte<1>(hi), xs.hi[4 * i + 1], s1);
            s1 = fmaf(ubyte<2>(hi), xs.hi[4 * i + 2], s1);
            s1 = fmaf(ubyte<3>(hi), xs.hi[4 * i + 3], s1);
        }
        // 6-bit scale S_j and min M_j of sub-blocks j0 = 2p and j1 = 2p+1
        const uint32_t p = xs.t >> 1;
        const uint32_t sft = 16 * (p & 1);          // byte (j & 3) of each scale word
        const uint32_t y = r.hdr.y >> sft, z = r.hdr.z >> sft, w = r.hdr.w >> sft;
        uint32_t S0, M0, S1, M1;
        if (p < 2) {
            S0 = y & 63; M0 = z & 63;
            S1 = (y >> 8) & 63; M1 = (z >> 8) & 63;
        } else {
            S0 = (w & 15) | (((y >> 6) & 3) << 4);
            M0 = ((w >> 4) & 15) | (((z >> 6) & 3) << 4);
            S1 = ((w >> 8) & 15) | (((y >> 14) & 3) << 4);
            M1 = ((w >> 12) & 15) | (((z >> 14) & 3) << 4);
        }
        const float d = h2f(r.hdr.x), dmin = h2f(r.hdr.x >> 16);
        const float pos = fmaf(float(S0), s0, float(S1) * s1);
        const float neg = fmaf(float(M0), xs.slo, float(M1) * xs.shi);
        return fmaf(d, pos, -dmin * neg);
    }
};

// ---- Q6_K: one unit = 32 values of a 210-byte super-block -------------------
// Unit t (0..7): half h = t/4, lane slot m = t%4; values 128h + 32k + 8m + i
// for k = 0..3, i = 0..7.  Bytes used: ql[64h + 8m + i] (k = 0 low, k = 2
// high nibble), ql[64h + 32 + 8m + i] (k = 1 low, k = 3 high), qh[32h + 8m + i]
// (2 bits per k), scales[8h + 2k + m/2], d.
struct Q6K {
    static constexpr int kBlockElems = 256, kBlockBytes = 210;
    struct Raw { u32x3 qa, qb, qh, sc; uint32_t dd, sh; };
    struct X { float v[4][8]; float s[4]; uint32_t t; };

    __device__ static void load_x(const float *x, int64_t unit, X &xs) {
        const int64_t b = unit >> 3;
        const uint32_t t = uint32_t(unit & 7), h = t >> 2, m = t & 3;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const float4 *p = reinterpret_cast<const float4 *>(x + b * 256 + 128 * h + 32 * k + 8 * m);
            float4 a = p[0], c = p[1];
            xs.v[k][0] = a.x; xs.v[k][1] = a.y; xs.v[k][2] = a.z; xs.v[k][3] = a.w;
            xs.v[k][4] = c.x; xs.v[k][5] = c.y; xs.v[k][6] = c.z; xs.v[k][7] = c.w;
            xs.s[k] = ((a.x + a.y) + (a.z + a.w)) + ((c.x + c.y) + (c.z + c.w));
        }
        xs.t = t;
    }
    __device__ static void load(const uint8_t *W, int64_t g, uint32_t t, Raw &r) {
        const int64_t off = g * 210;
        r.sh = uint32_t(off & 3);
        const uint8_t *p = W + (off - r.sh);
        const uint32_t h = t >> 2, m = t & 3;
        r.qa = ld3(p + 64 * h + 8 * m);
        r.qb = ld3(p + 64 * h + 32 + 8 * m);
        r.qh = ld3(p + 128 + 32 * h + 8 * m);
        r.sc = ld3(p + 192 + 8 * h);
        r.dd = ld1(p + 208);
    }
    __device__ static float dot(const Raw &r, const X &xs) {
        const uint32_t sel = shift_sel(r.sh);
        const uint32_t qa[2] = {funnel(r.qa.y, r.qa.x, sel), funnel(r.qa.z, r.qa.y, sel)};
        const uint32_t qb[2] = {funnel(r.qb.y, r.qb.x, sel), funnel(r.qb.z, r.qb.y, sel)};
        const uint32_t qh[2] = {funnel(r.qh.y, r.qh.x, sel), funnel(r.qh.z, r.qh.y, sel)};
        const uint32_t sc0 = funnel(r.sc.y, r.sc.x, sel), sc1 = funnel(r.sc.z, r.sc.y, sel);
        float s[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const uint32_t q0 = (qa[j] & kLo4) | ((qh[j] & 0x03030303u) << 4);
            const uint32_t q1 = (qb[j] & kLo4) | (((qh[j] >> 2) & 0x03030303u) << 4);
            const uint32_t q2 = ((qa[j] >> 4) & kLo4) | (((qh[j] >> 4) & 0x03030303u) << 4);
            const uint32_t q3 = ((qb[j] >> 4) & kLo4) | (((qh[j] >> 6) & 0x03030303u) << 4);
            const uint32_t qq[4] = {q0, q1, q2, q3};
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                s[k] = fmaf(ubyte<0>(qq[k]), xs.v[k][4 * j + 0], s[k]);
                s[k] = fmaf(ubyte<1>(qq[k]), xs.v[k][4 * j + 1], s[k]);
                s[k] = fmaf(ubyte<2>(qq[k]), xs.v[k][4 * j + 2], s[k]);
                s[k] = fmaf(ubyte<3>(qq[k]), xs.v[k][4 * j + 3], s[k]);
            }
        }
        // int8 scales[8h + 2k + m/2]: byte 2k + (m/2) of sc0:sc1
        const uint32_t half = (xs.t & 3) >> 1;
        const uint32_t scw0 = sc0 >> (8 * half), scw1 = sc1 >> (8 * half);
        const float c0 = float(int8_t(scw0 & 0xff)), c1 = float(int8_t((scw0 >> 16) & 0xff));
        const float c2 = float(int8_t(scw1 & 0xff)), c3 = float(int8_t((scw1 >> 16) & 0xff));
        float acc = c0 * fmaf(-32.f, xs.s[0], s[0]);
        acc = fmaf(c1, fmaf(-32.f, xs.s[1], s[1]), acc);
        acc = fmaf(c2, fmaf(-32.f, xs.s[2], s[2]), acc);
        acc = fmaf(c3, fmaf(-32.f, xs.s[3], s[3]), acc);
        return h2f(r.dd >> (8 * r.sh)) * acc;
    }
};

template <class Tr> __device__ __forceinline__ void load_raw(const uint8_t *W, int64_t row, int64_t bpr,
                                                             int64_t unit, const typename Tr::X &xs,
                                                             typename Tr::Raw &r) {
    if constexpr (Tr::kBlockElems == 32) {
        Tr::load(W, row * bpr + unit, r);
    } else {
        Tr::load(W, row * bpr + (unit >> 3), xs.t, r);
    }
}

// Generic path (any whole number of blocks per row).  One workgroup: nw
// waves x 64 lanes.  Wave w owns units [64*UPL*w, 64*UPL*(w+1)) of every row;
// the workgroup walks rows [blockIdx.x*tile, +tile) R at a time.
template <class Tr, int R, int UPL>
__global__ void __launch_bounds__(1024) gemv_generic(const uint8_t *__restrict__ W,
                                                     const float *__restrict__ x,
                                                     float *__restrict__ y, int rows,
                                                     int units_per_row, int64_t blocks_per_row,
                                                     int tile, int accumulate) {
    extern __shared__ float part[];   // [nw][tile]
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;

    typename Tr::X xs[UPL];
    int64_t unit[UPL];
    bool ok[UPL];
#pragma unroll
    for (int k = 0; k < UPL; ++k) {
        unit[k] = int64_t(wave * UPL + k) * 64 + lane;
        ok[k] = unit[k] < units_per_row;
        if (ok[k]) Tr::load_x(x, unit[k], xs[k]);
    }

    const int r0 = blockIdx.x * tile;
    for (int rr = 0; rr < tile; rr += R) {
        typename Tr::Raw raw[R][UPL];
#pragma unroll
        for (int i = 0; i < R; ++i) {
            const int r = r0 + rr + i;
#pragma unroll
            for (int k = 0; k < UPL; ++k)
                if (ok[k] && r < rows) load_raw<Tr>(W, r, blocks_per_row, unit[k], xs[k], raw[i][k]);
        }
        float acc[R];
#pragma unroll
        for (int i = 0; i < R; ++i) {
            const int r = r0 + rr + i;
            acc[i] = 0.f;
#pragma unroll
            for (int k = 0; k < UPL; ++k)
                if (ok[k] && r < rows) acc[i] += Tr::dot(raw[i][k], xs[k]);
        }
#pragma unroll
        for (int i = 0; i < R; ++i) {
            const float v = wave_sum(acc[i]);
            if (lane == 0) part[wave * tile + rr + i] = v;
        }
    }
    __syncthreads();
    for (int t = threadIdx.x; t < tile; t += blockDim.x) {
        const int r = r0 + t;
        if (r < rows) {
            float s = 0.f;
            for (int w = 0; w < nw; ++w) s += part[w * tile + t];
            y[r] = accumulate ? y[r] + s : s;
        }
    }
}

// =============================================================================
// Fast path: 64 values per lane, rows whose byte length is a multiple of 4
// (an even number of Q8_0 / Q4_0 / Q6_K blocks; any Q4_K row).  A lane's
// loads are at fixed byte offsets from the row start, so the row pointer is
// wave-uniform (scalar registers) and the per-lane part a 32-bit offset.
// =============================================================================

constexpr uint32_t kMagic16 = 0x3c003c00u;   // two fp16 1.0
constexpr uint32_t kNib16 = 0x03c003c0u;     // a nibble at fp16 fraction bits 6..9

// Two fp16 values 1 + q/16 from nibbles already shifted to bits 6..9 and
// 22..25 (v_and_or_b32 with the magic held in a VGPR).
__device__ __forceinline__ uint32_t nib_pair(uint32_t shifted, uint32_t magic) {
    return (shifted & kNib16) | magic;
}

// Sum over the 8 nibbles of w of (1 + q/16) * x: low nibbles pair with xl[0..3],
// high nibbles with xh[0..3] (byte k of w <-> index k).
__device__ __forceinline__ void nib_fma(uint32_t w, const float *xl, const float *xh, uint32_t magic,
                                        float &al, float &ah) {
    const uint32_t c0 = nib_pair(w << 6, magic);   // low nibbles of bytes 0, 2
    const uint32_t c1 = nib_pair(w >> 2, magic);   // low nibbles of bytes 1, 3
    const uint32_t c2 = nib_pair(w << 2, magic);   // high nibbles of bytes 0, 2
    const uint32_t c3 = nib_pair(w >> 6, magic);   // high nibbles of bytes 1, 3
    al = fmaf(h_lo(c0), xl[0], al);
    al = fmaf(h_lo(c1), xl[1], al);
    al = fmaf(h_hi(c0), xl[2], al);
    al = fmaf(h_hi(c1), xl[3], al);
    ah = fmaf(h_lo(c2), xh[0], ah);
    ah = fmaf(h_lo(c3), xh[1], ah);
    ah = fmaf(h_hi(c2), xh[2], ah);
    ah = fmaf(h_hi(c3), xh[3], ah);
}

__device__ __forceinline__ void load_x64(const float *x, float *v, float &sum) {
    const float4 *p = reinterpret_cast<const float4 *>(x);
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const float4 a = p[i];
        v[4 * i] = a.x; v[4 * i + 1] = a.y; v[4 * i + 2] = a.z; v[4 * i + 3] = a.w;
        s += (a.x + a.y) + (a.z + a.w);
    }
    sum = s;
}

// ---- Q8_0 fast: one lane = blocks 2u, 2u+1 (68 bytes at 68u, word-aligned) --
struct F80 {
    static constexpr int kRows = 2;
    struct L { uint32_t off; };
    struct X { float v[64]; float s0, s1; };
    struct Raw { u32x4 a, b, c, d; uint32_t e; };
    __device__ static L lane(int64_t u) { return {uint32_t(u * 68)}; }
    __device__ static void load_x(const float *x, int64_t u, X &xs) {
        float s;
        load_x64(x + u * 64, xs.v, s);
        float s0 = 0.f;
#pragma unroll
        for (int i = 0; i < 32; ++i) s0 += xs.v[i];
        xs.s0 = s0;
        xs.s1 = s - s0;
    }
    __device__ static void load(const uint8_t *row, const L &l, Raw &r) {
        const uint8_t *p = row + l.off;
        r.a = ld4(p); r.b = ld4(p + 16); r.c = ld4(p + 32); r.d = ld4(p + 48); r.e = ld1(p + 64);
    }
    __device__ static float dot(const Raw &r, const X &xs, const L &, uint32_t) {
        const uint32_t w[17] = {r.a.x, r.a.y, r.a.z, r.a.w, r.b.x, r.b.y, r.b.z, r.b.w,
                                r.c.x, r.c.y, r.c.z, r.c.w, r.d.x, r.d.y, r.d.z, r.d.w, r.e};
        float s0 = 0.f, s1 = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            // block 0: codes at bytes 2..33; flipping the sign bit gives q + 128
            const uint32_t u = __builtin_amdgcn_perm(w[i + 1], w[i], 0x05040302u) ^ 0x80808080u;
            s0 = fmaf(ubyte<0>(u), xs.v[4 * i + 0], s0);
            s0 = fmaf(ubyte<1>(u), xs.v[4 * i + 1], s0);
            s0 = fmaf(ubyte<2>(u), xs.v[4 * i + 2], s0);
            s0 = fmaf(ubyte<3>(u), xs.v[4 * i + 3], s0);
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            // block 1: codes at bytes 36..67 = words 9..16
            const uint32_t u = w[9 + i] ^ 0x80808080u;
            s1 = fmaf(ubyte<0>(u), xs.v[32 + 4 * i + 0], s1);
            s1 = fmaf(ubyte<1>(u), xs.v[32 + 4 * i + 1], s1);
            s1 = fmaf(ubyte<2>(u), xs.v[32 + 4 * i + 2], s1);
            s1 = fmaf(ubyte<3>(u), xs.v[32 + 4 * i + 3], s1);
        }
        const float d0 = h2f(w[0]), d1 = h2f(w[8] >> 16);
        return fmaf(d0, fmaf(-128.f, xs.s0, s0), d1 * fmaf(-128.f, xs.s1, s1));
    }
};

// ---- Q4_0 fast: one lane = blocks 2u, 2u+1 (36 bytes at 36u, word-aligned) --
struct F40 {
    static constexpr int kRows = 2;
    struct L { uint32_t off; };
    struct X { float v[64]; float s0, s1; };
    struct Raw { u32x4 a, b; uint32_t c; };
    __device__ static L lane(int64_t u) { return {uint32_t(u * 36)}; }
    __device__ static void load_x(const float *x, int64_t u, X &xs) {
        float s;
        load_x64(x + u * 64, xs.v, s);
        float s0 = 0.f;
#pragma unroll
        for (int i = 0; i < 32; ++i) s0 += xs.v[i];
        xs.s0 = s0;
        xs.s1 = s - s0;
    }
    __device__ static void load(const uint8_t *row, const L &l, Raw &r) {
        const uint8_t *p = row + l.off;
        r.a = ld4(p); r.b = ld4(p + 16); r.c = ld1(p + 32);
    }
    // sum over one block of (1 + q/16) x: byte i holds value i (low) and i+16 (high)
    __device__ static float block_acc(const uint32_t *q, const float *v, uint32_t magic) {
        float al = 0.f, ah = 0.f;
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const float xl[4] = {v[4 * m + 0], v[4 * m + 1], v[4 * m + 2], v[4 * m + 3]};
            const float xh[4] = {v[16 + 4 * m + 0], v[16 + 4 * m + 1], v[16 + 4 * m + 2], v[16 + 4 * m + 3]};
            nib_fma(q[m], xl, xh, magic, al, ah);
        }
        return al + ah;
    }
    __device__ static float dot(const Raw &r, const X &xs, const L &, uint32_t magic) {
        const uint32_t w[9] = {r.a.x, r.a.y, r.a.z, r.a.w, r.b.x, r.b.y, r.b.z, r.b.w, r.c};
        const uint32_t q0[4] = {__builtin_amdgcn_perm(w[1], w[0], 0x05040302u),
                                __builtin_amdgcn_perm(w[2], w[1], 0x05040302u),
                                __builtin_amdgcn_perm(w[3], w[2], 0x05040302u),
                                __builtin_amdgcn_perm(w[4], w[3], 0x05040302u)};
        const uint32_t q1[4] = {w[5], w[6], w[7], w[8]};
        const float a0 = block_acc(q0, xs.v, magic), a1 = block_acc(q1, xs.v + 32, magic);
        // sum (q-8) x = 16*(acc - X) - 8X = 16 acc - 24 X
        const float d0 = h2f(w[0]), d1 = h2f(w[4] >> 16);
        return fmaf(d0, fmaf(16.f, a0, -24.f * xs.s0), d1 * fmaf(16.f, a1, -24.f * xs.s1));
    }
};

// ---- Q4_K fast: one lane = code pair p (32 bytes) of super-block b ---------
// byte 32p + i: low nibble = value 64p + i (sub-block 2p), high nibble = value
// 64p + 32 + i (sub-block 2p+1).
struct F4K {
    static constexpr int kRows = 2;
    struct L { uint32_t off_h, off_q, p; };
    struct X { float v[64]; float slo, shi; };   // v[i]: value 64p+i (lo: i<32, hi: i>=32)
    struct Raw { u32x4 h, q0, q1; };
    __device__ static L lane(int64_t u) {
        const uint32_t b = uint32_t(u >> 2), p = uint32_t(u & 3);
        return {144 * b, 144 * b + 16 + 32 * p, p};
    }
    __device__ static void load_x(const float *x, int64_t u, X &xs) {
        const int64_t b = u >> 2, p = u & 3;
        load_x64(x + b * 256 + 64 * p, xs.v, xs.slo);
        float sh = 0.f;
#pragma unroll
        for (int i = 0; i < 32; ++i) sh += xs.v[32 + i];
        xs.shi = sh;
        xs.slo -= sh;
    }
    __device__ static void load(const uint8_t *row, const L &l, Raw &r) {
        r.h = ld4(row + l.off_h);
        r.q0 = ld4(row + l.off_q);
        r.q1 = ld4(row + l.off_q + 16);
    }
    __device__ static float dot(const Raw &r, const X &xs, const L &l, uint32_t magic) {
        const uint32_t q[8] = {r.q0.x, r.q0.y, r.q0.z, r.q0.w, r.q1.x, r.q1.y, r.q1.z, r.q1.w};
        float al = 0.f, ah = 0.f;
#pragma unroll
        for (int m = 0; m < 8; ++m) nib_fma(q[m], xs.v + 4 * m, xs.v + 32 + 4 * m, magic, al, ah);
        const uint32_t p = l.p, sft = 16 * (p & 1);
        const uint32_t y = r.h.y >> sft, z = r.h.z >> sft, w = r.h.w >> sft;
        // both encodings computed, one selected: no divergent branch
        const bool low = p < 2;
        const uint32_t S0 = low ? (y & 63) : ((w & 15) | (((y >> 6) & 3) << 4));
        const uint32_t M0 = low ? (z & 63) : (((w >> 4) & 15) | (((z >> 6) & 3) << 4));
        const uint32_t S1 = low ? ((y >> 8) & 63) : (((w >> 8) & 15) | (((y >> 14) & 3) << 4));
        const uint32_t M1 = low ? ((z >> 8) & 63) : (((w >> 12) & 15) | (((z >> 14) & 3) << 4));
        const float d = h2f(r.h.x), dmin = h2f(r.h.x >> 16);
        // sum q x over a sub-block = 16 * (acc - X)
        const float pos = fmaf(float(S0), al - xs.slo, float(S1) * (ah - xs.shi));
        const float neg = fmaf(float(M0), xs.slo, float(M1) * xs.shi);
        return fmaf(16.f * d, pos, -dmin * neg);
    }
};

// ---- Q6_K fast: one lane = 64 values of a 210-byte super-block -------------
// Lane t (0..3) of super-block b: half h = t/2, slot j = t%2; values
// 128h + 32k + 16j + i (k = 0..3, i = 0..15) from ql[64h + 16j + i] (k = 0
// low, k = 2 high nibble), ql[64h + 32 + 16j + i] (k = 1 low, k = 3 high),
// qh[32h + 16j + i] (bits 2k..2k+1), scales[8h + 2k + j] and d.  Odd blocks
// start 2 bytes into a word: loads are word-aligned and v_perm realigns.
struct F6K {
    static constexpr int kRows = 1;
    struct L { uint32_t base, sel, h, j; };
    struct X { float v[4][16]; float s[4]; };
    struct Raw { u32x4 a; uint32_t a4; u32x4 b; uint32_t b4; u32x4 c; uint32_t c4; u32x3 sc; uint32_t d; };
    __device__ static L lane(int64_t u) {
        const uint32_t b = uint32_t(u >> 2), t = uint32_t(u & 3);
        const uint32_t off = 210 * b, sh = off & 3;
        return {off - sh, sh ? 0x05040302u : 0x03020100u, t >> 1, t & 1};
    }
    __device__ static void load_x(const float *x, int64_t u, X &xs) {
        const int64_t b = u >> 2, t = u & 3, h = t >> 1, j = t & 1;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const float4 *p = reinterpret_cast<const float4 *>(x + b * 256 + 128 * h + 32 * k + 16 * j);
            float s = 0.f;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float4 a = p[i];
                xs.v[k][4 * i] = a.x; xs.v[k][4 * i + 1] = a.y; xs.v[k][4 * i + 2] = a.z; xs.v[k][4 * i + 3] = a.w;
                s += (a.x + a.y) + (a.z + a.w);
            }
            xs.s[k] = s;
        }
    }
    __device__ static void load(const uint8_t *row, const L &l, Raw &r) {
        const uint8_t *p = row + l.base;
        const uint32_t oa = 64 * l.h + 16 * l.j, oc = 128 + 32 * l.h + 16 * l.j;
        r.a = ld4(p + oa); r.a4 = ld1(p + oa + 16);
        r.b = ld4(p + oa + 32); r.b4 = ld1(p + oa + 48);
        r.c = ld4(p + oc); r.c4 = ld1(p + oc + 16);
        r.sc = ld3(p + 192 + 8 * l.h);
        r.d = ld1(p + 208);
    }
    __device__ static float dot(const Raw &r, const X &xs, const L &l, uint32_t) {
        const uint32_t sel = l.sel;
        const uint32_t A[5] = {r.a.x, r.a.y, r.a.z, r.a.w, r.a4};
        const uint32_t B[5] = {r.b.x, r.b.y, r.b.z, r.b.w, r.b4};
        const uint32_t C[5] = {r.c.x, r.c.y, r.c.z, r.c.w, r.c4};
        float s[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const uint32_t a = __builtin_amdgcn_perm(A[m + 1], A[m], sel);
            const uint32_t b = __builtin_amdgcn_perm(B[m + 1], B[m], sel);
            const uint32_t c = __builtin_amdgcn_perm(C[m + 1], C[m], sel);
            // 6-bit codes, one per byte; opaque() keeps byte conversions whole
            const uint32_t q0 = opaque((a & kLo4) | ((c << 4) & 0x30303030u));
            const uint32_t q1 = opaque((b & kLo4) | ((c << 2) & 0x30303030u));
            const uint32_t q2 = opaque(((a >> 4) & kLo4) | (c & 0x30303030u));
            const uint32_t q3 = opaque(((b >> 4) & kLo4) | ((c >> 2) & 0x30303030u));
            const uint32_t qq[4] = {q0, q1, q2, q3};
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                s[k] = fmaf(ubyte<0>(qq[k]), xs.v[k][4 * m + 0], s[k]);
                s[k] = fmaf(ubyte<1>(qq[k]), xs.v[k][4 * m + 1], s[k]);
                s[k] = fmaf(ubyte<2>(qq[k]), xs.v[k][4 * m + 2], s[k]);
                s[k] = fmaf(ubyte<3>(qq[k]), xs.v[k][4 * m + 3], s[k]);
            }
        }
        // int8 scales[8h + 2k + j] = byte 2k + j of the realigned scale words
        const uint32_t sc0 = __builtin_amdgcn_perm(r.sc.y, r.sc.x, sel) >> (8 * l.j);
        const uint32_t sc1 = __builtin_amdgcn_perm(r.sc.z, r.sc.y, sel) >> (8 * l.j);
        const float c0 = float(int8_t(sc0)), c1 = float(int8_t(sc0 >> 16));
        const float c2 = float(int8_t(sc1)), c3 = float(int8_t(sc1 >> 16));
        float acc = c0 * fmaf(-32.f, xs.s[0], s[0]);
        acc = fmaf(c1, fmaf(-32.f, xs.s[1], s[1]), acc);
        acc = fmaf(c2, fmaf(-32.f, xs.s[2], s[2]), acc);
        acc = fmaf(c3, fmaf(-32.f, xs.s[3], s[3]), acc);
        const uint32_t dbits = (l.sel == 0x03020100u) ? r.d : (r.d >> 16);
        return h2f(dbits) * acc;
    }
};

// Persistent, software-pipelined fast kernel.  A workgroup of nw waves (one
// per 4096-value column slice) walks row tiles blockIdx.x, +gridDim.x, ...
// A tile is G row groups of R rows.  The tile body is fully unrolled with two
// register buffers: while a wave decodes group g it already has the loads of
// group g+1 in flight (the last group prefetches the first group of the next
// tile), so every load is unconditional and the compiler can wait for exactly
// the group it decodes.  Row sums are reduced over the wave with DPP, kept in
// one VGPR (lane i = row i of the tile), written to LDS once per tile, and the
// nw column slices are added in a fixed order.
template <class Tr, int G>
__global__ void __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(3)))
gemv_fast(const uint8_t *__restrict__ W, const float *__restrict__ x, float *__restrict__ y,
          int rows, int64_t row_bytes, int units_per_row, int accumulate) {
    constexpr int R = Tr::kRows, T = R * G;
    static_assert(G % 2 == 0 && T <= 64, "tile shape");
    __shared__ float part[2][8 * T];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
    const int64_t unit = int64_t(wave) * 64 + lane;
    const bool ok = unit < units_per_row;
    const uint32_t magic = opaque(kMagic16);
    const typename Tr::L L = Tr::lane(ok ? unit : 0);
    const int ntiles = (rows + T - 1) / T;
    int t = blockIdx.x;
    if (t >= ntiles) return;

    // rows past the end re-read the last row; idle lanes read unit 0
    auto issue = [&](typename Tr::Raw *buf, int tile, int g) {
#pragma unroll
        for (int i = 0; i < R; ++i)
            Tr::load(W + int64_t(min(tile * T + g * R + i, rows - 1)) * row_bytes, L, buf[i]);
    };

    typename Tr::Raw A[R], B[R];
    issue(A, t, 0);
    asm volatile("" ::: "memory");      // the first weight loads go out before the activations
    typename Tr::X xs;
    Tr::load_x(x, ok ? unit : 0, xs);

    int pb = 0;
    for (; t < ntiles; t += gridDim.x) {
        const int tn = t + int(gridDim.x) < ntiles ? t + int(gridDim.x) : t;
        float rowsum = 0.f;             // lane i: sum of row i of this tile (this slice)
#pragma unroll
        for (int g = 0; g < G; ++g) {
            typename Tr::Raw *cur = (g & 1) ? B : A;
            typename Tr::Raw *nxt = (g & 1) ? A : B;
            if (g + 1 < G) issue(nxt, t, g + 1);
            else issue(nxt, tn, 0);
#pragma unroll
            for (int i = 0; i < R; ++i) {
                float a = Tr::dot(cur[i], xs, L, magic);
                a = ok ? a : 0.f;
                a = wave_sum_to_lane63(a);
                const float s = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(a), 63));
                rowsum = (lane == g * R + i) ? s : rowsum;
            }
        }
        if (lane < T) part[pb][wave * T + lane] = rowsum;
        __syncthreads();
        if (wave == 0 && lane < T) {
            const int r = t * T + lane;
            if (r < rows) {
                float sum = 0.f;
                for (int w = 0; w < nw; ++w) sum += part[pb][w * T + lane];
                y[r] = accumulate ? y[r] + sum : sum;
            }
        }
        pb ^= 1;
    }
}

int env_int(const char *name, int dflt) {
    const char *v = std::getenv(name);
    return v ? std::atoi(v) : dflt;
}

template <class Tr>
hipError_t launch_generic(const void *W, const float *x, float *y, int64_t rows, int64_t cols, int acc,
                          hipStream_t st) {
    constexpr int R = 4;
    const int units = int(cols / 32);
    const int64_t bpr = cols / Tr::kBlockElems;
    const int upl = units <= 1024 ? 1 : 2;
    const int nw = (units + 64 * upl - 1) / (64 * upl);
    int64_t t = rows * nw / 8192;
    int tile = t < R ? R : t > 32 ? 32 : int(t / R * R);
    const int64_t grid = (rows + tile - 1) / tile;
    const size_t lds = size_t(nw) * tile * sizeof(float);
    const uint8_t *w = static_cast<const uint8_t *>(W);
    if (upl == 1)
        gemv_generic<Tr, R, 1><<<dim3(unsigned(grid)), dim3(64 * nw), lds, st>>>(
            w, x, y, int(rows), units, bpr, tile, acc);
    else
        gemv_generic<Tr, R, 2><<<dim3(unsigned(grid)), dim3(64 * nw), lds, st>>>(
            w, x, y, int(rows), units, bpr, tile, acc);
    return hipGetLastError();
}

struct FastShape {
    int nw, G;
    int64_t grid;
};

FastShape fast_shape(int R, int64_t rows, int64_t cols) {
    static const int waves_env = env_int("NT_GEMV_WAVES", 0);
    static const int g_env = env_int("NT_GEMV_G", 0);
    FastShape f;
    const int units = int(cols / 64);
    f.nw = (units + 63) / 64;                      // <= 8 for cols <= 32768
    // groups per tile: 8 for tall matrices, 4 (or 2) when that leaves too few tiles
    f.G = g_env;
    if (f.G <= 0) {
        f.G = 8;
        while (f.G > 2 && (rows + R * f.G - 1) / (R * f.G) * f.nw < 2048) f.G /= 2;
    }
    const int T = R * f.G;
    const int64_t ntiles = (rows + T - 1) / T;
    // persistent grid: about 12 resident waves per CU on 256 CUs
    const int64_t waves = waves_env > 0 ? waves_env : 256 * 12;
    f.grid = waves / f.nw;
    if (f.grid > ntiles) f.grid = ntiles;
    if (f.grid < 1) f.grid = 1;
    return f;
}

template <class Tr>
hipError_t launch_fast(const void *W, const float *x, float *y, int64_t rows, int64_t cols, int64_t row_bytes,
                       int acc, hipStream_t st) {
    const int units = int(cols / 64);
    const FastShape fs = fast_shape(Tr::kRows, rows, cols);
    const int nw = fs.nw, G = fs.G;
    const int64_t grid = fs.grid;
    const uint8_t *w = static_cast<const uint8_t *>(W);
    const dim3 gd = dim3(unsigned(grid)), bd = dim3(unsigned(64 * nw));
    switch (G) {
    case 2: gemv_fast<Tr, 2><<<gd, bd, 0, st>>>(w, x, y, int(rows), row_bytes, units, acc); break;
    case 4: gemv_fast<Tr, 4><<<gd, bd, 0, st>>>(w, x, y, int(rows), row_bytes, units, acc); break;
    default: gemv_fast<Tr, 8><<<gd, bd, 0, st>>>(w, x, y, int(rows), row_bytes, units, acc); break;
    }
    return hipGetLastError();
}

}  // namespace

static bool use_fast(nt_qtype t, int64_t cols) {
    // fast path: word-aligned rows (an even number of 2-byte-aligned blocks)
    // and at most 8 slices of 4096 values
    static const bool force_generic = env_int("NT_GEMV_GENERIC", 0) != 0;
    const int64_t rb = cols / block_elems(t) * block_bytes(t);
    return !force_generic && rb % 4 == 0 && cols % 64 == 0 && cols <= 32768;
}

void gemv_launch_info(nt_qtype t, int64_t rows, int64_t cols, int32_t info[4]) {
    if (use_fast(t, cols)) {
        const int R = t == NT_Q6_K ? F6K::kRows : t == NT_Q8_0 ? F80::kRows : t == NT_Q4_0 ? F40::kRows : F4K::kRows;
        const FastShape f = fast_shape(R, rows, cols);
        info[0] = 1;
        info[1] = R * f.G;
        info[2] = int32_t(f.grid);
        info[3] = 64 * f.nw;
    } else {
        const int units = int(cols / 32), upl = units <= 1024 ? 1 : 2;
        const int nw = (units + 64 * upl - 1) / (64 * upl);
        const int64_t tt = rows * nw / 8192;
        const int tile = tt < 4 ? 4 : tt > 32 ? 32 : int(tt / 4 * 4);
        info[0] = 0;
        info[1] = tile;
        info[2] = int32_t((rows + tile - 1) / tile);
        info[3] = 64 * nw;
    }
}

hipError_t launch_gemv(nt_qtype t, const void *W, const float *x, float *y, int64_t rows,
                       int64_t cols, int accumulate, hipStream_t st) {
    const int64_t rb = cols / block_elems(t) * block_bytes(t);
    const bool fast = use_fast(t, cols);
    switch (t) {
    case NT_Q8_0: return fast ? launch_fast<F80>(W, x, y, rows, cols, rb, accumulate, st)
                              : launch_generic<Q80>(W, x, y, rows, cols, accumulate, st);
    case NT_Q4_0: return fast ? launch_fast<F40>(W, x, y, rows, cols, rb, accumulate, st)
                              : launch_generic<Q40>(W, x, y, rows, cols, accumulate, st);
    case NT_Q4_K: return fast ? launch_fast<F4K>(W, x, y, rows, cols, rb, accumulate, st)
                              : launch_generic<Q4K>(W, x, y, rows, cols, accumulate, st);
    case NT_Q6_K: return fast ? launch_fast<F6K>(W, x, y, rows, cols, rb, accumulate, st)
                              : launch_generic<Q6K>(W, x, y, rows, cols, accumulate, st);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace nt
