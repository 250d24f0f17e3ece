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
#include <algorithm>
#include <atomic>
#include <mutex>
#include <type_traits>

#include "device_util.h"
#include "nt_internal.h"

namespace nt {

// Arguments of one fast-path launch: up to three matrices of one format and
// width read against the same activation vector (their rows concatenated), or
// in SwiGLU mode a gate and an up matrix whose rows are interleaved.
struct GemvArgs {
    const uint8_t *W[3];
    float *y[3];
    int32_t seg_end[3];      // cumulative row counts
    uint32_t seg_lim[3];     // last byte offset a copy may start at, per matrix
    const float *x;
    const float *gain;       // RMSNorm gain; null: x is used as is
    float eps;
    int cols;
    int rows;                // rows of all matrices together
    int units;               // 64-value units per row
    uint32_t row_bytes;
    int accumulate;
    int swiglu;
    // per launch, set where the grid is chosen (integer division is a long
    // instruction chain on the device): workgroup b of G takes items_q items,
    // plus one if b < items_r; SHARED layout: `groups` row groups of nw waves,
    // inv_nw = ceil(2^16 / nw), inv_groups = ceil(2^16 / groups), so that
    // (n * inv) >> 16 = n / d for the small counts n the kernel divides
    int items_q;
    int items_r;
    int groups;
    uint32_t inv_nw;
    uint32_t inv_groups;
};

GemvArgs gemv_args(nt_qtype t, int nseg, const void *const *W, const int64_t *rows, float *const *y, int64_t cols,
                   const float *x, const float *gain, float eps, int accumulate);

namespace {

constexpr uint32_t kLo4 = 0x0f0f0f0fu;

// ---- Q8_0: one unit = one 34-byte block ------------------------------------
struct Q80 {
    static constexpr int kBlockElems = 32;
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
    static constexpr int kBlockElems = 32;
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
    static constexpr int kBlockElems = 256;
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

// ---- Q5_K: one unit = one 16-byte code chunk of a 176-byte super-block ------
// The Q4_K chunk (bytes 48 + 16t .. of qs: pair p = t/2, half hh = t%2, low
// nibbles sub-block 2p, high nibbles 2p+1, element l = 16hh + i of each) plus
// the 16 bytes qh[16hh ..] whose bits 2p and 2p+1 are the two sub-blocks'
// fifth bits.  Codes q in [0, 31] are assembled one per byte and converted
// with byte-to-float conversions; scale and min as in Q4_K.
struct Q5K {
    static constexpr int kBlockElems = 256;
    struct Raw { u32x4 hdr, qh, q; };
    using X = Q4K::X;

    __device__ static void load_x(const float *x, int64_t unit, X &xs) { Q4K::load_x(x, unit, xs); }
    __device__ static void load(const uint8_t *W, int64_t g, uint32_t t, Raw &r) {
        const uint8_t *p = W + g * 176;
        r.hdr = ld4(p);
        r.qh = ld4(p + 16 + 16 * (t & 1));
        r.q = ld4(p + 48 + 16 * t);
    }
    __device__ static float dot(const Raw &r, const X &xs) {
        const uint32_t qw[4] = {r.q.x, r.q.y, r.q.z, r.q.w};
        const uint32_t hw[4] = {r.qh.x, r.qh.y, r.qh.z, r.qh.w};
        const uint32_t p = xs.t >> 1;
        float s0 = 0.f, s1 = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t lo = opaque((qw[i] & kLo4) | (((hw[i] >> (2 * p)) & 0x01010101u) << 4));
            const uint32_t hi = opaque(((qw[i] >> 4) & kLo4) | (((hw[i] >> (2 * p + 1)) & 0x01010101u) << 4));
            s0 = fmaf(ubyte<0>(lo), xs.lo[4 * i + 0], s0);
            s0 = fmaf(ubyte<1>(lo), xs.lo[4 * i + 1], s0);
            s0 = fmaf(ubyte<2>(lo), xs.lo[4 * i + 2], s0);
            s0 = fmaf(ubyte<3>(lo), xs.lo[4 * i + 3], s0);
            s1 = fmaf(ubyte<0>(hi), xs.hi[4 * i + 0], s1);
            s1 = fmaf(ubyte<1>(hi), xs.hi[4 * i + 1], s1);
            s1 = fmaf(ubyte<2>(hi), xs.hi[4 * i + 2], s1);
            s1 = fmaf(ubyte<3>(hi), xs.hi[4 * i + 3], s1);
        }
        const uint32_t sft = 16 * (p & 1);
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
    static constexpr int kBlockElems = 256;
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
// Fast path: rows whose byte length is a multiple of 4 (an even number of
// Q8_0 / Q4_0 blocks, any Q4_K row, Q6_K rows of an even number of
// super-blocks), cols % 64 == 0, cols <= 32768.
//
// Lane l of wave w owns 64 consecutive values of every row ("unit" 64w + l):
// two Q8_0 / Q4_0 blocks, one 32-byte code pair of a Q4_K super-block, or a
// quarter of a Q6_K super-block.  The 64 lanes of a wave therefore own one
// contiguous byte range of each row, its "slice" (kSlice bytes).  The slice
// is copied from HBM into a per-wave LDS ring by global_load_lds (each
// instruction moves 64 x VEC contiguous bytes, fully coalesced, straight into
// LDS without passing through VGPRs); a lane then reads its own unit back
// from LDS.  The ring keeps one row (two for Q4_K rows) in flight per wave, so 8
// waves per CU keep 20-35 KB of weight reads outstanding per CU, about what
// HBM latency times bandwidth needs.  Waits are explicit (s_waitcnt vmcnt)
// because the ring's loads return to LDS, not to registers the compiler could
// track.
// =============================================================================

constexpr int kMaxRowsPerWG = 256;           // rows one workgroup reduces (LDS row sums)


// Nibble products without a bias term: a 4-bit code in bits 0..3 of an fp16
// half is the subnormal q * 2^-24, in bits 4..7 the subnormal q * 2^-20, both
// exact, and v_fma_mix_f32 widens them to fp32 exactly (fp16 denormals are
// kept).  al collects 2^-24 * sum q x over the low nibbles of w, ah 2^-20 *
// sum q x over the high nibbles (byte k of w <-> xl[k], xh[k]).  One shift
// and four masks per 8 codes.
__device__ __forceinline__ void nib_fma(uint32_t w, const float *xl, const float *xh, float &al, float &ah) {
    const uint32_t t = w >> 8;
    const uint32_t c0 = w & 0x000f000fu;   // low nibbles of bytes 0, 2
    const uint32_t c1 = t & 0x000f000fu;   // low nibbles of bytes 1, 3
    const uint32_t c2 = w & 0x00f000f0u;   // high nibbles of bytes 0, 2
    const uint32_t c3 = t & 0x00f000f0u;   // high nibbles of bytes 1, 3
    al = fmaf(h_lo(c0), xl[0], al);
    al = fmaf(h_lo(c1), xl[1], al);
    al = fmaf(h_hi(c0), xl[2], al);
    al = fmaf(h_hi(c1), xl[3], al);
    ah = fmaf(h_lo(c2), xh[0], ah);
    ah = fmaf(h_lo(c3), xh[1], ah);
    ah = fmaf(h_hi(c2), xh[2], ah);
    ah = fmaf(h_hi(c3), xh[3], ah);
}

// 2^20 * (16 al + ah): the two nibble sums of nib_fma on one scale
constexpr float kNib20 = 1048576.0f;

// Sum of N values: pairwise within groups of four, groups added in order.
template <int N>
__device__ __forceinline__ float sum_vals(const float *v) {
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < N / 4; ++i) s += (v[4 * i] + v[4 * i + 1]) + (v[4 * i + 2] + v[4 * i + 3]);
    return s;
}

// ---- Q8_0 fast: one lane = blocks 2u, 2u+1 (68 bytes at 68u, word-aligned) --
struct F80 {
    static constexpr int kSlice = 64 * 68, kStagesShared = 2, kStagesWide = 2;
    struct L { uint32_t off; };
    struct X { float v[64]; float s0, s1; };
    struct Raw { u32x4 a, b, c, d; uint32_t e; };
    __device__ static L lane(int l) { return {uint32_t(l * 68)}; }
    __device__ static uint32_t x_chunk(int l, int j) { return uint32_t(16 * l + j); }
    __device__ static void sums(X &xs) { xs.s0 = sum_vals<32>(xs.v); xs.s1 = sum_vals<32>(xs.v + 32); }
    __device__ static void load(const uint8_t *base, const L &l, Raw &r) {
        const uint8_t *p = base + l.off;
        r.a = ld4(p); r.b = ld4(p + 16); r.c = ld4(p + 32); r.d = ld4(p + 48); r.e = ld1(p + 64);
    }
    __device__ static float dot(const Raw &r, const X &xs, const L &) {
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
    static constexpr int kSlice = 64 * 36, kStagesShared = 2, kStagesWide = 3;
    struct L { uint32_t off; };
    struct X { float v[64]; float s0, s1; };
    struct Raw { u32x4 a, b; uint32_t c; };
    __device__ static L lane(int l) { return {uint32_t(l * 36)}; }
    __device__ static uint32_t x_chunk(int l, int j) { return uint32_t(16 * l + j); }
    __device__ static void sums(X &xs) { xs.s0 = sum_vals<32>(xs.v); xs.s1 = sum_vals<32>(xs.v + 32); }
    __device__ static void load(const uint8_t *base, const L &l, Raw &r) {
        const uint8_t *p = base + l.off;
        r.a = ld4(p); r.b = ld4(p + 16); r.c = ld1(p + 32);
    }
    // sum over one block of q x: byte i holds value i (low) and i+16 (high)
    __device__ static float block_acc(const uint32_t *q, const float *v) {
        float al = 0.f, ah = 0.f;
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const float xl[4] = {v[4 * m + 0], v[4 * m + 1], v[4 * m + 2], v[4 * m + 3]};
            const float xh[4] = {v[16 + 4 * m + 0], v[16 + 4 * m + 1], v[16 + 4 * m + 2], v[16 + 4 * m + 3]};
            nib_fma(q[m], xl, xh, al, ah);
        }
        return kNib20 * fmaf(16.f, al, ah);
    }
    __device__ static float dot(const Raw &r, const X &xs, const L &) {
        const uint32_t w[9] = {r.a.x, r.a.y, r.a.z, r.a.w, r.b.x, r.b.y, r.b.z, r.b.w, r.c};
        const uint32_t q0[4] = {__builtin_amdgcn_perm(w[1], w[0], 0x05040302u),
                                __builtin_amdgcn_perm(w[2], w[1], 0x05040302u),
                                __builtin_amdgcn_perm(w[3], w[2], 0x05040302u),
                                __builtin_amdgcn_perm(w[4], w[3], 0x05040302u)};
        const uint32_t q1[4] = {w[5], w[6], w[7], w[8]};
        const float a0 = block_acc(q0, xs.v), a1 = block_acc(q1, xs.v + 32);
        // sum (q-8) x = sum q x - 8 X
        const float d0 = h2f(w[0]), d1 = h2f(w[4] >> 16);
        return fmaf(d0, fmaf(-8.f, xs.s0, a0), d1 * fmaf(-8.f, xs.s1, a1));
    }
};

// ---- Q4_K fast: one lane = code pair p (32 bytes) of super-block b ---------
// byte 32p + i: low nibble = value 64p + i (sub-block 2p), high nibble = value
// 64p + 32 + i (sub-block 2p+1).
struct F4K {
    static constexpr int kSlice = 16 * 144, kStagesShared = 3, kStagesWide = 3;
    struct L { uint32_t off_h, off_q, p; };
    struct X { float v[64]; float slo, shi; };   // v[i]: value 64p+i (lo: i<32, hi: i>=32)
    struct Raw { u32x4 h, q0, q1; };
    __device__ static L lane(int l) {
        const uint32_t b = uint32_t(l >> 2), p = uint32_t(l & 3);
        return {144 * b, 144 * b + 16 + 32 * p, p};
    }
    // value i of lane l's 64 is x[64 l + i] within the wave's 4096
    __device__ static uint32_t x_chunk(int l, int j) { return uint32_t(16 * l + j); }
    __device__ static void sums(X &xs) { xs.slo = sum_vals<32>(xs.v); xs.shi = sum_vals<32>(xs.v + 32); }
    __device__ static void load(const uint8_t *base, const L &l, Raw &r) {
        r.h = ld4(base + l.off_h);
        r.q0 = ld4(base + l.off_q);
        r.q1 = ld4(base + l.off_q + 16);
    }
    __device__ static float dot(const Raw &r, const X &xs, const L &l) {
        const uint32_t q[8] = {r.q0.x, r.q0.y, r.q0.z, r.q0.w, r.q1.x, r.q1.y, r.q1.z, r.q1.w};
        float al = 0.f, ah = 0.f;
#pragma unroll
        for (int m = 0; m < 8; ++m) nib_fma(q[m], xs.v + 4 * m, xs.v + 32 + 4 * m, al, ah);
        const uint32_t p = l.p, sft = 16 * (p & 1);
        const uint32_t y = r.h.y >> sft, z = r.h.z >> sft, w = r.h.w >> sft;
        // both encodings computed, one kept by a lane mask: no branch
        const uint32_t lm = opaque(p < 2 ? 0xffffffffu : 0u), hm = ~lm;
        const uint32_t S0 = ((y & 63) & lm) | (((w & 15) | (((y >> 6) & 3) << 4)) & hm);
        const uint32_t M0 = ((z & 63) & lm) | ((((w >> 4) & 15) | (((z >> 6) & 3) << 4)) & hm);
        const uint32_t S1 = (((y >> 8) & 63) & lm) | ((((w >> 8) & 15) | (((y >> 14) & 3) << 4)) & hm);
        const uint32_t M1 = (((z >> 8) & 63) & lm) | ((((w >> 12) & 15) | (((z >> 14) & 3) << 4)) & hm);
        const float d = h2f(r.h.x), dmin = h2f(r.h.x >> 16);
        // sum q x over sub-block 2p = 2^24 al, over 2p+1 = 2^20 ah
        const float pos = fmaf(float(16 * S0), al, float(S1) * ah);
        const float neg = fmaf(float(M0), xs.slo, float(M1) * xs.shi);
        return fmaf(kNib20 * d, pos, -dmin * neg);
    }
};

// ---- Q5_K fast: one lane = code pair p (32 bytes) of super-block b ---------
// As F4K (byte 32p + i of qs: low nibble = value 64p + i, high nibble = value
// 64p + 32 + i), plus all 32 bytes of qh, whose bits 2p and 2p+1 are the
// fifth bits of those values.  Codes are assembled one per byte (nibble |
// bit << 4) and converted with byte-to-float conversions.
struct F5K {
    static constexpr int kSlice = 16 * 176, kStagesShared = 2, kStagesWide = 3;
    struct L { uint32_t off_h, off_q, p; };
    using X = F4K::X;
    struct Raw { u32x4 h, qh0, qh1, q0, q1; };
    __device__ static L lane(int l) {
        const uint32_t b = uint32_t(l >> 2), p = uint32_t(l & 3);
        return {176 * b, 176 * b + 48 + 32 * p, p};
    }
    __device__ static uint32_t x_chunk(int l, int j) { return F4K::x_chunk(l, j); }
    __device__ static void sums(X &xs) { F4K::sums(xs); }
    __device__ static void load(const uint8_t *base, const L &l, Raw &r) {
        r.h = ld4(base + l.off_h);
        r.qh0 = ld4(base + l.off_h + 16);
        r.qh1 = ld4(base + l.off_h + 32);
        r.q0 = ld4(base + l.off_q);
        r.q1 = ld4(base + l.off_q + 16);
    }
    __device__ static float dot(const Raw &r, const X &xs, const L &l) {
        const uint32_t q[8] = {r.q0.x, r.q0.y, r.q0.z, r.q0.w, r.q1.x, r.q1.y, r.q1.z, r.q1.w};
        const uint32_t hb[8] = {r.qh0.x, r.qh0.y, r.qh0.z, r.qh0.w, r.qh1.x, r.qh1.y, r.qh1.z, r.qh1.w};
        const uint32_t p = l.p, sl = 2 * p, sh = 2 * p + 1;
        float al = 0.f, ah = 0.f;
#pragma unroll
        for (int m = 0; m < 8; ++m) {
            const uint32_t lo = opaque((q[m] & kLo4) | (((hb[m] >> sl) & 0x01010101u) << 4));
            const uint32_t hi = opaque(((q[m] >> 4) & kLo4) | (((hb[m] >> sh) & 0x01010101u) << 4));
            al = fmaf(ubyte<0>(lo), xs.v[4 * m + 0], al);
            al = fmaf(ubyte<1>(lo), xs.v[4 * m + 1], al);
            al = fmaf(ubyte<2>(lo), xs.v[4 * m + 2], al);
            al = fmaf(ubyte<3>(lo), xs.v[4 * m + 3], al);
            ah = fmaf(ubyte<0>(hi), xs.v[32 + 4 * m + 0], ah);
            ah = fmaf(ubyte<1>(hi), xs.v[32 + 4 * m + 1], ah);
            ah = fmaf(ubyte<2>(hi), xs.v[32 + 4 * m + 2], ah);
            ah = fmaf(ubyte<3>(hi), xs.v[32 + 4 * m + 3], ah);
        }
        const uint32_t sft = 16 * (p & 1);
        const uint32_t y = r.h.y >> sft, z = r.h.z >> sft, w = r.h.w >> sft;
        // both encodings computed, one kept by a lane mask: no branch
        const uint32_t lm = opaque(p < 2 ? 0xffffffffu : 0u), hm = ~lm;
        const uint32_t S0 = ((y & 63) & lm) | (((w & 15) | (((y >> 6) & 3) << 4)) & hm);
        const uint32_t M0 = ((z & 63) & lm) | ((((w >> 4) & 15) | (((z >> 6) & 3) << 4)) & hm);
        const uint32_t S1 = (((y >> 8) & 63) & lm) | ((((w >> 8) & 15) | (((y >> 14) & 3) << 4)) & hm);
        const uint32_t M1 = (((z >> 8) & 63) & lm) | ((((w >> 12) & 15) | (((z >> 14) & 3) << 4)) & hm);
        const float d = h2f(r.h.x), dmin = h2f(r.h.x >> 16);
        const float pos = fmaf(float(S0), al, float(S1) * ah);
        const float neg = fmaf(float(M0), xs.slo, float(M1) * xs.shi);
        return fmaf(d, pos, -dmin * neg);
    }
};

// ---- Q6_K fast: one lane = 64 values of a 210-byte super-block -------------
// Lane t (0..3) of super-block b: half h = t/2, slot j = t%2; values
// 128h + 32k + 16j + i (k = 0..3, i = 0..15) from ql[64h + 16j + i] (k = 0
// low, k = 2 high nibble), ql[64h + 32 + 16j + i] (k = 1 low, k = 3 high),
// qh[32h + 16j + i] (bits 2k..2k+1), scales[8h + 2k + j] and d.  Odd blocks
// start 2 bytes into a word: loads are word-aligned and v_perm realigns.
struct F6K {
    static constexpr int kSlice = 16 * 210, kStagesShared = 2, kStagesWide = 2;
    struct L { uint32_t base, sel, h, j; };
    struct X { float v[64]; float s[4]; };       // v[16k + i]
    struct Raw { u32x4 a; uint32_t a4; u32x4 b; uint32_t b4; u32x4 c; uint32_t c4; u32x3 sc; uint32_t d; };
    __device__ static L lane(int l) {
        const uint32_t b = uint32_t(l >> 2), t = uint32_t(l & 3);
        const uint32_t off = 210 * b, sh = off & 3;
        return {off - sh, sh ? 0x05040302u : 0x03020100u, t >> 1, t & 1};
    }
    // values v[16k + 4m .. +3] = x[256b + 128h + 32k + 16j + 4m ..] (16-byte chunk 4k + m)
    __device__ static uint32_t x_chunk(int l, int c) {
        const int b = l >> 2, t = l & 3, h = t >> 1, j = t & 1, k = c >> 2, m = c & 3;
        return uint32_t(64 * b + 32 * h + 8 * k + 4 * j + m);
    }
    __device__ static void sums(X &xs) {
#pragma unroll
        for (int k = 0; k < 4; ++k) xs.s[k] = sum_vals<16>(xs.v + 16 * k);
    }
    __device__ static void load(const uint8_t *base, const L &l, Raw &r) {
        const uint8_t *p = base + l.base;
        const uint32_t oa = 64 * l.h + 16 * l.j, oc = 128 + 32 * l.h + 16 * l.j;
        r.a = ld4(p + oa); r.a4 = ld1(p + oa + 16);
        r.b = ld4(p + oa + 32); r.b4 = ld1(p + oa + 48);
        r.c = ld4(p + oc); r.c4 = ld1(p + oc + 16);
        r.sc = ld3(p + 192 + 8 * l.h);
        r.d = ld1(p + 208);
    }
    __device__ static float dot(const Raw &r, const X &xs, const L &l) {
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
                s[k] = fmaf(ubyte<0>(qq[k]), xs.v[16 * k + 4 * m + 0], s[k]);
                s[k] = fmaf(ubyte<1>(qq[k]), xs.v[16 * k + 4 * m + 1], s[k]);
                s[k] = fmaf(ubyte<2>(qq[k]), xs.v[16 * k + 4 * m + 2], s[k]);
                s[k] = fmaf(ubyte<3>(qq[k]), xs.v[16 * k + 4 * m + 3], s[k]);
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

// How one row slice is copied: NFULL instructions of 64 x VEC bytes, then, if
// the slice is not a whole number of those, one instruction on the first
// REM / VEC lanes.  VEC = 16 needs 16-byte-aligned rows, VEC = 4 word-aligned.
// Ring stages: two (one row in flight per wave) except for Q4_K's 2304-byte
// slices (and wide Q4_0 rows), which need a second row in flight to keep
// enough bytes outstanding per CU (measured per format in the decode step).
template <class Tr, int VEC, bool SHARED = true>
struct Plan {
    static constexpr int kPer = 64 * VEC;
    static constexpr int kFull = Tr::kSlice / kPer;
    static constexpr int kRem = Tr::kSlice % kPer;
    static constexpr int kInstr = kFull + (kRem ? 1 : 0);
    static constexpr int kStages = SHARED ? Tr::kStagesShared : Tr::kStagesWide;
    static_assert(kRem % VEC == 0, "slice tail");
    static_assert((kStages - 1) * kInstr <= 63, "vmcnt holds at most 63 outstanding loads");
};

// Copy one row slice (this wave's part of one row) into the LDS ring stage at
// LDS address dst.
template <class Tr, int VEC>
__device__ __forceinline__ void copy_slice(const uint8_t *W, uint32_t base, uint32_t lim, uint32_t dst, int lane) {
    using P = Plan<Tr, VEC>;
#pragma unroll
    for (int k = 0; k < P::kFull; ++k) dma<VEC, true>(W, min(base + uint32_t(k * P::kPer), lim), dst + k * P::kPer);
    if constexpr (P::kRem > 0) {
        if (lane < P::kRem / VEC) dma<VEC, true>(W, min(base + uint32_t(P::kFull * P::kPer), lim), dst + P::kFull * P::kPer);
    }
}

// A wave's 64 lanes need 64 activations each: 4096 consecutive values, 16 KB
// (the wave's column slice).  Loading them lane by lane would touch 64 cache
// lines per instruction; instead the slice is copied into a 16 KB LDS area by
// 16 coalesced 1 KB copies and each lane reads its 16 chunks of 16 bytes back.
// The copy places chunk j of lane l at LDS chunk 16 l + (j + l) mod 16, so a
// read step j spreads the 64 lanes over all banks; v[4j .. 4j+3] receives
// chunk Tr::x_chunk(l, j) of the slice.  Past the end of the vector the copy
// re-reads its last 16 bytes (those values belong to lanes with no columns).
template <class Tr>
__device__ __forceinline__ void stage_vec(const float *src, int cols, int wave, int lane, const uint8_t *lds,
                                          uint32_t lds_a, float *v) {
    const uint8_t *g = reinterpret_cast<const uint8_t *>(src);
    const uint32_t lim = uint32_t(cols) * 4u - 16u, base = uint32_t(wave) * 16384u;
#pragma unroll
    for (int k = 0; k < 16; ++k) {
        const int p = 64 * k + lane, l = p >> 4, j = ((p & 15) - l) & 15;
        dma<16>(g, min(base + 16u * Tr::x_chunk(l, j), lim), lds_a + 1024 * k);
    }
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        const float4 q = *reinterpret_cast<const float4 *>(lds + 16 * (16 * lane + ((j + lane) & 15)));
        v[4 * j] = q.x; v[4 * j + 1] = q.y; v[4 * j + 2] = q.z; v[4 * j + 3] = q.w;
    }
    // the area is reused as soon as the reads are done
    __builtin_amdgcn_s_waitcnt(kLgkm0);
    __builtin_amdgcn_sched_barrier(0);
}

// The shared-area variant of the activation copy: pieces k = first,
// first + step, ... < 16 of column slice `slice` are copied to the 16 KB area
// at LDS address area (same placement as stage_vec), so the waves that share a
// slice split the copy between them.
template <class Tr>
__device__ __forceinline__ void copy_vec_pieces(const float *src, int cols, int slice, int lane, uint32_t area,
                                                int first, int step) {
    const uint8_t *g = reinterpret_cast<const uint8_t *>(src);
    const uint32_t lim = uint32_t(cols) * 4u - 16u, base = uint32_t(slice) * 16384u;
    for (int k = first; k < 16; k += step) {
        const int p = 64 * k + lane, l = p >> 4, j = ((p & 15) - l) & 15;
        dma<16>(g, min(base + 16u * Tr::x_chunk(l, j), lim), area + 1024 * k);
    }
}

// This lane's 64 values of a slice staged by copy_vec_pieces.
__device__ __forceinline__ void read_vec(const uint8_t *area, int lane, float *v) {
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        const float4 q = *reinterpret_cast<const float4 *>(area + 16 * (16 * lane + ((j + lane) & 15)));
        v[4 * j] = q.x; v[4 * j + 1] = q.y; v[4 * j + 2] = q.z; v[4 * j + 3] = q.w;
    }
}

// One workgroup = `groups` row groups of nw waves; wave w of a group owns
// column slice w of the rows the group takes.  SHARED: the activations (and
// gains) are copied once per workgroup into their own LDS area, issued
// together with the first ring loads so the two latencies overlap; otherwise
// each wave stages its slice through its own ring before the first row.
// The body of one launch's workgroup b of G (a plain launch runs it with
// blockIdx.x and gridDim.x; a paired launch splits its grid between two).
template <class Tr, int VEC, bool NORM, bool SHARED>
__device__ __forceinline__ void gemv_body(const GemvArgs &a, const int b, const int G) {
    using P = Plan<Tr, VEC, SHARED>;
    constexpr int S = P::kStages, SL = Tr::kSlice, NI = P::kInstr;
    static_assert(S >= 2, "the ring holds the row being read and at least one in flight");
    // per-wave LDS: the ring, at least 16 KB so that one activation slice
    // can be staged through it before the first row
    constexpr int RS = SHARED ? S * SL : (S * SL > 16384 ? S * SL : 16384);
    static_assert(!SHARED || S * NI <= 63, "vmcnt range of the first wait");
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    // nw waves per row (one per 4096 columns); row groups only with the
    // shared area; wave = grp * nw + cw
    const int nwv = blockDim.x >> 6;
    // every argument (and the launch dimensions, read from the same block)
    // asked for here, so that all their loads go out in one round trip (left
    // alone, the compiler issues some after a first wait, where it needs them)
    asm volatile("" :: "s"(nwv), "s"(G), "s"(a.W[0]), "s"(a.W[1]), "s"(a.W[2]), "s"(a.y[0]), "s"(a.y[1]), "s"(a.y[2]),
                 "s"(a.seg_end[0]), "s"(a.seg_end[1]), "s"(a.seg_lim[0]), "s"(a.seg_lim[1]), "s"(a.seg_lim[2]),
                 "s"(a.x), "s"(a.gain), "s"(a.cols), "s"(a.rows), "s"(a.units), "s"(a.row_bytes), "s"(a.accumulate),
                 "s"(a.swiglu), "s"(a.items_q), "s"(a.items_r), "s"(a.groups), "s"(a.inv_nw), "s"(a.inv_groups));
    const int nw = SHARED ? (a.units + 63) >> 6 : nwv;
    int cw = wave, grp = 0, R = 1;                  // column slice, row group, groups
    uint32_t inv_r = 65536u;                        // ceil(2^16 / R)
    if constexpr (SHARED) {
        grp = int((uint32_t(wave) * a.inv_nw) >> 16);
        cw = wave - grp * nw;
        R = a.groups;
        inv_r = a.inv_groups;
    }
    // LDS: [SHARED: activations nw x 16 KB, gains nw x 16 KB] rings, row sums, norm partials
    uint8_t *const xa = smem;
    uint8_t *const ga = smem + nw * 16384;
    uint8_t *const rings = smem + (SHARED ? nw * 16384 * (NORM ? 2 : 1) : 0);
    uint8_t *ring = rings + wave * RS;
    const uint32_t ring_a = lds_addr(ring);                          // the same, as an LDS address
    float *part = reinterpret_cast<float *>(rings + nwv * RS);        // [nwv][kMaxRowsPerWG]
    float *red = part + nwv * kMaxRowsPerWG;                          // [nwv]
    float *ypre = red + nwv;                                          // [nwv][64]

    // Workgroup b takes items b, b + G, b + 2G, ... (an item is a row, or in
    // SwiGLU mode a gate row and its up row), so at any moment the workgroups
    // stream one band of neighbouring rows; row group g takes the workgroup's
    // items g, g + R, g + 2R, ...
    const bool pairs = a.swiglu != 0;
    const int nitems = a.items_q + (b < a.items_r ? 1 : 0);   // items of this workgroup: b, b + G, ...
    const int mine = SHARED ? (nitems > grp ? int((uint32_t(nitems - grp + R - 1) * inv_r) >> 16) : 0) : nitems;
    const int n = pairs ? 2 * mine : mine;           // rows of this wave, in ring order

    const int u = cw * 64 + lane;
    const bool ok = u < a.units;
    const typename Tr::L L = Tr::lane(lane);
    const uint32_t lane_off = uint32_t(cw) * SL + uint32_t(lane * VEC);
    const int end0 = a.seg_end[0], end1 = a.seg_end[1];
    const uint32_t rb = a.row_bytes;
    const uint8_t *const W0 = a.W[0], *const W1 = a.W[1], *const W2 = a.W[2];
    const uint32_t lim0 = a.seg_lim[0], lim1 = a.seg_lim[1], lim2 = a.seg_lim[2];

    // global row r -> matrix seg_, row local_ within it
#define NT_SEG(r)                                                                          \
    const int seg_ = pairs ? ((r) & 1) : ((r) < end0 ? 0 : ((r) < end1 ? 1 : 2));         \
    const int local_ = pairs ? ((r) >> 1) : (r) - (seg_ == 0 ? 0 : (seg_ == 1 ? end0 : end1))
    // ring row j of this wave -> global row
#define NT_LOCATE(j)                                                                       \
    const int t_ = grp + (pairs ? ((j) >> 1) : (j)) * R;                                   \
    const int r_ = pairs ? 2 * (b + t_ * G) + ((j) & 1) : b + t_ * G;                      \
    NT_SEG(r_)
    // copy row j's slice into ring stage st
#define NT_ISSUE(j, st)                                                                          \
    do {                                                                                         \
        NT_LOCATE(j);                                                                            \
        const uint8_t *W_ = seg_ == 0 ? W0 : (seg_ == 1 ? W1 : W2);                              \
        const uint32_t lim_ = seg_ == 0 ? lim0 : (seg_ == 1 ? lim1 : lim2);                      \
        copy_slice<Tr, VEC>(W_, uint32_t(local_) * rb + lane_off, lim_, ring_a + (st) * SL, lane); \
    } while (0)

    // accumulating into one matrix's outputs: the old values of items
    // 64w .. 64w+63 are copied into LDS now (one 4-byte copy per lane, landing
    // with the activations), so the epilogue does not wait on memory for them
    const bool y_early = a.accumulate && !pairs && a.seg_end[0] == a.rows && nitems <= 64 * nwv;
    if (y_early) {
        const int t = 64 * wave + lane;
        const uint32_t off = uint32_t(b + (t < nitems ? t : 0) * G) * 4u;
        dma<4>(reinterpret_cast<const uint8_t *>(a.y[0]), off, lds_addr(ypre) + 256u * uint32_t(wave));
    }
    typename Tr::X xs;
    float gv[NORM ? 64 : 1];
    float ss = 0.f;
    if constexpr (SHARED) {
        // this wave's share of the activation (and gain) copies; they land
        // while the first rows are in flight
        const uint32_t xa_a = lds_addr(xa) + uint32_t(cw) * 16384u;
        copy_vec_pieces<Tr>(a.x, a.cols, cw, lane, xa_a, grp, R);
        if constexpr (NORM) copy_vec_pieces<Tr>(a.gain, a.cols, cw, lane, xa_a + uint32_t(nw) * 16384u, grp, R);
    } else {
        // activations (and gains) through this wave's ring area, before any row
        stage_vec<Tr>(a.x, a.cols, cw, lane, ring, ring_a, xs.v);
        if constexpr (NORM) stage_vec<Tr>(a.gain, a.cols, cw, lane, ring, ring_a, gv);
    }
    // S ring slots (placeholders past the last row, so the count is fixed)
#pragma unroll
    for (int j = 0; j < S; ++j) {
        if (j < n) NT_ISSUE(j, j);
        else copy_slice<Tr, VEC>(W0, uint32_t(lane * VEC), 0u, ring_a + j * SL, lane);   // placeholder: 16 bytes
    }
    if constexpr (SHARED) {
        // own copies done (the ring loads issued after them may still be in
        // flight), then every wave's
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(S * NI));
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
        read_vec(xa + cw * 16384, lane, xs.v);
        if constexpr (NORM) read_vec(ga + cw * 16384, lane, gv);
    }
    if constexpr (NORM) {
        // RMSNorm of the activation vector: the nw waves of a row group
        // cover every column, so each group forms 1/rms itself
#pragma unroll
        for (int i = 0; i < 64; ++i) ss = fmaf(xs.v[i], xs.v[i], ss);
        ss = ok ? ss : 0.f;
        ss = wave_sum_to_lane63(ss);
        if (lane == 63) red[wave] = ss;
        __builtin_amdgcn_s_waitcnt(kLgkm0);
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
        float tot = 0.f;
        for (int w = 0; w < nw; ++w) tot += red[grp * nw + w];
        const float inv = 1.0f / sqrtf(tot / float(a.cols) + a.eps);
#pragma unroll
        for (int i = 0; i < 64; ++i) xs.v[i] = gv[i] * (xs.v[i] * inv);
    }
    Tr::sums(xs);

    // Row j is decoded from registers while row j+1 is read from LDS and rows
    // up to j+S are in flight: row j's stage (j mod S) was read into registers
    // during the previous step, so it is refilled at once.
    typename Tr::Raw ra, rb2;
    __builtin_amdgcn_s_waitcnt(vmcnt_imm((S - 1) * NI));    // row 0 has landed
    __builtin_amdgcn_sched_barrier(0);
    Tr::load(ring, L, ra);
    int cs = 0;
#define NT_STEP(j, cur, nxt)                                                                 \
    {                                                                                        \
        __builtin_amdgcn_sched_barrier(0);                                                   \
        const int sn = cs + 1 == S ? 0 : cs + 1;                /* stage of row j+1 */       \
        __builtin_amdgcn_s_waitcnt(kLgkm0);           /* row j is in registers, its stage free */ \
        if ((j) + S < n) {                                                                   \
            NT_ISSUE((j) + S, cs);                                                           \
            __builtin_amdgcn_s_waitcnt(vmcnt_imm((S - 1) * NI)); /* row j+1 has landed */    \
        } else {                                                                             \
            __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));                                        \
        }                                                                                    \
        __builtin_amdgcn_sched_barrier(0);                                                   \
        if ((j) + 1 < n) Tr::load(ring + sn * SL, L, nxt);                                   \
        float v_ = Tr::dot(cur, xs, L);                                                      \
        v_ = ok ? v_ : 0.f;                                                                  \
        v_ = wave_sum_to_lane63(v_);                                                         \
        if (lane == 63) part[wave * kMaxRowsPerWG + (j)] = v_;                               \
        cs = sn;                                                                             \
    }
    // the first wave on each SIMD outranks the second by age; alternate an
    // explicit priority per row so both advance at the same pace
    const bool first_slot = wave < 4;
    for (int j = 0; j < n; j += 2) {
        if (first_slot) __builtin_amdgcn_s_setprio(1); else __builtin_amdgcn_s_setprio(0);
        NT_STEP(j, ra, rb2);
        if (j + 1 >= n) break;
        if (first_slot) __builtin_amdgcn_s_setprio(0); else __builtin_amdgcn_s_setprio(1);
        NT_STEP(j + 1, rb2, ra);
    }
    __builtin_amdgcn_s_setprio(0);
    // a wave with no rows still has its placeholder copies outstanding
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    __syncthreads();

    // combine the column slices in a fixed order
    if (pairs) {
        float *h = a.y[0];
        for (int t = threadIdx.x; t < nitems; t += blockDim.x) {
            const int jj = int((uint32_t(t) * inv_r) >> 16), g = t - jj * R;
            const float *pp = part + g * nw * kMaxRowsPerWG + 2 * jj;
            float gs = 0.f, up = 0.f;
            for (int w = 0; w < nw; ++w) {
                gs += pp[w * kMaxRowsPerWG];
                up += pp[w * kMaxRowsPerWG + 1];
            }
            h[b + t * G] = gs / (1.0f + expf(-gs)) * up;
        }
    } else {
        for (int t = threadIdx.x; t < nitems; t += blockDim.x) {
            const int jj = int((uint32_t(t) * inv_r) >> 16), g = t - jj * R;
            const float *pp = part + g * nw * kMaxRowsPerWG + jj;
            float sum = 0.f;
            for (int w = 0; w < nw; ++w) sum += pp[w * kMaxRowsPerWG];
            const int r = b + t * G;
            NT_SEG(r);
            float *y = (seg_ == 0 ? a.y[0] : (seg_ == 1 ? a.y[1] : a.y[2])) + local_;
            *y = a.accumulate ? (y_early ? ypre[t] : *y) + sum : sum;
        }
    }
#undef NT_STEP
#undef NT_ISSUE
#undef NT_LOCATE
#undef NT_SEG
}

template <class Tr, int VEC, bool NORM, bool SHARED>
__global__ void __launch_bounds__(512) gemv_lds(const GemvArgs a) {
    gemv_body<Tr, VEC, NORM, SHARED>(a, blockIdx.x, gridDim.x);
}

// Two GEMVs of different formats over the same activations in one launch
// (shared layout, same row width): workgroups [0, ga) run the first, the rest
// the second.  The decode step uses it for the q/k (Q4_K) and v (Q6_K)
// projections of the mixed-format models.
template <class TrA, class TrB, bool NORM>
__global__ void __launch_bounds__(512) gemv_pair(const GemvArgs a, const GemvArgs c, const int ga) {
    if (int(blockIdx.x) < ga)
        gemv_body<TrA, 16, NORM, true>(a, blockIdx.x, ga);
    else
        gemv_body<TrB, 16, NORM, true>(c, blockIdx.x - ga, gridDim.x - ga);
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

// Per-device facts the launch shape depends on.
struct DevInfo {
    int cus = 0;
    int lds_per_cu = 0;
};

int current_device() {
    int d = 0;
    if (hipGetDevice(&d) != hipSuccess || d < 0 || d >= 64) d = 0;
    return d;
}

// Filled once per device, under a lock (launches may come from several
// threads).
DevInfo dev_info() {
    static std::mutex mu;
    static DevInfo cache[64];
    const int d = current_device();
    std::lock_guard<std::mutex> lock(mu);
    DevInfo &di = cache[d];
    if (di.cus == 0) {
        int cus = 0, lds = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, d) != hipSuccess || cus <= 0) cus = 256;
        if (hipDeviceGetAttribute(&lds, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor, d) != hipSuccess ||
            lds <= 0)
            lds = 160 * 1024;
        di.lds_per_cu = lds;
        di.cus = cus;
    }
    return di;
}

// Lets kernel `fn` use all of a CU's LDS as dynamic LDS: set once per device
// (a second, concurrent setting is harmless).  A launch that still exceeds
// the limit fails and is reported by the launch check.
void allow_full_lds(const void *fn, std::atomic<uint64_t> &done) {
    const int d = current_device();
    if ((done.load(std::memory_order_acquire) >> d) & 1) return;
    if (hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, dev_info().lds_per_cu) != hipSuccess)
        (void)hipGetLastError();                // not left for the launch check to report
    done.fetch_or(uint64_t(1) << d, std::memory_order_release);
}

struct LdsShape {
    int nw;              // waves per row group (column slices)
    int groups;          // row groups per workgroup
    bool shared;         // activations in their own LDS area
    int64_t grid;
    size_t lds;
    int rows_per_wg;
};

// Workgroups of `groups` row groups of nw waves (one per 64-unit column
// slice), 8 waves per CU.  Each wave keeps one row in flight while it decodes
// the previous one (a two-stage ring): measured on this part, a streaming read
// through LDS reaches its best rate with about 32 KB in flight per CU (8
// waves, 4 KB each), and deeper rings or more waves lose bandwidth.  Rows of up
// to two column slices (8192 columns) use the shared layout: one workgroup of
// up to 8 waves per CU, activations (and gains) copied once per workgroup into
// an area of their own while the first rows are in flight.  Wider rows: each
// wave stages its slice through a 16 KB area that then holds its ring.  The
// workgroups take even shares of the rows.
template <class Tr>
LdsShape lds_shape(int64_t items, int64_t cols, bool pairs, bool norm, bool vec16) {
    const DevInfo di = dev_info();
    LdsShape s;
    const int64_t units = cols / 64;
    s.nw = int((units + 63) / 64);
    const size_t area = size_t(s.nw) * 16384 * (norm ? 2 : 1);
    // rows of up to two column slices (8192 columns) use the shared layout,
    // and so do wider rows whose activation area fits beside two row groups
    // (which then share one copy of it; with a single group the per-wave
    // layout and its deeper ring measured faster: Q5_K 8192x28672 35.4 vs
    // 36.3 us)
    const size_t ring_sh = size_t(Tr::kStagesShared) * Tr::kSlice;
    const bool fits_one = area + 2 * size_t(s.nw) * (ring_sh + kMaxRowsPerWG * 4 + 4 + 256) <= size_t(di.lds_per_cu);
    const bool shared = vec16 && (cols <= 8192 || fits_one);
    const size_t ring = size_t(shared ? Tr::kStagesShared : Tr::kStagesWide) * Tr::kSlice;
    const size_t per_wave = (shared ? ring : (ring > 16384 ? ring : 16384)) + kMaxRowsPerWG * 4 + 4 + 256;
    s.groups = 1;
    if (shared) {
        int g = 8 / s.nw;
        while (g > 0 && area + size_t(g) * s.nw * per_wave > size_t(di.lds_per_cu)) --g;
        s.groups = g > 0 ? g : 1;      // two slices and their areas always fit one group
    }
    s.shared = shared;
    const int nwv = s.nw * s.groups;
    s.lds = (shared ? area : 0) + size_t(nwv) * per_wave;
    constexpr int waves_cu = 8;
    int64_t per_cu = int64_t(di.lds_per_cu) / int64_t(s.lds);
    const int64_t by_waves = waves_cu / nwv > 0 ? waves_cu / nwv : 1;
    if (per_cu > by_waves) per_cu = by_waves;
    if (per_cu < 1) per_cu = 1;
    int64_t grid = int64_t(di.cus) * per_cu;
    if (grid > items) grid = items;
    const int64_t cap = int64_t(s.groups) * (pairs ? kMaxRowsPerWG / 2 : kMaxRowsPerWG);
    if (grid < (items + cap - 1) / cap) grid = (items + cap - 1) / cap;
    if (grid < 1) grid = 1;
    s.grid = grid;
    const int64_t per = (items + grid - 1) / grid;      // items of workgroup 0, the most
    s.rows_per_wg = int(pairs ? 2 * per : per);
    return s;
}

// ceil(2^16 / d), 1 <= d <= 8: (n * m) >> 16 equals n / d for 0 <= n < 8192
// (the excess n (m - 2^16 / d) / 2^16 stays below 1/8 <= 1/d, and the
// fraction of n / d is at most 1 - 1/d); every count divided this way (a
// wave index, the waves of a workgroup, items per workgroup plus a group
// index) is below 2^11
uint32_t small_inv(int d) { return (65535u + uint32_t(d)) / uint32_t(d); }

// The launch constants of one GEMV (or one side of a paired launch) over
// `grid` workgroups of `groups` row groups of nw waves.
GemvArgs with_launch(GemvArgs a, int64_t grid, int nw, int groups) {
    const int64_t items = a.swiglu ? a.rows / 2 : a.rows;
    a.items_q = int(items / grid);
    a.items_r = int(items % grid);
    a.groups = groups;
    a.inv_nw = nw <= 8 ? small_inv(nw) : 0u;       // used by the shared layout only (nw <= 8 there)
    a.inv_groups = small_inv(groups);
    return a;
}

template <class Tr, int VEC, bool NORM, bool SHARED>
hipError_t launch_lds_inst(const GemvArgs &a0, const LdsShape &s, hipStream_t st) {
    const GemvArgs a = with_launch(a0, s.grid, s.nw, SHARED ? s.groups : 1);
    // allow the large dynamic LDS areas (a launch that still exceeds the
    // limit fails and is reported by the launch check below)
    static std::atomic<uint64_t> done{0};          // devices this kernel is set up on
    allow_full_lds(reinterpret_cast<const void *>(&gemv_lds<Tr, VEC, NORM, SHARED>), done);
    gemv_lds<Tr, VEC, NORM, SHARED><<<dim3(unsigned(s.grid)), dim3(unsigned(64 * s.nw * s.groups)), s.lds, st>>>(a);
    return hipGetLastError();
}

// VEC = 16 when rows are 16-byte aligned (every Q4_K row is), else 4; the
// shared-area layout only with VEC = 16
template <class Tr, bool WORD_ROWS>
hipError_t launch_lds(const GemvArgs &a, bool pairs, bool vec16, hipStream_t st) {
    const bool norm = a.gain != nullptr;
    const LdsShape s = lds_shape<Tr>(pairs ? a.rows / 2 : a.rows, a.cols, pairs, norm, vec16);
    if constexpr (WORD_ROWS) {
        if (!vec16)
            return norm ? launch_lds_inst<Tr, 4, true, false>(a, s, st) : launch_lds_inst<Tr, 4, false, false>(a, s, st);
    }
    if (s.shared)
        return norm ? launch_lds_inst<Tr, 16, true, true>(a, s, st) : launch_lds_inst<Tr, 16, false, true>(a, s, st);
    return norm ? launch_lds_inst<Tr, 16, true, false>(a, s, st) : launch_lds_inst<Tr, 16, false, false>(a, s, st);
}

// Shared-layout shape of one half of a paired launch with `groups` row groups.
template <class Tr>
size_t pair_lds(int nw, int groups, bool norm) {
    return size_t(nw) * 16384 * (norm ? 2 : 1) +
           size_t(nw) * groups * (size_t(Tr::kStagesShared) * Tr::kSlice + kMaxRowsPerWG * 4 + 4 + 256);
}

template <class TrA, class TrB>
hipError_t launch_pair_inst(const GemvArgs &a, const GemvArgs &c, hipStream_t st) {
    // two different formats, RMSNorm prologue: the q/k/v case
    if constexpr (std::is_same_v<TrA, TrB>) {
        return hipErrorInvalidValue;
    } else {
    const DevInfo di = dev_info();
    if (a.gain == nullptr) return hipErrorInvalidValue;
    constexpr bool norm = true;
    const int nw = (a.units + 63) / 64;
    const int ga_max = std::max(8 / nw, 1);
    int groups = ga_max;
    while (groups > 1 && std::max(pair_lds<TrA>(nw, groups, norm), pair_lds<TrB>(nw, groups, norm)) >
                             size_t(di.lds_per_cu))
        --groups;
    const size_t lds = std::max(pair_lds<TrA>(nw, groups, norm), pair_lds<TrB>(nw, groups, norm));
    // one workgroup per CU, split in proportion to the weight bytes, each side
    // within its row-sum capacity and at most one workgroup per row
    const int64_t bytes_a = int64_t(a.rows) * a.row_bytes, bytes_c = int64_t(c.rows) * c.row_bytes;
    const int64_t cap = int64_t(groups) * kMaxRowsPerWG;
    const int64_t min_a = (a.rows + cap - 1) / cap, min_c = (c.rows + cap - 1) / cap;
    int64_t ga = (int64_t(di.cus) * bytes_a + (bytes_a + bytes_c) / 2) / (bytes_a + bytes_c);
    ga = std::min<int64_t>(std::max<int64_t>(ga, min_a), a.rows);
    int64_t gc = std::min<int64_t>(std::max<int64_t>(int64_t(di.cus) - ga, min_c), c.rows);
    if (ga < 1) ga = 1;
    if (gc < 1) gc = 1;
    static std::atomic<uint64_t> done{0};
    allow_full_lds(reinterpret_cast<const void *>(&gemv_pair<TrA, TrB, true>), done);
    gemv_pair<TrA, TrB, true><<<dim3(unsigned(ga + gc)), dim3(unsigned(64 * nw * groups)), lds, st>>>(
        with_launch(a, ga, nw, groups), with_launch(c, gc, nw, groups), int(ga));
    return hipGetLastError();
    }
}

template <class TrA>
hipError_t launch_pair_b(nt_qtype tb, const GemvArgs &a, const GemvArgs &c, hipStream_t st) {
    switch (tb) {
    case NT_Q8_0: return launch_pair_inst<TrA, F80>(a, c, st);
    case NT_Q4_0: return launch_pair_inst<TrA, F40>(a, c, st);
    case NT_Q4_K: return launch_pair_inst<TrA, F4K>(a, c, st);
    case NT_Q5_K: return launch_pair_inst<TrA, F5K>(a, c, st);
    case NT_Q6_K: return launch_pair_inst<TrA, F6K>(a, c, st);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace

bool gemv_pair_ok(nt_qtype t, int64_t rows, int64_t cols) {
    return gemv_fast_ok(t, rows, cols) && cols <= 8192 && gemv_row_bytes(t, cols) % 16 == 0;
}

hipError_t launch_gemv_pair(nt_qtype ta, int na, const void *const *Wa, const int64_t *rows_a, float *const *ya,
                            nt_qtype tb, int nb, const void *const *Wb, const int64_t *rows_b, float *const *yb,
                            int64_t cols, const float *x, const float *gain, float eps, hipStream_t st) {
    const GemvArgs a = gemv_args(ta, na, Wa, rows_a, ya, cols, x, gain, eps, 0);
    const GemvArgs c = gemv_args(tb, nb, Wb, rows_b, yb, cols, x, gain, eps, 0);
    switch (ta) {
    case NT_Q8_0: return launch_pair_b<F80>(tb, a, c, st);
    case NT_Q4_0: return launch_pair_b<F40>(tb, a, c, st);
    case NT_Q4_K: return launch_pair_b<F4K>(tb, a, c, st);
    case NT_Q5_K: return launch_pair_b<F5K>(tb, a, c, st);
    case NT_Q6_K: return launch_pair_b<F6K>(tb, a, c, st);
    default: return hipErrorInvalidValue;
    }
}

int64_t gemv_row_bytes(nt_qtype t, int64_t cols) { return cols / block_elems(t) * block_bytes(t); }

bool gemv_fast_ok(nt_qtype t, int64_t rows, int64_t cols) {
    const int64_t rb = gemv_row_bytes(t, cols);
    // word-aligned rows, whole 64-value units, at most 8 column slices, and
    // byte offsets that fit in 32 bits
    return rb % 4 == 0 && cols % 64 == 0 && cols > 0 && cols <= 32768 &&
           rows * rb < (int64_t(1) << 32);
}

void gemv_launch_info(nt_qtype t, int64_t rows, int64_t cols, int32_t info[4]) {
    if (gemv_fast_ok(t, rows, cols)) {
        const bool vec16 = gemv_row_bytes(t, cols) % 16 == 0;
        LdsShape s{};
        switch (t) {
        case NT_Q8_0: s = lds_shape<F80>(rows, cols, false, false, vec16); break;
        case NT_Q4_0: s = lds_shape<F40>(rows, cols, false, false, vec16); break;
        case NT_Q4_K: s = lds_shape<F4K>(rows, cols, false, false, vec16); break;
        case NT_Q5_K: s = lds_shape<F5K>(rows, cols, false, false, vec16); break;
        default: s = lds_shape<F6K>(rows, cols, false, false, vec16); break;
        }
        info[0] = 1 + (vec16 ? 1 : 0);   // 2: 16-byte copies, 1: 4-byte
        info[1] = s.rows_per_wg;
        info[2] = int32_t(s.grid);
        info[3] = 64 * s.nw * s.groups;
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

hipError_t launch_gemv_fused(nt_qtype t, const GemvArgs &a, bool pairs, hipStream_t st) {
    const bool vec16 = a.row_bytes % 16 == 0;
    switch (t) {
    case NT_Q8_0: return launch_lds<F80, true>(a, pairs, vec16, st);
    case NT_Q4_0: return launch_lds<F40, true>(a, pairs, vec16, st);
    case NT_Q4_K: return launch_lds<F4K, false>(a, pairs, true, st);
    case NT_Q5_K: return launch_lds<F5K, false>(a, pairs, true, st);
    case NT_Q6_K: return launch_lds<F6K, true>(a, pairs, vec16, st);
    default: return hipErrorInvalidValue;
    }
}

GemvArgs gemv_args(nt_qtype t, int nseg, const void *const *W, const int64_t *rows, float *const *y, int64_t cols,
                   const float *x, const float *gain, float eps, int accumulate) {
    GemvArgs a{};
    const int64_t rb = gemv_row_bytes(t, cols);
    const int vec = rb % 16 == 0 ? 16 : 4;
    int64_t end = 0;
    for (int s = 0; s < 3; ++s) {
        const int k = s < nseg ? s : nseg - 1;        // unused slots repeat the last matrix
        a.W[s] = static_cast<const uint8_t *>(W[k]);
        a.y[s] = y[k];
        if (s < nseg) end += rows[s];
        a.seg_end[s] = int32_t(end);
        a.seg_lim[s] = uint32_t(rows[k] * rb - vec);
    }
    a.x = x;
    a.gain = gain;
    a.eps = eps;
    a.cols = int(cols);
    a.rows = int(end);
    a.units = int(cols / 64);
    a.row_bytes = uint32_t(rb);
    a.accumulate = accumulate;
    a.swiglu = 0;
    return a;
}

hipError_t launch_gemv(nt_qtype t, const void *W, const float *x, float *y, int64_t rows,
                       int64_t cols, int accumulate, hipStream_t st) {
    if (gemv_fast_ok(t, rows, cols)) {
        const GemvArgs a = gemv_args(t, 1, &W, &rows, &y, cols, x, nullptr, 0.f, accumulate);
        return launch_gemv_fused(t, a, false, st);
    }
    switch (t) {
    case NT_Q8_0: return launch_generic<Q80>(W, x, y, rows, cols, accumulate, st);
    case NT_Q4_0: return launch_generic<Q40>(W, x, y, rows, cols, accumulate, st);
    case NT_Q4_K: return launch_generic<Q4K>(W, x, y, rows, cols, accumulate, st);
    case NT_Q5_K: return launch_generic<Q5K>(W, x, y, rows, cols, accumulate, st);
    case NT_Q6_K: return launch_generic<Q6K>(W, x, y, rows, cols, accumulate, st);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_gemv_multi(nt_qtype t, int nseg, const void *const *W, const int64_t *rows, float *const *y,
                             int64_t cols, const float *x, const float *gain, float eps, int accumulate,
                             hipStream_t st) {
    const GemvArgs a = gemv_args(t, nseg, W, rows, y, cols, x, gain, eps, accumulate);
    return launch_gemv_fused(t, a, false, st);
}

hipError_t launch_gemv_swiglu(nt_qtype t, const void *Wg, const void *Wu, int64_t rows, int64_t cols,
                              const float *x, const float *gain, float eps, float *h, hipStream_t st) {
    const void *W[2] = {Wg, Wu};
    const int64_t r[2] = {rows, rows};
    float *y[2] = {h, h};
    GemvArgs a = gemv_args(t, 2, W, r, y, cols, x, gain, eps, 0);
    a.swiglu = 1;
    return launch_gemv_fused(t, a, true, st);
}

}  // namespace nt
