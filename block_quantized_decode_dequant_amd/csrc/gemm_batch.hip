// gemm_batch.hip -- y_n = W x_n (+ y_n) for k <= 8 activation vectors against
// one block-quantized matrix: the verify pass of self-speculative decoding.
//
// The ntransformer write-up ("Overview", self-speculative decoding) has the
// VRAM-resident layers draft several tokens that the whole model then checks
// in one pass, so the matrices are read once for k tokens instead of k times.
// At k = 8 the arithmetic is 16 flops per weight; Q4_K at HBM speed would
// need about 230 TFLOP/s of fp32 FMA, above the vector units' peak, so the
// products run on the matrix cores (v_mfma_f32_16x16x16_f16):
//
//  * the MFMA's M dimension holds the activations, N the 16 weight rows of a
//    tile, K 16 codes of one scale group (Q8_0, Q4_0) or any 16 codes of a
//    super-block whose scales are folded into the codes (K-quants).  With N = weight row, every lane applies the
//    scales of its own row to its own accumulators.
//  * weight codes become fp16 exactly: small integers, or with the scales
//    folded in (Q4_K, Q5_K: S_j * q * 2^-14; Q6_K: sc * ql4 and
//    16 sc (qh2 - 2), the two parts of its code, in two MFMAs).  Nothing
//    about the weights is rounded.
//  * each activation is split into fp16 hi + lo (hi = fp16(x), lo =
//    fp16(x - hi)), which leaves about 2^-22 relative error; the hi parts fill
//    M rows 0-7 and the lo parts rows 8-15, which the padding of k <= 8 to 16
//    would otherwise waste.  Products are exact in fp32; the MFMA sums in fp32.
//  * a prologue kernel writes the split activations once per call in the
//    order the lanes consume them: each of a wave's eight 16-byte loads per
//    256 columns reads one contiguous kilobyte.
//  * MFMA lane layout (16x16x16 f16): src0 lane l holds A[l % 16][4(l/16) + i],
//    src1 lane l holds B[4(l/16) + i][l % 16], the result lane l holds
//    D[4(l/16) + i][l % 16], i = 0..3.  Inside one MFMA the order of the 16
//    K slots is free as long as A and B agree, so each lane takes the codes of
//    its row that lie together in memory.
//
// A workgroup of kWaves waves owns 16 * kTiles rows; each wave takes all its
// tiles and interleaved 256-column steps, and the waves add their partial
// sums through LDS in a fixed order.
#include <algorithm>
#include <type_traits>

#include "device_util.h"
#include "nt_internal.h"

namespace nt {
namespace {

typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef uint32_t w2 __attribute__((ext_vector_type(2)));

constexpr int kWaves = 4;   // waves of a workgroup (they split the columns)
// 16-row tiles of a wave (they share the activation loads): 2, or 4 for
// Q4_K matrices of at least kTallRows rows (enough workgroups to fill the
// chip; fewer activation bytes per weight byte)
constexpr int kTallRows = 16384;

// Order of a dword's four bytes in the K slots of one lane: the halves of
// (w & 0x00ff00ff) then of (w >> 8 & 0x00ff00ff), i.e. bytes 0, 2, 1, 3.
__host__ __device__ constexpr int perm4(int i) { return (i & 1) * 2 + (i >> 1); }

__device__ __forceinline__ h4 pack(uint32_t lo, uint32_t hi) { return __builtin_bit_cast(h4, w2{lo, hi}); }
__device__ __forceinline__ uint32_t hadd(uint32_t w, _Float16 c) {
    return __builtin_bit_cast(uint32_t, __builtin_bit_cast(h2, w) + h2{c, c});
}
__device__ __forceinline__ uint32_t hmul(uint32_t w, _Float16 c) {
    return __builtin_bit_cast(uint32_t, __builtin_bit_cast(h2, w) * h2{c, c});
}
__device__ __forceinline__ f4 mfma(h4 a, h4 b, f4 c) { return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0); }

// Per format: load() issues every global load of one 256-column step into
// a Raw of registers (no use of the data), compute() turns a loaded Raw into
// MFMAs, so the main loop can keep the next step's loads in flight.

// ---- Q8_0: a step is 8 blocks; MFMA m covers block m/2, values
// 8g + 4(m&1) + perm4(i) for lane group g.  A block starts 2-byte aligned
// (bs = its address mod 4, 0 or 2); each lane loads the 12 bytes at the
// word-aligned address b - bs + 8g, which hold its 8 code bytes (from byte
// 2 + bs of the load) and, in lane group 0, the block's d (bytes bs, bs + 1),
// handed to the row's other lanes by a lane permute.  The load ends at most
// at byte 36 - bs of the block, inside the word that holds its last bytes.
// Blocks past the end of a row (a partial last step) load block 0 of the row
// and get scale 0.
struct BQ80 {
    static constexpr bool kMin = false;
    struct Raw { u32x3 v[8]; };
    __host__ __device__ static int elem(int m, int g, int i) { return 32 * (m >> 1) + 8 * g + 4 * (m & 1) + perm4(i); }
    __device__ static void load(const uint8_t *row, int s, int g, int nblk, Raw &r) {
#pragma unroll
        for (int bb = 0; bb < 8; ++bb) {
            const int blk = 8 * s + bb;
            const uint8_t *b = row + int64_t(blk < nblk ? blk : 0) * 34;
            const uint32_t bs = uint32_t(reinterpret_cast<uintptr_t>(b) & 3);   // 0 or 2
            r.v[bb] = ld3(b - bs + 8 * g);
        }
    }
    // int8 codes of a word -> two fp16 pairs q (bytes 0,2 and 1,3): 0x64uu is
    // 1024 + uu, the sign bit flipped makes uu = q + 128.
    __device__ static h4 codes(uint32_t w) {
        const uint32_t a = hadd((w & 0x00ff00ffu) ^ 0x64806480u, _Float16(-1152.f));
        const uint32_t b = hadd(((w >> 8) & 0x00ff00ffu) ^ 0x64806480u, _Float16(-1152.f));
        return pack(a, b);
    }
    __device__ static void compute(const Raw &r, const uint8_t *row, int s, int nblk, const h4 *xa, h4, f4 &acc) {
        const int src = int(__lane_id() & 15);          // lane group 0 of this row
        const uint32_t sel2 = shift_sel(2);
#pragma unroll
        for (int bb = 0; bb < 8; ++bb) {
            const int blk = 8 * s + bb;
            const bool live = blk < nblk;
            const uint8_t *b = row + int64_t(live ? blk : 0) * 34;
            const uint32_t bs = uint32_t(reinterpret_cast<uintptr_t>(b) & 3);
            const u32x3 v = r.v[bb];
            const uint32_t w0 = bs ? v.y : funnel(v.y, v.x, sel2);
            const uint32_t w1 = bs ? v.z : funnel(v.z, v.y, sel2);
            const uint32_t dw = uint32_t(__shfl(int(v.x), src, 64));
            const float d = live ? h2f(bs ? dw >> 16 : dw) : 0.f;
            f4 c = mfma(xa[2 * bb], codes(w0), f4{0.f, 0.f, 0.f, 0.f});
            c = mfma(xa[2 * bb + 1], codes(w1), c);
            acc += d * c;
        }
    }
};

// ---- Q4_K: a step is one super-block.  The 6-bit scales are folded into
// the codes: (q * 2^-24 or q * 2^-20 as an fp16 subnormal) * fp16(S * 2^10
// or S * 2^6) = S q 2^-14 exactly (S q <= 945), so one MFMA chain covers the
// whole super-block and any value may sit in any K slot.  Lane group g takes
// code bytes [16g, 16g + 16) and [64 + 16g, 64 + 16g + 16), so each load
// instruction reads 64 contiguous bytes of a row.  MFMA m uses word m / 2 of
// those eight (low nibbles for even m, high for odd); code byte c holds
// values 32 (2 (c / 32)) + c % 32 (low) and 32 (2 (c / 32) + 1) + c % 32
// (high).  The mins go through one more MFMA: A = per-sub-block activation
// sums (hi in K slots 0-7, lo in 8-15), B = M_j.
struct BQ4K {
    static constexpr bool kMin = true;
    struct Raw { u32x4 h, q0, q1; };
    __host__ __device__ static int code_byte(int w, int g) { return w < 4 ? 16 * g + 4 * w : 64 + 16 * g + 4 * (w - 4); }
    __host__ __device__ static int elem(int m, int g, int i) {
        const int c = code_byte(m >> 1, g) + perm4(i);
        return 32 * (2 * (c >> 5) + (m & 1)) + (c & 31);
    }
    __device__ static void load(const uint8_t *row, int s, int g, int, Raw &r) {
        const uint8_t *b = row + int64_t(s) * 144;
        r.h = ld4(b);
        r.q0 = ld4(b + 16 + 16 * g);
        r.q1 = ld4(b + 80 + 16 * g);
    }
    __device__ static void scale_min(const u32x4 &h, int j, uint32_t &S, uint32_t &M) {
        const uint32_t sc[3] = {h.y, h.z, h.w};
        auto byte = [&](int k) { return (sc[k >> 2] >> (8 * (k & 3))) & 0xffu; };
        if (j < 4) {
            S = byte(j) & 63;
            M = byte(j + 4) & 63;
        } else {
            S = (byte(j + 4) & 15) | ((byte(j - 4) >> 6) << 4);
            M = (byte(j + 4) >> 4) | ((byte(j) >> 6) << 4);
        }
    }
    __device__ static void compute(const Raw &r, int g, const h4 *xa, h4 xm, f4 &acc) {
        uint32_t S[8], M[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) scale_min(r.h, j, S[j], M[j]);
        // the two code pairs of this lane: chunks g / 2 (bytes 16g..) and 2 + g / 2 (bytes 64 + 16g..)
        const int hp = g >> 1;
        const uint32_t Sa0 = hp ? S[2] : S[0], Sa1 = hp ? S[3] : S[1];
        const uint32_t Sb0 = hp ? S[6] : S[4], Sb1 = hp ? S[7] : S[5];
        const _Float16 fa0 = _Float16(float(Sa0 * 1024u)), fa1 = _Float16(float(Sa1 * 64u));
        const _Float16 fb0 = _Float16(float(Sb0 * 1024u)), fb1 = _Float16(float(Sb1 * 64u));
        const uint32_t words[8] = {r.q0.x, r.q0.y, r.q0.z, r.q0.w, r.q1.x, r.q1.y, r.q1.z, r.q1.w};
        f4 c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int w = 0; w < 8; ++w) {
            const uint32_t v = words[w], t = v >> 8;
            const _Float16 f0 = w < 4 ? fa0 : fb0, f1 = w < 4 ? fa1 : fb1;
            c = mfma(xa[2 * w], pack(hmul(v & 0x000f000fu, f0), hmul(t & 0x000f000fu, f0)), c);
            c = mfma(xa[2 * w + 1], pack(hmul(v & 0x00f000f0u, f1), hmul(t & 0x00f000f0u, f1)), c);
        }
        // B of the min MFMA: K slot 4g + i takes M_{(4g + i) & 7}
        const int jb = 4 * (g & 1);
        const uint32_t m0 = jb ? M[4] : M[0], m1 = jb ? M[5] : M[1], m2 = jb ? M[6] : M[2], m3 = jb ? M[7] : M[3];
        const h4 mb = {_Float16(float(m0)), _Float16(float(m1)), _Float16(float(m2)), _Float16(float(m3))};
        const f4 cm = mfma(xm, mb, f4{0.f, 0.f, 0.f, 0.f});
        const float d = h2f(r.h.x) * 16384.f, dmin = h2f(r.h.x >> 16);
        acc += d * c - dmin * cm;
    }
};

// ---- Q4_0: a step is 8 blocks of 18 bytes; lane group g takes code bytes
// 4g..4g+3 of a block: MFMA 2bb holds their low nibbles (values
// 4g + perm4(i)), MFMA 2bb + 1 their high nibbles (16 + 4g + perm4(i)).
// Codes become q - 8 exactly.  As for Q8_0, each lane loads 8 bytes from the
// word-aligned address b - bs + 4g (its code bytes from byte 2 + bs; d in
// lane group 0, permuted to the others); the load ends at most at byte
// 20 - bs of the block, inside the word that holds its last bytes.
struct BQ40 {
    static constexpr bool kMin = false;
    struct Raw { u32x2 v[8]; };
    __host__ __device__ static int elem(int m, int g, int i) { return 32 * (m >> 1) + 16 * (m & 1) + 4 * g + perm4(i); }
    __device__ static void load(const uint8_t *row, int s, int g, int nblk, Raw &r) {
#pragma unroll
        for (int bb = 0; bb < 8; ++bb) {
            const int blk = 8 * s + bb;
            const uint8_t *b = row + int64_t(blk < nblk ? blk : 0) * 18;
            const uint32_t bs = uint32_t(reinterpret_cast<uintptr_t>(b) & 3);   // 0 or 2
            r.v[bb] = *reinterpret_cast<const u32x2 *>(b - bs + 4 * g);
        }
    }
    __device__ static h4 nib(uint32_t w) {   // bits 0-3 of each byte: q - 8 as fp16, bytes 0,2 then 1,3
        const uint32_t a = hadd((w & 0x000f000fu) | 0x64006400u, _Float16(-1032.f));
        const uint32_t b = hadd(((w >> 8) & 0x000f000fu) | 0x64006400u, _Float16(-1032.f));
        return pack(a, b);
    }
    __device__ static void compute(const Raw &r, const uint8_t *row, int s, int nblk, const h4 *xa, h4, f4 &acc) {
        const int src = int(__lane_id() & 15);          // lane group 0 of this row
        const uint32_t sel2 = shift_sel(2);
#pragma unroll
        for (int bb = 0; bb < 8; ++bb) {
            const int blk = 8 * s + bb;
            const bool live = blk < nblk;
            const uint8_t *b = row + int64_t(live ? blk : 0) * 18;
            const uint32_t bs = uint32_t(reinterpret_cast<uintptr_t>(b) & 3);
            const u32x2 v = r.v[bb];
            const uint32_t w = bs ? v.y : funnel(v.y, v.x, sel2);
            const uint32_t dw = uint32_t(__shfl(int(v.x), src, 64));
            const float d = live ? h2f(bs ? dw >> 16 : dw) : 0.f;
            f4 c = mfma(xa[2 * bb], nib(w), f4{0.f, 0.f, 0.f, 0.f});
            c = mfma(xa[2 * bb + 1], nib(w >> 4), c);
            acc += d * c;
        }
    }
};

// ---- Q5_K: as Q4_K (same lanes and K slots, scales folded into the
// codes, one more MFMA for the mins) with the fifth bit of value 32j + l in
// bit j of qh[l].  A lane's code bytes c all have c % 32 in
// [16 (g % 2), 16 (g % 2) + 16), so one 16-byte piece of qh serves them.
// S q <= 63 * 31 = 1953 keeps S q 2^-14 exact in fp16.
struct BQ5K {
    static constexpr bool kMin = true;
    struct Raw { u32x4 h, qh, q0, q1; };
    __host__ __device__ static int elem(int m, int g, int i) { return BQ4K::elem(m, g, i); }
    __device__ static void load(const uint8_t *row, int s, int g, int, Raw &r) {
        const uint8_t *b = row + int64_t(s) * 176;
        r.h = ld4(b);
        r.qh = ld4(b + 16 + 16 * (g & 1));
        r.q0 = ld4(b + 48 + 16 * g);
        r.q1 = ld4(b + 112 + 16 * g);
    }
    __device__ static void compute(const Raw &r, int g, const h4 *xa, h4 xm, f4 &acc) {
        uint32_t S[8], M[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) BQ4K::scale_min(r.h, j, S[j], M[j]);
        const int hp = g >> 1;
        const uint32_t words[8] = {r.q0.x, r.q0.y, r.q0.z, r.q0.w, r.q1.x, r.q1.y, r.q1.z, r.q1.w};
        const uint32_t hw[4] = {r.qh.x, r.qh.y, r.qh.z, r.qh.w};
        f4 c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int w = 0; w < 8; ++w) {
            const int p = w < 4 ? hp : 2 + hp;                 // code chunk: sub-blocks 2p, 2p + 1
            const uint32_t S0 = (w < 4 ? (hp ? S[2] : S[0]) : (hp ? S[6] : S[4]));
            const uint32_t S1 = (w < 4 ? (hp ? S[3] : S[1]) : (hp ? S[7] : S[5]));
            const _Float16 f0 = _Float16(float(S0 * 1024u)), f1 = _Float16(float(S1 * 1024u));
            const uint32_t v = words[w], hb = hw[w & 3];
            const uint32_t q0 = (v & 0x0f0f0f0fu) | (((hb >> (2 * p)) & 0x01010101u) << 4);
            const uint32_t q1 = ((v >> 4) & 0x0f0f0f0fu) | (((hb >> (2 * p + 1)) & 0x01010101u) << 4);
            c = mfma(xa[2 * w], pack(hmul(q0 & 0x001f001fu, f0), hmul((q0 >> 8) & 0x001f001fu, f0)), c);
            c = mfma(xa[2 * w + 1], pack(hmul(q1 & 0x001f001fu, f1), hmul((q1 >> 8) & 0x001f001fu, f1)), c);
        }
        const int jb = 4 * (g & 1);
        const uint32_t m0 = jb ? M[4] : M[0], m1 = jb ? M[5] : M[1], m2 = jb ? M[6] : M[2], m3 = jb ? M[7] : M[3];
        const h4 mb = {_Float16(float(m0)), _Float16(float(m1)), _Float16(float(m2)), _Float16(float(m3))};
        const f4 cm = mfma(xm, mb, f4{0.f, 0.f, 0.f, 0.f});
        const float d = h2f(r.h.x) * 16384.f, dmin = h2f(r.h.x >> 16);
        acc += d * c - dmin * cm;
    }
};

// ---- Q6_K: a step is one super-block (210 bytes, so only 2-byte aligned).
// Value (h, k, l) = 128h + 32k + l has code q = ql4 + 16 qh2 (ql4: nibble
// k / 2 of ql[64h + 32 (k % 2) + l], qh2: bits 2k, 2k + 1 of qh[32h + l]) and
// scale sc = scales[8h + 2k + l / 16]; q - 32 = ql4 + 16 (qh2 - 2), and both
// sc * ql4 (<= 1920) and 16 sc (qh2 - 2) (16 times an integer <= 256) are
// exact in fp16, so the scales fold into the codes: two MFMAs per operand
// (one per part) cover any mix of scale groups and d is applied once.  Lane
// group g takes ql bytes [16g, 16g + 16) and [64 + 16g, 64 + 16g + 16) (each
// load reads 64 contiguous bytes of a row), the qh bytes of the same values
// ([16 (g % 2), + 16) of each 32-byte half) and scale bytes g, g + 4,
// g + 8, g + 12.  Every 16-byte piece is two aligned loads and a funnel.
struct BQ6K {
    static constexpr bool kMin = false;
    struct Raw { u32x4 v[5]; uint32_t e[5], dw; };   // ql pieces 0, 1, qh pieces 0, 1, scales; next words; d
    __host__ __device__ static int elem(int m, int g, int i) {
        const int c = BQ4K::code_byte(m >> 1, g) + perm4(i);
        return 128 * (c >> 6) + 32 * (((c >> 5) & 1) + 2 * (m & 1)) + (c & 31);
    }
    __device__ static void load(const uint8_t *row, int s, int g, int, Raw &r) {
        const uint8_t *b = row + int64_t(s) * 210;
        const uint32_t sh = uint32_t(reinterpret_cast<uintptr_t>(b) & 2);
        const uint8_t *a = b - sh;
        const int off[5] = {16 * g, 64 + 16 * g, 128 + 16 * (g & 1), 160 + 16 * (g & 1), 192};
#pragma unroll
        for (int t = 0; t < 5; ++t) {
            r.v[t] = ld4(a + off[t]);
            r.e[t] = ld1(a + off[t] + (sh ? 16 : 12));     // with sh == 0 the last word again
        }
        r.dw = ld1(a + 208);                                 // d: bytes 208, 209
    }
    __device__ static void compute(const Raw &r, const uint8_t *row, int s, int g, const h4 *xa, f4 &acc) {
        const uint32_t sh = uint32_t(reinterpret_cast<uintptr_t>(row + int64_t(s) * 210) & 2);
        const uint32_t sel = shift_sel(sh);
        uint32_t w[5][4];
#pragma unroll
        for (int t = 0; t < 5; ++t) {
            w[t][0] = funnel(r.v[t].y, r.v[t].x, sel);
            w[t][1] = funnel(r.v[t].z, r.v[t].y, sel);
            w[t][2] = funnel(r.v[t].w, r.v[t].z, sel);
            w[t][3] = funnel(r.e[t], r.v[t].w, sel);
        }
        const float d = h2f(sh ? r.dw >> 16 : r.dw);
        const uint32_t kk2 = 2 * uint32_t(g >> 1);          // qh bit of k = g / 2 (+4 for the high nibbles)
        f4 c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int m = 0; m < 16; ++m) {
            const int wi = m >> 1, nib = m & 1, half = wi >> 2;
            const uint32_t v = w[half][wi & 3], hb = w[2 + half][wi & 3];
            const int scw = nib + 2 * half;                 // scale groups g + 4 nib + 8 half: byte g of word scw
            const float sc = float(int8_t((w[4][scw] >> (8 * g)) & 0xffu));
            const _Float16 f = _Float16(sc), f16x = _Float16(16.f * sc);
            const uint32_t ql4 = (nib ? v >> 4 : v) & 0x0f0f0f0fu;
            const uint32_t qh2 = (hb >> (kk2 + 4 * nib)) & 0x03030303u;
            const h4 b1 = pack(hmul(hadd((ql4 & 0x00ff00ffu) | 0x64006400u, _Float16(-1024.f)), f),
                               hmul(hadd(((ql4 >> 8) & 0x00ff00ffu) | 0x64006400u, _Float16(-1024.f)), f));
            const h4 b2 = pack(hmul(hadd((qh2 & 0x00ff00ffu) | 0x64006400u, _Float16(-1026.f)), f16x),
                               hmul(hadd(((qh2 >> 8) & 0x00ff00ffu) | 0x64006400u, _Float16(-1026.f)), f16x));
            c = mfma(xa[m], b1, c);
            c = mfma(xa[m], b2, c);
        }
        acc += d * c;
    }
};

// Split activations in lane order: xp[(((s * 8 + m / 2) * 64 + lane) * 2 + m % 2) * 4 + i]
// (fp16) = hi or lo part of x_n[256 s + elem(m, g, i)], n = lane % 8,
// lo for lane % 16 >= 8, zero for n >= k or past cols.  For K-quant mins,
// xm[(s * 64 + lane) * 4 + i]: K slot 4g + i of lane (b, g) is the hi (slots
// 0-7) or lo (8-15) part of the fp32 sum of x_b over sub-block (4g + i) & 7
// (four-way partial sums of 8 float4s, in a fixed order); zero for b >= 8.
__device__ __forceinline__ uint16_t hbits(float v) { return __half_as_ushort(__float2half_rn(v)); }
__device__ __forceinline__ uint16_t split_part(float v, bool lo) {
    const __half hi = __float2half_rn(v);
    return lo ? hbits(v - __half2float(hi)) : __half_as_ushort(hi);
}

template <class F>
__global__ void __launch_bounds__(256) bgemm_prep(const float *__restrict__ X, int64_t cols, int k, int nsteps,
                                                  uint32_t *__restrict__ xp, uint16_t *__restrict__ xm) {
    const int64_t t = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
    const int64_t nx = int64_t(nsteps) * 1024;
    if (t < nx) {
        // one thread per (step, lane, MFMA): four fp16 parts
        const int m = int(t & 15), lane = int((t >> 4) & 63);
        const int64_t s = t >> 10;
        const int b = lane & 15, g = lane >> 4, n = b & 7;
        const bool lo = b >= 8;
        // the four values are x[e0 + perm4(i)] for a 4-aligned e0 in every
        // format: one 16-byte load (cols is a multiple of 32)
        const int64_t e0 = s * 256 + F::elem(m, g, 0);
        const float4 v = (n < k && e0 < cols) ? *reinterpret_cast<const float4 *>(X + n * cols + e0)
                                              : float4{0.f, 0.f, 0.f, 0.f};
        const float vv[4] = {v.x, v.y, v.z, v.w};
        uint32_t hv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) hv[i] = split_part(vv[perm4(i)], lo);
        // MFMA pair m / 2 of every lane of a step is one contiguous 1 KB run
        const int64_t o = ((s * 8 + (m >> 1)) * 64 + lane) * 4 + (m & 1) * 2;
        xp[o] = hv[0] | (hv[1] << 16);
        xp[o + 1] = hv[2] | (hv[3] << 16);
        return;
    }
    if constexpr (F::kMin) {
        // one thread per (step, lane, K slot) of the min MFMA's A operand
        const int64_t u = t - nx;
        if (u >= int64_t(nsteps) * 256) return;
        const int i = int(u & 3), lane = int((u >> 2) & 63);
        const int64_t s = u >> 8;
        const int b = lane & 15, g = lane >> 4, kk = 4 * g + i, j = kk & 7;
        float sx = 0.f;
        if (b < 8 && b < k) {
            const float4 *p = reinterpret_cast<const float4 *>(X + b * cols + s * 256 + 32 * j);
#pragma unroll
            for (int v = 0; v < 8; ++v) {
                const float4 q = p[v];
                sx += (q.x + q.y) + (q.z + q.w);
            }
        }
        xm[u] = split_part(sx, kk >= 8);
    }
}

template <class F, int kTiles>
__device__ __forceinline__ void load_step(const uint8_t *const (&row)[kTiles], int s, int lane, int g, int nblk,
                                          const uint32_t *__restrict__ xp, const uint32_t *__restrict__ xm,
                                          typename F::Raw (&r)[kTiles], u32x4 (&xr)[8], u32x2 &xmr) {
    const u32x4 *px = reinterpret_cast<const u32x4 *>(xp) + int64_t(s) * 512 + lane;
#pragma unroll
    for (int q = 0; q < 8; ++q) xr[q] = px[64 * q];
    if constexpr (F::kMin) xmr = *reinterpret_cast<const u32x2 *>(xm + (int64_t(s) * 64 + lane) * 2);
#pragma unroll
    for (int t = 0; t < kTiles; ++t) F::load(row[t], s, g, nblk, r[t]);
}

template <class F, int kTiles>
__device__ __forceinline__ void compute_step(const typename F::Raw (&r)[kTiles], const u32x4 (&xr)[8],
                                             const u32x2 &xmr, const uint8_t *const (&row)[kTiles], int s, int g,
                                             int nblk, f4 (&acc)[kTiles]) {
    h4 xa[16];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
        xa[2 * q] = pack(xr[q].x, xr[q].y);
        xa[2 * q + 1] = pack(xr[q].z, xr[q].w);
    }
#pragma unroll
    for (int t = 0; t < kTiles; ++t) {
        if constexpr (std::is_same<F, BQ80>::value || std::is_same<F, BQ40>::value)
            F::compute(r[t], row[t], s, nblk, xa, h4{}, acc[t]);
        else if constexpr (F::kMin) F::compute(r[t], g, xa, pack(xmr.x, xmr.y), acc[t]);
        else F::compute(r[t], row[t], s, g, xa, acc[t]);
    }
}

template <class F, int kTiles>
__global__ void __launch_bounds__(64 * kWaves) bgemm(const uint8_t *__restrict__ W, int64_t row_bytes, int rows,
                                                      int nsteps, int nblk, const uint32_t *__restrict__ xp,
                                                      const uint32_t *__restrict__ xm, float *__restrict__ Y,
                                                      int k, int accumulate, float *__restrict__ partial) {
    __shared__ float part[kWaves][16 * kTiles][8];
    // column split: workgroup row blockIdx.y takes steps [s_lo, s_hi) and,
    // when there are several, writes its sums to partial[blockIdx.y][n][row]
    const int nsplit = gridDim.y;
    const int s_lo = int(int64_t(nsteps) * blockIdx.y / nsplit), s_hi = int(int64_t(nsteps) * (blockIdx.y + 1) / nsplit);
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6, r = lane & 15, g = lane >> 4;
    const int64_t R0 = int64_t(blockIdx.x) * 16 * kTiles + r;
    // rows past the end read row 0 (in bounds); their results are not written
    const uint8_t *row[kTiles];
#pragma unroll
    for (int t = 0; t < kTiles; ++t) row[t] = W + (R0 + 16 * t < rows ? R0 + 16 * t : 0) * row_bytes;
    f4 acc[kTiles];
#pragma unroll
    for (int t = 0; t < kTiles; ++t) acc[t] = f4{0.f, 0.f, 0.f, 0.f};
    if (s_lo + wv < s_hi) {
        // one step ahead, in two register sets used in turn: the loads of the
        // next step are in flight while this one is computed (a step past
        // the end re-loads the current one, from cache)
        typename F::Raw ra[kTiles], rb[kTiles];
        u32x4 xa_[8], xb_[8];
        u32x2 ma = {0u, 0u}, mb = {0u, 0u};
        load_step<F, kTiles>(row, s_lo + wv, lane, g, nblk, xp, xm, ra, xa_, ma);
        for (int s = s_lo + wv; s < s_hi; s += 2 * kWaves) {
            const int s1 = s + kWaves < s_hi ? s + kWaves : s;
            load_step<F, kTiles>(row, s1, lane, g, nblk, xp, xm, rb, xb_, mb);
            // keeps the loads above ahead of the arithmetic (the scheduler
            // would otherwise sink them to their first use)
            asm volatile("" ::: "memory");
            compute_step<F, kTiles>(ra, xa_, ma, row, s, g, nblk, acc);
            if (s + kWaves >= s_hi) break;
            const int s2 = s + 2 * kWaves < s_hi ? s + 2 * kWaves : s1;
            load_step<F, kTiles>(row, s2, lane, g, nblk, xp, xm, ra, xa_, ma);
            asm volatile("" ::: "memory");
            compute_step<F, kTiles>(rb, xb_, mb, row, s1, g, nblk, acc);
        }
    }
    // lanes g and g + 2 hold the hi and lo parts of outputs n = 4g + i
#pragma unroll
    for (int t = 0; t < kTiles; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float o = acc[t][i] + __shfl_down(acc[t][i], 32, 64);
            if (g < 2) part[wv][16 * t + r][4 * g + i] = o;
        }
    __syncthreads();
    for (int j = threadIdx.x; j < 128 * kTiles; j += 64 * kWaves) {
        const int rr = j % (16 * kTiles), n = j / (16 * kTiles);
        const int64_t R2 = int64_t(blockIdx.x) * 16 * kTiles + rr;
        if (n < k && R2 < rows) {
            float v = 0.f;
#pragma unroll
            for (int w = 0; w < kWaves; ++w) v += part[w][rr][n];
            if (nsplit > 1) {
                partial[(int64_t(blockIdx.y) * k + n) * rows + R2] = v;
            } else {
                float *py = Y + n * int64_t(rows) + R2;
                *py = accumulate ? *py + v : v;
            }
        }
    }
}

// Y[n][r] (+)= sum over splits, in split order, of partial[split][n][r].
__global__ void __launch_bounds__(256) bgemm_reduce(const float *__restrict__ partial, int nsplit, int k, int rows,
                                                    float *__restrict__ Y, int accumulate) {
    const int64_t t = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
    if (t >= int64_t(k) * rows) return;
    float v = 0.f;
    for (int sp = 0; sp < nsplit; ++sp) v += partial[int64_t(sp) * k * rows + t];
    Y[t] = accumulate ? Y[t] + v : v;
}

}  // namespace

int64_t bgemm_steps(int64_t cols) { return (cols + 255) / 256; }

bool gemm_batch_type_ok(nt_qtype t) {
    return t == NT_Q8_0 || t == NT_Q4_0 || t == NT_Q4_K || t == NT_Q5_K || t == NT_Q6_K;
}

// fp32 partial sums of a column-split launch: at most 8 vectors x 65536
// (split, row) pairs
constexpr int64_t kPartialFloats = 8 * 65536;

size_t gemm_batch_workspace_bytes(nt_qtype t, int64_t cols) {
    const int64_t ns = bgemm_steps(cols);
    const bool mins = t == NT_Q4_K || t == NT_Q5_K;
    return size_t(ns) * 8192 + (mins ? size_t(ns) * 512 : 0) + size_t(kPartialFloats) * 4;
}

// Column splits for a matrix whose row groups alone give fewer than 256
// workgroups: about 512 workgroups in all, at least one step per wave, and
// within the partial-sum area.
// (Splitting 8192-row matrices as well, to 1024 workgroups, made them slower:
// Q4_K 8192x8192 at k = 8 25 -> 34 us.)
int bgemm_splits(int64_t groups, int ns, int64_t rows) {
    if (groups >= 256) return 1;
    int64_t sp = (512 + groups - 1) / groups;
    sp = std::min<int64_t>(sp, std::max(1, ns / kWaves));
    sp = std::min<int64_t>(sp, 65536 / std::max<int64_t>(rows, 1));
    return int(std::max<int64_t>(sp, 1));
}

template <class F>
hipError_t run_bgemm(const void *W, int64_t row_bytes, int64_t rows, int64_t cols, int64_t nblk, const float *X,
                     int k, float *Y, int accumulate, void *ws, hipStream_t st) {
    const int ns = int(bgemm_steps(cols));
    uint32_t *xp = static_cast<uint32_t *>(ws);
    uint32_t *xm = F::kMin ? xp + int64_t(ns) * 2048 : nullptr;
    float *partial = reinterpret_cast<float *>(static_cast<uint8_t *>(ws) + int64_t(ns) * 8192 +
                                               (F::kMin ? int64_t(ns) * 512 : 0));
    const int64_t nt = int64_t(ns) * (F::kMin ? 1024 + 256 : 1024);
    hipLaunchKernelGGL(bgemm_prep<F>, dim3(unsigned((nt + 255) / 256)), dim3(256), 0, st, X, cols, k, ns, xp,
                       reinterpret_cast<uint16_t *>(xm));
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || rows == 0) return e;
    if constexpr (std::is_same<F, BQ4K>::value) {
        if (rows >= kTallRows) {
            hipLaunchKernelGGL((bgemm<F, 4>), dim3(unsigned((rows + 63) / 64)), dim3(64 * kWaves), 0, st,
                               static_cast<const uint8_t *>(W), row_bytes, int(rows), ns, int(nblk), xp, xm, Y, k,
                               accumulate, partial);
            return hipGetLastError();
        }
    }
    const int64_t groups = (rows + 31) / 32;
    const int sp = bgemm_splits(groups, ns, rows);
    hipLaunchKernelGGL((bgemm<F, 2>), dim3(unsigned(groups), unsigned(sp)), dim3(64 * kWaves), 0, st,
                       static_cast<const uint8_t *>(W), row_bytes, int(rows), ns, int(nblk), xp, xm, Y, k, accumulate,
                       partial);
    if (sp == 1) return hipGetLastError();
    if ((e = hipGetLastError()) != hipSuccess) return e;
    const int64_t nt2 = int64_t(k) * rows;
    hipLaunchKernelGGL(bgemm_reduce, dim3(unsigned((nt2 + 255) / 256)), dim3(256), 0, st, partial, sp, k, int(rows),
                       Y, accumulate);
    return hipGetLastError();
}

hipError_t launch_gemm_batch(nt_qtype t, const void *W, int64_t rows, int64_t cols, const float *X, int k, float *Y,
                             int accumulate, void *ws, hipStream_t st) {
    const int64_t nblk = cols / block_elems(t), row_bytes = nblk * block_bytes(t);
    switch (t) {
    case NT_Q8_0: return run_bgemm<BQ80>(W, row_bytes, rows, cols, nblk, X, k, Y, accumulate, ws, st);
    case NT_Q4_0: return run_bgemm<BQ40>(W, row_bytes, rows, cols, nblk, X, k, Y, accumulate, ws, st);
    case NT_Q5_K: return run_bgemm<BQ5K>(W, row_bytes, rows, cols, nblk, X, k, Y, accumulate, ws, st);
    case NT_Q4_K: return run_bgemm<BQ4K>(W, row_bytes, rows, cols, nblk, X, k, Y, accumulate, ws, st);
    case NT_Q6_K: return run_bgemm<BQ6K>(W, row_bytes, rows, cols, nblk, X, k, Y, accumulate, ws, st);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace nt
