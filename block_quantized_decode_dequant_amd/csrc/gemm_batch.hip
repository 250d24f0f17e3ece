// gemm_batch.hip -- y_n = W x_n (+ y_n) for k <= 8 activation vectors against
// one block-quantized matrix: the verify pass of self-speculative decoding.
//
// The ntransformer write-up ("Overview", self-speculative decoding) has the
// VRAM-resident layers draft several tokens that the whole model then checks
// in one pass, so the matrices are read once for k tokens instead of k times.
// At k = 8 the arithmetic is 16 flops per weight; Q4_K at HBM speed would
// need about 230 TFLOP/s of fp32 FMA, above the vector units' peak, so the
// products run on the matrix cores (v_mfma_f32_16x16x16_f16, and
// v_mfma_f32_16x16x32_f16 for Q4_K):
//
//  * the MFMA's M dimension holds the activations, N the 16 weight rows of a
//    tile, K 16 codes of one scale group (Q8_0, Q4_0, Q6_K) or the 32 codes
//    of one Q4_K sub-block, whose scale is applied to the MFMA's fp32 sums,
//    or any 16 codes of a Q5_K super-block, whose 6-bit scales are folded
//    into the codes.  With N = weight row, every lane applies the scales of
//    its own row to its own accumulators.
//  * weight codes become fp16 exactly: small integers (q, q - 8, q - 32),
//    Q4_K nibbles masked in place (the subnormals q 2^-24 and 16 q 2^-24,
//    which the matrix cores multiply exactly), or S_j q 2^-14 (Q5_K).
//    Nothing about the weights is rounded.
//  * each activation is split into fp16 hi + lo (hi = fp16(x), lo =
//    fp16(x - hi)), which leaves about 2^-22 relative error; the hi parts fill
//    M rows 0-7 and the lo parts rows 8-15, which the padding of k <= 8 to 16
//    would otherwise waste.  Products are exact in fp32; the MFMA sums in fp32.
//    Activations large enough for a part or a 32-value sum to overflow fp16
//    are split scaled by a power of two per 256 columns, undone in fp32.
//  * a first kernel writes each 256-column step's split activations once
//    (an "activation record") in the order the lanes consume them, so every
//    row tile reads them with eight 1 KB contiguous loads.
//  * the weights move through LDS: each wave copies its tiles' row runs with
//    global_load_lds (whole contiguous runs of a row per instruction; loads
//    that put 16 rows' bytes into one instruction's lanes, as the MFMA layout
//    would, reach far less of HBM's bandwidth) and reads its MFMA operands
//    from LDS.
//  * MFMA lane layout (16x16x16 f16): src0 lane l holds A[l % 16][4(l/16) + i],
//    src1 lane l holds B[4(l/16) + i][l % 16], the result lane l holds
//    D[4(l/16) + i][l % 16], i = 0..3 (16x16x32: eight K slots per lane, the
//    same result layout).  Inside one MFMA the order of the K slots is free
//    as long as A and B agree, so each lane takes the codes of its row that
//    lie together in memory.
//  * one workgroup of eight waves per CU; the waves of a workgroup split the
//    rows and, where that leaves too few workgroups, the columns, whose sums
//    meet in LDS at the end.  Where all eight waves work on one column range
//    (and LDS allows: the one-tile K-quants), they share each step's
//    activation record through a ring in LDS instead of each loading it.
#include <algorithm>
#include <atomic>
#include <type_traits>

#include "device_util.h"
#include "nt_internal.h"

namespace nt {
namespace {

typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef uint32_t w2 __attribute__((ext_vector_type(2)));
typedef float f2 __attribute__((ext_vector_type(2)));

constexpr int kNumCUs = 256;   // compute units of an MI355X
// The workspace starts with the counters of the column splits between
// workgroups (one per wave's rows of a workgroup column), zero between calls.
constexpr int kMaxTickets = 4096;
constexpr size_t kTicketBytes = 4 * kMaxTickets;

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

// 16x16x32 f16: src lane l holds 8 K slots of row / column l % 16 (the same
// slots for A and B), the result the same layout as 16x16x16.
typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4n __attribute__((ext_vector_type(4)));   // natural (16-byte) alignment
typedef uint32_t u32x2n __attribute__((ext_vector_type(2)));   // 8-byte alignment
__device__ __forceinline__ f4 mfma32(h8 a, h8 b, f4 c) { return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0); }
__device__ __forceinline__ h8 cat(h4 a, h4 b) { return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7); }
__device__ __forceinline__ h8 h8bits(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
    return __builtin_bit_cast(h8, u32x4n{a, b, c, d});
}
__device__ __forceinline__ float ubyte(uint32_t w, int k) { return float((w >> (8 * k)) & 0xffu); }

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
    static constexpr int kStepBytes = 272, kTiles = 1;
    // 114 KB of weight rings leave room for five record slots; a Q8_0 step
    // reads its own records cheaply, so forming them costs slightly more
    // (measured at k = 8: 14336 x 4096 25.8 -> 22.1 us shared, 4096 x 14336
    // 25.5 -> 21.1, 128256 x 4096 164-168 -> 170, 4096 x 4096 12.5 either way)
    static constexpr int kRingSlots = 5, kRingAhead = 3, kRingReport = 2, kShareCost = 21;
    struct Raw { u32x3 v[8]; };
    __host__ __device__ static int elem(int m, int g, int i) { return 32 * (m >> 1) + 8 * g + 4 * (m & 1) + perm4(i); }
    __host__ __device__ static void blk(int jb, int e, int &m, int &g, int &o) {   // as for BQ4K
        m = 2 * jb + (e & 1);
        g = e >> 1;
        o = 8 * g + 4 * (e & 1);
    }
    __device__ static void load(const uint8_t *p, int s, int g, int nblk, Raw &r) {
#pragma unroll
        for (int bb = 0; bb < 8; ++bb) {
            const uint8_t *b = p + (8 * s + bb < nblk ? bb : 0) * 34;
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
    __device__ static void compute(const Raw &r, const uint8_t *p, int s, int, int nblk, const h4 *xa, h4, f4 &acc) {
        const int src = int(__lane_id() & 15);          // lane group 0 of this row
        const uint32_t sel2 = shift_sel(2);
#pragma unroll
        for (int bb = 0; bb < 8; ++bb) {
            const bool live = 8 * s + bb < nblk;
            const uint8_t *b = p + (live ? bb : 0) * 34;
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

// ---- Q4_K: a step is one super-block.  One 16x16x32 MFMA per sub-block j
// (32 values sharing a 6-bit scale S_j and min M_j): lane group g takes code
// bytes [8g, 8g + 8) of chunk j / 2 (low nibbles for even j, high for odd),
// value 32 j + 8 g + 4 (m % 2) + perm4(i) for record slot m = 2j + m % 2.  A
// nibble masked in place is an fp16 subnormal, q 2^-24 (low) or 16 q 2^-24
// (high), which the matrix cores take exactly; S_j then scales the MFMA's
// fp32 sums, so the codes need no arithmetic beyond their masks.  The mins
// go through one more MFMA: A = per-sub-block activation sums (hi in K slots
// 0-7, lo in 8-15), B = M_j, also as subnormals.  Rows of 144-byte blocks
// keep every step start 16-byte aligned.
struct BQ4K {
    static constexpr bool kMin = true;
    static constexpr int kStepBytes = 144, kTiles = 1;   // one tile: LDS room for the record ring
    static constexpr bool kAligned = true;                // 144-byte blocks
    // wide form: sixteen waves (four per SIMD), three ring stages (108 KB), five record slots
    static constexpr int kWideWaves = 16, kWideStages = 3;
    static constexpr int kWideRingSlots = 5, kWideRingAhead = 3, kWideRingReport = 2, kWideCost = 27;
    struct Raw { u32x4n h; u32x2n q[4]; };
    __host__ __device__ static int elem(int m, int g, int i) { return 32 * (m >> 1) + 8 * g + 4 * (m & 1) + perm4(i); }
    // the eight (m, g) whose values lie in the step's 32-column block jb:
    // entry e gives m, g and the offset o in the block (elem(m, g, i) = 32
    // jb + o + perm4(i))
    __host__ __device__ static void blk(int jb, int e, int &m, int &g, int &o) {
        m = 2 * jb + (e & 1);
        g = e >> 1;
        o = 8 * g + 4 * (e & 1);
    }
    __device__ static void load(const uint8_t *b, int, int g, int, Raw &r) {
        const uint8_t *const a = static_cast<const uint8_t *>(__builtin_assume_aligned(b, 16));
        r.h = *reinterpret_cast<const u32x4n *>(a);
#pragma unroll
        for (int c = 0; c < 4; ++c) r.q[c] = *reinterpret_cast<const u32x2n *>(a + 16 + 32 * c + 8 * g);
    }
    // 6-bit scale S_j and min M_j of sub-block j from the 12 scale bytes
    // (words h.y, h.z, h.w): j < 4: low 6 bits of bytes j and j + 4; j >= 4:
    // low / high nibble of byte j + 4 with the top two bits of byte j - 4 / j.
    // As bytes: S_0..3 = h.y & 0x3f.., S_4..7 = (h.w & 0x0f..) | (h.y >> 2 &
    // 0x30..), M_0..3 = h.z & 0x3f.., M_4..7 = (h.w >> 4 & 0x0f..) | (h.z >> 2
    // & 0x30..).
    __device__ static void compute(const Raw &r, const uint8_t *, int, int g, int, const h4 *xa, h4 xm, f4 &acc) {
        const uint32_t s03 = r.h.y & 0x3f3f3f3fu;
        const uint32_t s47 = (r.h.w & 0x0f0f0f0fu) | ((r.h.y >> 2) & 0x30303030u);
        f4 lo = {0.f, 0.f, 0.f, 0.f}, hi = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const uint32_t w0 = r.q[c].x, w1 = r.q[c].y, t0 = w0 >> 8, t1 = w1 >> 8;
            const uint32_t sw = c < 2 ? s03 : s47;
            const f4 cl = mfma32(cat(xa[4 * c], xa[4 * c + 1]),
                                 h8bits(w0 & 0x000f000fu, t0 & 0x000f000fu, w1 & 0x000f000fu, t1 & 0x000f000fu),
                                 f4{0.f, 0.f, 0.f, 0.f});
            const f4 ch = mfma32(cat(xa[4 * c + 2], xa[4 * c + 3]),
                                 h8bits(w0 & 0x00f000f0u, t0 & 0x00f000f0u, w1 & 0x00f000f0u, t1 & 0x00f000f0u),
                                 f4{0.f, 0.f, 0.f, 0.f});
            lo += ubyte(sw, 2 * (c & 1)) * cl;
            hi += ubyte(sw, 2 * (c & 1) + 1) * ch;
        }
        // B of the min MFMA: K slot 4g + i takes M_{(4g + i) & 7}, i.e. M_i for
        // even g and M_{4+i} for odd g, each byte widened to a subnormal half
        const uint32_t mw = (g & 1) ? ((r.h.w >> 4) & 0x0f0f0f0fu) | ((r.h.z >> 2) & 0x30303030u)
                                    : r.h.z & 0x3f3f3f3fu;
        const f4 cm = mfma(xm, pack(__builtin_amdgcn_perm(0u, mw, 0x0c010c00u), __builtin_amdgcn_perm(0u, mw, 0x0c030c02u)),
                           f4{0.f, 0.f, 0.f, 0.f});
        const float d = h2f(r.h.x) * 16777216.f, dmin = h2f(r.h.x >> 16) * 16777216.f;
        // as two multiply-adds onto acc (acc - dmin cm first): a separate
        // "acc +" would cost an add per output even with acc = 0
        acc = d * (lo + 0.0625f * hi) + (acc - dmin * cm);
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
    static constexpr int kStepBytes = 144, kTiles = 2;
    struct Raw { u32x2 v[8]; };
    __host__ __device__ static int elem(int m, int g, int i) { return 32 * (m >> 1) + 16 * (m & 1) + 4 * g + perm4(i); }
    __device__ static void load(const uint8_t *p, int s, int g, int nblk, Raw &r) {
#pragma unroll
        for (int bb = 0; bb < 8; ++bb) {
            const uint8_t *b = p + (8 * s + bb < nblk ? bb : 0) * 18;
            const uint32_t bs = uint32_t(reinterpret_cast<uintptr_t>(b) & 3);   // 0 or 2
            r.v[bb] = *reinterpret_cast<const u32x2 *>(b - bs + 4 * g);
        }
    }
    __device__ static h4 nib(uint32_t w) {   // bits 0-3 of each byte: q - 8 as fp16, bytes 0,2 then 1,3
        const uint32_t a = hadd((w & 0x000f000fu) | 0x64006400u, _Float16(-1032.f));
        const uint32_t b = hadd(((w >> 8) & 0x000f000fu) | 0x64006400u, _Float16(-1032.f));
        return pack(a, b);
    }
    __device__ static void compute(const Raw &r, const uint8_t *p, int s, int, int nblk, const h4 *xa, h4, f4 &acc) {
        const int src = int(__lane_id() & 15);          // lane group 0 of this row
        const uint32_t sel2 = shift_sel(2);
#pragma unroll
        for (int bb = 0; bb < 8; ++bb) {
            const bool live = 8 * s + bb < nblk;
            const uint8_t *b = p + (live ? bb : 0) * 18;
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

// ---- Q5_K: scales folded into the codes: (q * 2^-24 as an fp16
// subnormal) * fp16(S * 2^10) = S q 2^-14 exactly, so one MFMA chain
// covers the whole super-block and any value may sit in any K slot; one more
// MFMA for the mins (as Q4_K).  The fifth bit of value 32j + l is bit j of
// qh[l].  A lane's code bytes c all have c % 32 in
// [16 (g % 2), 16 (g % 2) + 16), so one 16-byte piece of qh serves them.
// S q <= 63 * 31 = 1953 keeps S q 2^-14 exact in fp16.
struct BQ5K {
    static constexpr bool kMin = true;
    static constexpr int kStepBytes = 176, kTiles = 1;
    static constexpr bool kAligned = true;                // 176-byte blocks
    // wide form: sixteen waves, two ring stages (88 KB), seven record slots
    static constexpr int kWideWaves = 16, kWideStages = 2;
    static constexpr int kWideRingSlots = 7, kWideRingAhead = 4, kWideRingReport = 3, kWideCost = 29;
    struct Raw { u32x4 h, qh, q0, q1; };
    // lane group g takes code bytes [16g, 16g + 16) and [64 + 16g, 64 + 16g +
    // 16); MFMA m uses word m / 2 of those eight (low nibbles for even m, high
    // for odd); code byte c holds values 64 (c / 32) + c % 32 (low) and 32
    // more (high)
    __host__ __device__ static int code_byte(int w, int g) { return w < 4 ? 16 * g + 4 * w : 64 + 16 * g + 4 * (w - 4); }
    __host__ __device__ static int elem(int m, int g, int i) {
        const int c = code_byte(m >> 1, g) + perm4(i);
        return 32 * (2 * (c >> 5) + (m & 1)) + (c & 31);
    }
    __host__ __device__ static void blk(int jb, int e, int &m, int &g, int &o) {   // as for BQ4K
        m = 2 * (4 * (jb >> 2) + (e & 3)) + (jb & 1);
        g = 2 * ((jb >> 1) & 1) + (e >> 2);
        o = 16 * (e >> 2) + 4 * (e & 3);
    }
    // 6-bit scale S_j and min M_j of sub-block j from the 12 scale bytes
    // (words h.y, h.z, h.w): j < 4: low 6 bits of bytes j and j + 4; j >= 4:
    // low / high nibble of byte j + 4 with the top two bits of byte j - 4 / j.
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
    __device__ static void load(const uint8_t *b, int, int g, int, Raw &r) {
        r.h = ld4(b);
        r.qh = ld4(b + 16 + 16 * (g & 1));
        r.q0 = ld4(b + 48 + 16 * g);
        r.q1 = ld4(b + 112 + 16 * g);
    }
    __device__ static void compute(const Raw &r, const uint8_t *, int, int g, int, const h4 *xa, h4 xm, f4 &acc) {
        uint32_t S[8], M[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) scale_min(r.h, j, S[j], M[j]);
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
        acc = d * c + (acc - dmin * cm);   // two multiply-adds onto acc
    }
};

// ---- Q6_K: a step is one super-block (210 bytes, so only 2-byte aligned).
// Value (h, k, l) = 128h + 32k + l has code q = ql4 + 16 qh2 (ql4: nibble
// k / 2 of ql[64h + 32 (k % 2) + l], qh2: bits 2k, 2k + 1 of qh[32h + l]) and
// scale scales[8h + 2k + l / 16].  MFMA m covers scale group m = 8h + 2k +
// l / 16 (its 16 values share a scale): lane group g takes l = 16 (m % 2) +
// 4g + perm4(i), i.e. four consecutive ql bytes and four consecutive qh
// bytes, one word of each.  The six-bit codes become q - 32 exactly in fp16
// (a byte permute sets the exponent byte 0x64, one packed subtraction), the
// MFMA sums one group, and the group's d * scale is applied in fp32.  Every
// word is two aligned reads and a funnel.
struct BQ6K {
    static constexpr bool kMin = false;
    static constexpr int kStepBytes = 210, kTiles = 1;
    // wide form: sixteen waves, two ring stages (120 KB), four record slots
    static constexpr int kWideWaves = 16, kWideStages = 2;
    static constexpr int kWideRingSlots = 4, kWideRingAhead = 3, kWideRingReport = 2, kWideCost = 29;
    // word pairs at byte offsets 4g + 16j (ql, j < 8), 128 + 4g + 16j (qh,
    // j < 4) from the word-aligned block start; scale words 192..208 (the
    // last also holds d)
    struct Raw { uint32_t ql[8][2], qh[4][2], sc[5]; };
    __host__ __device__ static int elem(int m, int g, int i) {
        return 128 * (m >> 3) + 32 * ((m >> 1) & 3) + 16 * (m & 1) + 4 * g + perm4(i);
    }
    __host__ __device__ static void blk(int jb, int e, int &m, int &g, int &o) {   // as for BQ4K
        m = 8 * (jb >> 2) + 2 * (jb & 3) + (e & 1);
        g = e >> 1;
        o = 16 * (e & 1) + 4 * g;
    }
    __device__ static void load(const uint8_t *b, int, int g, int, Raw &r) {
        const uint8_t *a = b - (reinterpret_cast<uintptr_t>(b) & 2);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            r.ql[j][0] = ld1(a + 4 * g + 16 * j);
            r.ql[j][1] = ld1(a + 4 * g + 16 * j + 4);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            r.qh[j][0] = ld1(a + 128 + 4 * g + 16 * j);
            r.qh[j][1] = ld1(a + 128 + 4 * g + 16 * j + 4);
        }
#pragma unroll
        for (int j = 0; j < 5; ++j) r.sc[j] = ld1(a + 192 + 4 * j);
    }
    __device__ static void compute(const Raw &r, const uint8_t *b, int, int, int, const h4 *xa, h4, f4 &acc) {
        const uint32_t sh = uint32_t(reinterpret_cast<uintptr_t>(b) & 2);
        const uint32_t sel = shift_sel(sh);
        uint32_t ql[8], qh[4], sc[4];
#pragma unroll
        for (int j = 0; j < 8; ++j) ql[j] = funnel(r.ql[j][1], r.ql[j][0], sel);
#pragma unroll
        for (int j = 0; j < 4; ++j) qh[j] = funnel(r.qh[j][1], r.qh[j][0], sel);
#pragma unroll
        for (int j = 0; j < 4; ++j) sc[j] = funnel(r.sc[j + 1], r.sc[j], sel);
        const float d = h2f(sh ? r.sc[4] >> 16 : r.sc[4]);
#pragma unroll
        for (int m = 0; m < 16; ++m) {
            const int h = m >> 3, k = (m >> 1) & 3, lg = m & 1;
            const uint32_t w = ql[4 * h + 2 * (k & 1) + lg];
            const uint32_t ql4 = ((k >> 1) ? w >> 4 : w) & 0x0f0f0f0fu;
            const uint32_t q6 = ql4 | (((qh[2 * h + lg] >> (2 * k)) & 0x03030303u) << 4);
            // fp16 1024 + q for bytes 0, 2 and 1, 3; minus 1056 gives q - 32
            const uint32_t p0 = hadd(__builtin_amdgcn_perm(0x64646464u, q6, 0x04020400u), _Float16(-1056.f));
            const uint32_t p1 = hadd(__builtin_amdgcn_perm(0x64646464u, q6, 0x04030401u), _Float16(-1056.f));
            const f4 c = mfma(xa[m], pack(p0, p1), f4{0.f, 0.f, 0.f, 0.f});
            const float ds = d * float(int8_t((sc[m >> 2] >> (8 * (m & 3))) & 0xffu));
            acc += ds * c;
        }
    }
};

__device__ __forceinline__ uint16_t hbits(float v) { return __half_as_ushort(__float2half_rn(v)); }
__device__ __forceinline__ uint16_t split_part(float v, bool lo) {
    const __half hi = __float2half_rn(v);
    return lo ? hbits(v - __half2float(hi)) : __half_as_ushort(hi);
}

typedef uint32_t u32x4a __attribute__((ext_vector_type(4)));   // 16-byte aligned

// Geometry of one format's pipeline.  Each wave streams T 16-row tiles
// through its own ring of S LDS stages, one 256-column step per stage.  A
// tile row is the Lc bytes from the 16-byte granule that holds the row's
// step start: they cover the L bytes of the step whatever its offset in the
// granule, and each copy instruction moves 64 whole granules (1 KB).  Rows
// sit Lp bytes apart in LDS, an odd number of granules, so the 16 lanes that
// read one offset of 16 rows hit distinct banks; a tile takes NI copy
// instructions, the lanes past the 16 rows left out of the last one, so a
// tile takes exactly 16 Lp bytes, and the lanes of a row's padding granule
// (Lp > Lc) copy nothing.  Where every step starts 16-byte aligned
// (kAligned) a row is just the L bytes of the step.
// Launch forms of the main kernel: 0 = per-wave records (from the record
// kernel), 1 = shared records formed in LDS, eight waves (two per SIMD) and
// three weight-ring stages, 2 = shared records with the wide pipeline a
// format may set (kWideWaves waves, kWideStages stages, its own record ring:
// more waves per SIMD hide more latency on long column ranges).
constexpr int kOwn = 0, kShared = 1, kWide = 2;

// Record ring of a shared-record form: slots, how many steps ahead a step's
// activations are copied and its record formed, and the launch-shape cost of
// one of its steps in twentieths of a per-wave-record step (a format may set
// its own with kRingSlots, kRingAhead, kRingReport, kShareCost; the wide
// form with kWideRingSlots, kWideRingAhead, kWideRingReport, kWideCost).
template <class F, int FORM, class = void>
struct RingOf {
    static constexpr int slots = 7, ahead = 4, report = 3, cost = 16;
};
template <class F>
struct RingOf<F, kShared, std::void_t<decltype(F::kRingSlots)>> {
    static constexpr int slots = F::kRingSlots, ahead = F::kRingAhead, report = F::kRingReport, cost = F::kShareCost;
};
template <class F>
struct RingOf<F, kWide, std::void_t<decltype(F::kWideRingSlots)>> {
    static constexpr int slots = F::kWideRingSlots, ahead = F::kWideRingAhead, report = F::kWideRingReport,
                         cost = F::kWideCost;
};

// Formats whose 256-column steps all start 16-byte aligned (blocks a
// multiple of 16 bytes) copy exactly their tile rows (kAligned).
template <class F, class = void>
struct AlignedOf {
    static constexpr bool value = false;
};
template <class F>
struct AlignedOf<F, std::void_t<decltype(F::kAligned)>> {
    static constexpr bool value = F::kAligned;
};

// Waves per workgroup and weight-ring stages of a launch form.
template <class F, int FORM, class = void>
struct PipeOf {
    static constexpr int waves = 8, stages = 3;
    static constexpr bool exists = FORM != kWide;
};
template <class F>
struct PipeOf<F, kWide, std::void_t<decltype(F::kWideWaves)>> {
    static constexpr int waves = F::kWideWaves, stages = F::kWideStages;
    static constexpr bool exists = true;
};

template <class F, int FORM = kOwn>
struct Geo {
    static constexpr int T = F::kTiles;
    static constexpr int S = PipeOf<F, FORM>::stages;            // ring stages: S - 1 steps copied ahead
    static constexpr int NW = PipeOf<F, FORM>::waves;            // waves per workgroup
    static_assert(NW % 4 == 0 && NW <= 16 && (S == 2 || S == 3), "launch form");
    static constexpr int L = F::kStepBytes;
    static constexpr bool AL = AlignedOf<F>::value;              // every step starts 16-byte aligned
    // granules that cover a step: blocks are 2-byte aligned, so a step
    // starts at most 14 bytes into its first granule
    static constexpr int Lc = AL ? L : (L + 14 + 15) / 16 * 16;
    static constexpr int Lp = ((Lc / 16) & 1) ? Lc : Lc + 16;
    static constexpr int NI = (16 * Lp + 1023) / 1024;           // copy instructions per tile
    static constexpr int TB = 16 * Lp;                           // LDS bytes of one tile
    static constexpr int LAST = (TB - 1024 * (NI - 1)) / 16;     // lanes of the last copy
    static constexpr int WAVE = S * T * TB;                      // LDS bytes of one wave's ring
    static constexpr int LDS = NW * WAVE;
    static constexpr int REC = 8192 + (F::kMin ? 512 : 0) + 32;  // activation record of one step
    static_assert(LDS <= 160 * 1024, "LDS of one workgroup per CU");
    // shared records (all waves of a workgroup on one column range): a ring of
    // R record slots after the weight rings, then 2R step counters.  Step j's
    // activations are copied KA steps ahead and its record formed KR steps
    // ahead (fits for Q8_0 with four slots, Q4_K one-tile, Q5_K and Q6_K with
    // seven)
    static constexpr int KA = RingOf<F, FORM>::ahead, KR = RingOf<F, FORM>::report;
    static constexpr int R = RingOf<F, FORM>::slots;
    static_assert(R > KA && KA > KR && KR >= 0 && 2 * R <= 16, "record ring");
    static constexpr int RING_REC = LDS;                         // offset of the record ring
    static constexpr int CNT = LDS + R * REC;                    // offset of the counters
    static constexpr int LDS_SH = CNT + 64;
    // this shared-record form exists for the format (its rings fit in LDS)
    static constexpr bool kShare = FORM != kOwn && PipeOf<F, FORM>::exists && LDS_SH <= 160 * 1024;
};

// Activation records, one workgroup per 256-column step s.  Record layout
// (bytes): [0, 8192) the split activations in the order the lanes consume
// them: u32x2 at ((m / 2) * 64 + lane) * 16 + (m % 2) * 8 holds, as two
// fp16 pairs, the hi (lane % 16 < 8) or lo part of s_n x_n[256 s +
// elem(m, g, perm4(i))], n = lane % 8, g = lane / 16 (zero for n >= k or
// past cols); K-quants then [8192, 8704): uint16 at (lane * 4 + i) * 2, K
// slot 4g + i of the min MFMA: hi (slots 0-7) or lo part of the fp32 sum of
// s_b x_b over sub-block (4g + i) % 8, b = lane % 16 (zero for b >= 8); the
// last 32 bytes: 1 / s_n for n = 0..7.  s_n = 2^-e_n is the largest power
// of two scale (at most 1) that keeps 32 max |x_n| over the step below
// 2^14, so no fp16 part and no sub-block sum overflows: an exact scaling
// that the main kernel undoes on the step's fp32 sums.
template <class F>
__global__ void __launch_bounds__(256) bgemm_prep(const float *__restrict__ X, int64_t cols, int k,
                                                  uint8_t *__restrict__ rec) {
    using G = Geo<F>;
    __shared__ __attribute__((aligned(16))) float xs[8][260];
    const int s = blockIdx.x, t = threadIdx.x;
    uint8_t *const out = rec + int64_t(s) * G::REC;
    {
        const int n = t >> 5, c = 8 * (t & 31);
        const int64_t col = int64_t(s) * 256 + c;   // cols is a multiple of 32: all 8 columns or none
        float4 a = {0.f, 0.f, 0.f, 0.f}, b = {0.f, 0.f, 0.f, 0.f};
        if (n < k && col < cols) {
            const float4 *px = reinterpret_cast<const float4 *>(X + n * cols + col);
            a = px[0];
            b = px[1];
        }
        float mx = fmaxf(fmaxf(fmaxf(fabsf(a.x), fabsf(a.y)), fmaxf(fabsf(a.z), fabsf(a.w))),
                         fmaxf(fmaxf(fabsf(b.x), fabsf(b.y)), fmaxf(fabsf(b.z), fabsf(b.w))));
#pragma unroll
        for (int o = 16; o >= 1; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 32));
        int e2 = 0;
        (void)frexpf(fminf(mx, 1.0e36f) * 32.f, &e2);   // 32 max = f 2^e2, f in [0.5, 1)
        const int e = min(max(e2 - 14, 0), 120);
        const float sd = ldexpf(1.f, -e);
        float *row = &xs[n][c];
        row[0] = a.x * sd; row[1] = a.y * sd; row[2] = a.z * sd; row[3] = a.w * sd;
        row[4] = b.x * sd; row[5] = b.y * sd; row[6] = b.z * sd; row[7] = b.w * sd;
        if ((t & 31) == 0) reinterpret_cast<float *>(out + G::REC - 32)[n] = ldexpf(1.f, e);
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int it = t + 256 * u;                  // output u32x2 index: consecutive threads, consecutive bytes
        const int mo = it & 1, lane = (it >> 1) & 63, m = 2 * (it >> 7) + mo;
        const int b = lane & 15, g = lane >> 4;
        const float4 q = *reinterpret_cast<const float4 *>(&xs[b & 7][F::elem(m, g, 0)]);
        const float vv[4] = {q.x, q.y, q.z, q.w};
        uint32_t hv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) hv[i] = split_part(vv[perm4(i)], b >= 8);
        reinterpret_cast<u32x2 *>(out)[it] = u32x2{hv[0] | (hv[1] << 16), hv[2] | (hv[3] << 16)};
    }
    if constexpr (F::kMin) {
        const int i = t & 3, lane = t >> 2, b = lane & 15, kk = 4 * (lane >> 4) + i, j = kk & 7;
        float sx = 0.f;
        if (b < 8) {
#pragma unroll
            for (int v = 0; v < 8; ++v) {
                const float4 q = *reinterpret_cast<const float4 *>(&xs[b][32 * j + 4 * v]);
                sx += (q.x + q.y) + (q.z + q.w);
            }
        }
        reinterpret_cast<uint16_t *>(out + 8192)[t] = split_part(sx, kk >= 8);
    }
}

template <int N>
__device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N <= 63, "vmcnt holds 0..63");
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(N));
    __builtin_amdgcn_sched_barrier(0);
}
// wait until at most N (when more) or no vector-memory operations are outstanding
template <int N>
__device__ __forceinline__ void wait_vm_or_all(bool more) {
    if (more) wait_vm<N>(); else wait_vm<0>();
}

// Step counters of the shared record ring, in LDS: plain workgroup-scope
// atomics (no implied waits: the copies they report on were waited for
// explicitly), added by lane 0 of a wave.  A wait polls with a sleep
// between reads and gives up after about 2^20 polls (far beyond any real
// wait), so every wave always ends.
__device__ __forceinline__ void lds_count(uint32_t *p, uint32_t v = 1u) {
    if (__lane_id() == 0) __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}
__device__ __forceinline__ uint32_t lds_read_count(const uint32_t *p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}
// seen: a value of *p read earlier (counts only grow), so a wait whose
// target was already reached then costs no further read
__device__ __forceinline__ void lds_wait_count(uint32_t *p, uint32_t target, uint32_t seen = 0) {
    if (seen < target) {
        for (int spin = 0; spin < (1 << 20); ++spin) {
            if (lds_read_count(p) >= target) break;
            __builtin_amdgcn_s_sleep(1);
        }
    }
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("" ::: "memory");
}

// One step's activations in registers: the 16 MFMA A operands (from the
// record's split activations), the min MFMA's A operand, and 1 / s_n for
// the four outputs of this lane.
struct XRegs {
    u32x4a x[8];
    u32x2 m;
    f4 up;
};

template <class F>
__device__ __forceinline__ void load_x(const uint8_t *__restrict__ rec, int s, int lane, int g, XRegs &xr) {
    const uint8_t *const rc = rec + int64_t(s) * Geo<F>::REC;
#pragma unroll
    for (int q = 0; q < 8; ++q) xr.x[q] = *reinterpret_cast<const u32x4a *>(rc + (q * 64 + lane) * 16);
    if constexpr (F::kMin) xr.m = *reinterpret_cast<const u32x2 *>(rc + 8192 + lane * 8);
    xr.up = *reinterpret_cast<const f4 *>(rc + Geo<F>::REC - 32 + 16 * (g & 1));
}

// One wave forms the activation record of a step in LDS (the record
// bgemm_prep writes, bit for bit but for the sign of zeros that stand for
// vectors past k and columns past the end) from the step's fp32
// activations, copied into the same slot (vector n's 1 KB at 1024 n, its
// 16-byte chunk c at chunk position c ^ n, so the eight lanes of a read
// group hit distinct banks).  Lane l takes vector n = l mod 8 and the 32
// columns of block jb = l / 8 (columns col0 + 32 jb ...): the vector's
// maximum over the step comes from the eight lanes that hold it, then the
// lane scales its values, splits them into fp16 hi and lo parts and writes
// the eight (m, g) entries of its block (and, with mins, its sub-block
// sum).  All reads of the slot are issued before the first write (the
// writes depend on the maximum).
template <class F>
__device__ __forceinline__ void form_record(uint8_t *slot, int lane, int64_t col0, int k, int64_t cols) {
    const int n = lane & 7, jb = lane >> 3;
    float v[32];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
        const f4 x = *reinterpret_cast<const f4 *>(slot + 1024 * n + 16 * ((8 * jb + q) ^ n));
        v[4 * q] = x.x;
        v[4 * q + 1] = x.y;
        v[4 * q + 2] = x.z;
        v[4 * q + 3] = x.w;
    }
    // a vector past k or a block past the last column (cols is a multiple
    // of 32) holds zeros: it takes no part in the maximum and is scaled by 0
    // (a -0 from a negative value adds nothing to any sum)
    const bool live = n < k && col0 + 32 * jb < cols;
    float mx = 0.f;
#pragma unroll
    for (int i = 0; i < 32; ++i) mx = fmaxf(mx, fabsf(v[i]));
    mx = live ? mx : 0.f;
    mx = fmaxf(mx, __shfl_xor(mx, 8, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    int e2 = 0;
    (void)frexpf(fminf(mx, 1.0e36f) * 32.f, &e2);   // as in bgemm_prep
    const int e = min(max(e2 - 14, 0), 120);
    const float sd = live ? ldexpf(1.f, -e) : 0.f;
#pragma unroll
    for (int i = 0; i < 32; ++i) v[i] *= sd;
    __builtin_amdgcn_sched_barrier(0);
    u32x2 *const rw = reinterpret_cast<u32x2 *>(slot);
#pragma unroll
    for (int en = 0; en < 8; ++en) {
        int m = 0, gg = 0, o = 0;
        F::blk(jb, en, m, gg, o);
        // words (o, o + 2) and (o + 1, o + 3): values perm4(0..3) in K-slot order
        const h2 h0 = __builtin_convertvector(f2{v[o], v[o + 2]}, h2);
        const h2 h1 = __builtin_convertvector(f2{v[o + 1], v[o + 3]}, h2);
        const h2 l0 = __builtin_convertvector(f2{v[o] - float(h0.x), v[o + 2] - float(h0.y)}, h2);
        const h2 l1 = __builtin_convertvector(f2{v[o + 1] - float(h1.x), v[o + 3] - float(h1.y)}, h2);
        const int it = ((m >> 1) * 64 + n + 16 * gg) * 2 + (m & 1);   // hi part: lane n + 16 g
        rw[it] = u32x2{__builtin_bit_cast(uint32_t, h0), __builtin_bit_cast(uint32_t, h1)};
        rw[it + 16] = u32x2{__builtin_bit_cast(uint32_t, l0), __builtin_bit_cast(uint32_t, l1)};   // lane + 8: lo
    }
    if constexpr (F::kMin) {
        float sx = 0.f;
#pragma unroll
        for (int q = 0; q < 8; ++q) sx += (v[4 * q] + v[4 * q + 1]) + (v[4 * q + 2] + v[4 * q + 3]);
        // K slot kk = 4 g' + i of lane b' + 16 g': hi (kk < 8) or lo part of
        // sub-block kk mod 8's sum of vector b' (zero for b' >= 8)
        uint16_t *const s16 = reinterpret_cast<uint16_t *>(slot + 8192);
        const int i = jb & 3, lh = n + 16 * (jb >> 2), ll = lh + 32;
        s16[lh * 4 + i] = split_part(sx, false);
        s16[(lh + 8) * 4 + i] = 0;
        s16[ll * 4 + i] = split_part(sx, true);
        s16[(ll + 8) * 4 + i] = 0;
    }
    if (jb == 0) reinterpret_cast<float *>(slot + Geo<F>::REC - 32)[n] = ldexpf(1.f, e);
}

// Main pass.  A workgroup's NW waves form nr = NW / nc row groups of nc
// column splits: wave w takes the T 16-row tiles from row 16 T (nr x + w /
// nc) and the steps [c sps, (c + 1) sps) of column split c = nc y + w % nc
// (y > 0 only when the columns are also split between workgroups).  The
// waves work independently until the end (no barrier in the loop).  Each
// step's weights flow through the wave's ring of S LDS stages
// (global_load_lds of whole row runs, so every copy instruction reads long
// contiguous pieces of a few rows), copied two steps ahead; the step's
// activations come from the records (L2-resident, 1 KB contiguous per load
// instruction) into registers two steps ahead.  The loads of one wave
// complete in issue order, and each step issues its activations before the
// weights two steps on, so one wait covers both.  A wave reads its weight
// operands from LDS, computes each tile's sums for the step and undoes the
// record's scale.  At the end the nc splits of a row group add their sums
// through LDS in split order, and the first wave of the group writes them to
// Y, or (SPLIT: the columns also split between workgroups) to
// partial[y][n][row], where the last of the nsplit waves that cover the same
// rows adds them in workgroup order (below).  SHARE (nc = 1 only): the
// records come through a workgroup ring in LDS instead (below).
template <class F, int FORM, bool SPLIT>
__global__ void __launch_bounds__((64 * Geo<F, FORM>::NW), 1) bgemm(const uint8_t *__restrict__ W, int64_t row_bytes, int rows,
                                                          int nsteps, int nblk, const uint8_t *__restrict__ rec,
                                                          int nc, int sps, float *__restrict__ Y, int k, int accumulate,
                                                          float *__restrict__ partial, uint32_t *__restrict__ tickets,
                                                          const float *__restrict__ X, int64_t cols) {
    using G = Geo<F, FORM>;
    constexpr bool SHARE = FORM != kOwn;
    constexpr int T = G::T;
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    const int lane = threadIdx.x & 63, r = lane & 15, g = lane >> 4;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave index, kept in a scalar register
    // every argument in a scalar register before any other work: their
    // loads then go out in one round trip instead of two or three
    asm volatile("" :: "s"(W), "s"(row_bytes), "s"(rows), "s"(nsteps), "s"(nblk), "s"(rec), "s"(nc), "s"(sps),
                 "s"(Y), "s"(k), "s"(accumulate), "s"(partial), "s"(tickets), "s"(X), "s"(cols));
    const int wc = wv % nc, nr = G::NW / nc;
    const int s_lo = (blockIdx.y * nc + wc) * sps, n = max(0, min(sps, nsteps - s_lo));
    const int64_t T0 = (int64_t(blockIdx.x) * nr + wv / nc) * 16 * T;  // first row of this wave's tiles
    f4 acc[T];
#pragma unroll
    for (int u = 0; u < T; ++u) acc[u] = f4{0.f, 0.f, 0.f, 0.f};
    uint32_t *const cnt = reinterpret_cast<uint32_t *>(lds + G::CNT);   // SHARE: arrived[R], done[R]
    if constexpr (SHARE) {
        if (threadIdx.x < 2 * G::R) cnt[threadIdx.x] = 0u;
        __syncthreads();
    }
    // SHARE: every wave takes part in the record ring, including waves past
    // the last row, which copy and compute on the last rows (never stored)
    if ((SHARE || T0 < rows) && n > 0) {
        const int64_t last = rows - 1;
        const int64_t T0c = min<int64_t>(T0, last);                  // copy origin (T0 unless past the rows)
        // copies read whole 16-byte granules; none starts past the one that
        // holds the matrix's last byte (W is 16-byte aligned)
        const int64_t last_granule = (int64_t(rows) * row_bytes - 1) & ~int64_t(15);
        const int64_t base_rel = (T0c * row_bytes) & ~int64_t(15);
        const uint8_t *const wbase = W + base_rel;                         // this wave's copy base (uniform)
        uint8_t *const ring = lds + wv * G::WAVE;
        // this lane's part of a tile copy: instruction i fills LDS bytes
        // [1024 i, 1024 i + 1024) of the tile, lane l the granule at 1024 i + 16 l:
        // byte w of row q's run (lanes past row 15 or the run copy a granule of
        // the matrix into the padding)
        // Offsets are kept relative to the copy base in 32 bits (a wave's tiles
        // span at most 32 rows): the copy of step s starts at
        // (crel + s L) & ~15 (base_rel and w are multiples of 16).
        uint32_t crel[T][G::NI];
        bool cok[G::NI];                                  // a granule of the step, not padding
#pragma unroll
        for (int i = 0; i < G::NI; ++i) {
            const int P = 1024 * i + 16 * lane, q = min(P / G::Lp, 15);
            const int w = P - q * G::Lp;
            cok[i] = w < G::Lc;
#pragma unroll
            for (int u = 0; u < T; ++u) crel[u][i] = uint32_t(min(T0c + 16 * u + q, last) * row_bytes - base_rel) + uint32_t(w);
        }
        const uint32_t lim = uint32_t(min<int64_t>(last_granule - base_rel, 0xfffffff0));
        const auto issue_w = [&](int b, int s) {
            const uint32_t sL = uint32_t(s) * uint32_t(G::L);
#pragma unroll
            for (int u = 0; u < T; ++u) {
                const uint32_t dst = lds_addr(ring + (b * T + u) * G::TB);
#pragma unroll
                for (int i = 0; i < G::NI; ++i)
                    if (G::Lc == G::Lp ? (i + 1 < G::NI || lane < G::LAST) : cok[i])
                        dma<16>(wbase, min((crel[u][i] + sL) & ~15u, lim), dst + 1024 * i);
            }
        };
        uint32_t rlo[T];                                                   // low bits of this lane's row starts
#pragma unroll
        for (int u = 0; u < T; ++u) rlo[u] = uint32_t(min(T0c + 16 * u + r, last) * row_bytes);

        const auto compute = [&](int t, const XRegs &xr) {
            const int s = s_lo + t;
            h4 xa[16];
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                xa[2 * q] = pack(xr.x[q].x, xr.x[q].y);
                xa[2 * q + 1] = pack(xr.x[q].z, xr.x[q].w);
            }
            const h4 xm = F::kMin ? pack(xr.m.x, xr.m.y) : h4{};
            const uint8_t *const st = ring + (t % G::S) * T * G::TB;
#pragma unroll
            for (int u = 0; u < T; ++u) {
                const int mis = int((rlo[u] + uint32_t(s) * uint32_t(G::L)) & 15u);
                const uint8_t *const p = st + u * G::TB + r * G::Lp + mis;   // this lane's row, step s
                typename F::Raw raw;
                F::load(p, s, g, nblk, raw);
                f4 c = {0.f, 0.f, 0.f, 0.f};
                F::compute(raw, p, s, g, nblk, xa, xm, c);
                acc[u] += xr.up * c;
            }
        };

        constexpr int kW = T * G::NI;
        if constexpr (SHARE) {
            // The workgroup's waves share one record per step through a ring of R
            // LDS slots.  Record j is made by wave j mod 8: KA steps ahead it
            // copies the step's activations (eight 1 KB copies) into slot j mod R,
            // and KR < KA steps ahead, once they have landed, it forms the record
            // in place (form_record) and adds 8 to arrived[slot].  Issue order:
            // activations 0 .. KA - 2, weights 0, activations KA - 1, weights 1,
            // then per step t activations t + KA and weights t + 2, so at step t,
            // with only weights t + 1 still allowed in flight, weights t and
            // activations t + KA - 1 have landed: records 0 .. KR - 1 are formed
            // before the loop and record t + KR at step t.  done[b] counts the
            // waves that have read the record in slot b: a wave reads record t once
            // it is formed (arrived), and the maker of record t + KA copies into
            // its slot once all have read record t + KA - R.  The slowest wave
            // never waits (every other wave has formed and read those), so every
            // wait ends; a wave may run KR steps ahead of the maker of a record it
            // needs, a maker R - KA steps ahead of the slowest reader (R = 7, KA =
            // 4, KR = 3: three and three).
            constexpr int kAhead = G::KA, kReport = G::KR;
            const auto slot = [&](int j) { return lds + G::RING_REC + (j % G::R) * G::REC; };
            const auto issue_x = [&](int j) {
                const int64_t c0 = int64_t(s_lo + j) * 256;   // first column of the step
                const uint32_t dst = lds_addr(slot(j));
#pragma unroll
                for (int v = 0; v < 8; ++v) {
                    // lane l copies chunk l ^ v of vector min(v, k - 1) (any
                    // chunk past the last column: the row's first chunk)
                    const int64_t col = c0 + 4 * (lane ^ v);
                    const uint32_t off = uint32_t((int64_t(min(v, k - 1)) * cols + (col < cols ? col : 0)) * 4);
                    dma<16>(reinterpret_cast<const uint8_t *>(X), off, dst + 1024 * v);
                }
            };
            const auto form = [&](int j) {
                form_record<F>(slot(j), lane, int64_t(s_lo + j) * 256, k, cols);
                __builtin_amdgcn_s_waitcnt(kLgkm0);   // the record is in LDS
                __builtin_amdgcn_sched_barrier(0);
                lds_count(&cnt[j % G::R], uint32_t(G::NW));
            };
            const auto mine = [&](int j) { return j < n && j % G::NW == wv; };
            constexpr int kWA = G::S - 1;                        // weights copied kWA steps ahead
            constexpr uint32_t kAll = uint32_t(G::NW);
            for (int j = 0; j < kAhead - 1; ++j)
                if (mine(j)) issue_x(j);
            issue_w(0, s_lo);
            if (mine(kAhead - 1)) issue_x(kAhead - 1);
            if (kWA > 1 && n > 1) issue_w(1, s_lo + 1);
            if (wv < kReport && wv < n) {
                if (kWA > 1 && n > 1) wait_vm<2 * kW>(); else wait_vm<kW>();   // this wave's activations for record wv
                form(wv);
            }
            // the waves of a SIMD (w, w + 4, ...) take turns at the higher issue
            // priority, one step each, so they advance at the same pace and
            // none waits long for another at the counters
            for (int t = 0; t < n; ++t) {
                const int b = t % G::R, jn = t + kAhead;
                if ((G::NW == 8 ? (wv < 4) == ((t & 1) == 0) : ((wv >> 2) + t) % (G::NW / 4) == 0))
                    __builtin_amdgcn_s_setprio(1);
                else
                    __builtin_amdgcn_s_setprio(0);
                // both counters this step waits on, read before the weight wait
                const uint32_t arrived0 = lds_read_count(&cnt[b]);
                const uint32_t done0 = lds_read_count(&cnt[G::R + jn % G::R]);
                wait_vm_or_all<(kWA - 1) * kW>(t + 1 < n);       // weights t, activations t + KA - 1 landed
                if (mine(t + kReport)) form(t + kReport);
                lds_wait_count(&cnt[b], kAll * uint32_t(t / G::R + 1), arrived0);
                const uint8_t *const rc = slot(t);
                XRegs xr;
#pragma unroll
                for (int q = 0; q < 8; ++q) xr.x[q] = *reinterpret_cast<const u32x4a *>(rc + (q * 64 + lane) * 16);
                if constexpr (F::kMin) xr.m = *reinterpret_cast<const u32x2 *>(rc + 8192 + lane * 8);
                xr.up = *reinterpret_cast<const f4 *>(rc + G::REC - 32 + 16 * (g & 1));
                // the next copies go out while those reads are in flight
                if (mine(jn)) {
                    if (jn >= G::R) lds_wait_count(&cnt[G::R + jn % G::R], kAll * uint32_t(jn / G::R), done0);
                    issue_x(jn);
                }
                if (t + kWA < n) issue_w((t + kWA) % G::S, s_lo + t + kWA);
                __builtin_amdgcn_s_waitcnt(kLgkm0);               // record t is in registers
                __builtin_amdgcn_sched_barrier(0);
                lds_count(&cnt[G::R + b]);
                compute(t, xr);
            }
            __builtin_amdgcn_s_setprio(0);
        } else {
        // per step: activations (8 + kMin + 1 loads), then T NI weight copies;
        // both are issued two steps ahead, so step t's are in once at most those
        // of step t + 1 are outstanding
        constexpr int kX = 9 + (F::kMin ? 1 : 0);
        XRegs x0, x1, x2;
        const auto step = [&](int t, const XRegs &cur, XRegs &ahead) {
            wait_vm_or_all<kX + kW>(t + 1 < n);
            if (t + 2 < n) {
                load_x<F>(rec, s_lo + t + 2, lane, g, ahead);
                issue_w((t + 2) % G::S, s_lo + t + 2);
            }
            compute(t, cur);
        };
        issue_w(0, s_lo);
        load_x<F>(rec, s_lo, lane, g, x0);
        if (n > 1) {
            issue_w(1, s_lo + 1);
            load_x<F>(rec, s_lo + 1, lane, g, x1);
        }
        for (int t = 0; t < n; t += 3) {
            step(t, x0, x2);
            if (t + 1 >= n) break;
            step(t + 1, x1, x0);
            if (t + 2 >= n) break;
            step(t + 2, x2, x1);
        }
        }
    }
    if (nc > 1) {
        // every wave's copies have landed and its ring reads are done (the
        // last step waits for all loads); the rings become the exchange area
        __syncthreads();
        f4 *const xch = reinterpret_cast<f4 *>(lds);                     // [wave][tile][lane]
#pragma unroll
        for (int u = 0; u < T; ++u) xch[(wv * T + u) * 64 + lane] = acc[u];
        __syncthreads();
        if (wc == 0) {
#pragma unroll
            for (int u = 0; u < T; ++u)
                for (int c = 1; c < nc; ++c) acc[u] += xch[((wv + c) * T + u) * 64 + lane];
        }
    }
    if (wc != 0 || T0 >= rows) return;
    // lanes g and g + 2 hold the hi and lo parts of outputs n = 4g + i of row r
#pragma unroll
    for (int u = 0; u < T; ++u) {
        const int64_t R = T0 + 16 * u + r;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int nn = 4 * g + i;
            const float o = acc[u][i] + __shfl_down(acc[u][i], 32, 64);
            if (g < 2 && nn < k && R < rows) {
                if constexpr (SPLIT) {
                    __hip_atomic_store(partial + (int64_t(blockIdx.y) * k + nn) * rows + R, o, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
                } else {
                    float *py = Y + nn * int64_t(rows) + R;
                    *py = accumulate ? *py + o : o;
                }
            }
        }
    }
    if constexpr (SPLIT) {
        // Columns split between workgroups: the partial sums above are
        // agent-scope stores (written through to the level every XCD reads,
        // not left dirty in this XCD's L2).  Once they have completed, the
        // wave takes a ticket for its rows (a counter at the start of the
        // workspace, zero between calls); the wave that draws the last of
        // the nsplit sets it back to zero, adds the rows' partial sums in
        // split order (agent-scope loads) and writes Y.  Nothing waits on
        // another wave.
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
        uint32_t *const tp = tickets + int64_t(blockIdx.x) * nr + wv / nc;
        uint32_t tk = 0;
        if (lane == 0) tk = __hip_atomic_fetch_add(tp, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (__builtin_amdgcn_readfirstlane(tk) != gridDim.y - 1) return;
        // every split has drawn: the counter goes back to zero for the next call
        if (lane == 0) __hip_atomic_store(tp, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        // 2T outputs per lane (output i = lane + 64 j is n = i / 16T, row T0
        // + i mod 16T), eight splits at a time: 16T loads in flight before
        // the first add.  A split past the last reloads the last one and adds
        // +0 instead, which leaves every sum as it is (sums start at +0);
        // outputs past k or the last row load a valid one and store nothing.
        const int nrow = int(min<int64_t>(rows - T0, 16 * T)), ns = int(gridDim.y);
        float v[2 * T];
        int64_t o[2 * T];
#pragma unroll
        for (int j = 0; j < 2 * T; ++j) {
            const int i = lane + 64 * j, nn = i / (16 * T), rr = i % (16 * T);
            o[j] = int64_t(min(nn, k - 1)) * rows + T0 + min(rr, nrow - 1);
            v[j] = 0.f;
        }
        for (int sp0 = 0; sp0 < ns; sp0 += 8) {
            float p[8][2 * T];
#pragma unroll
            for (int q = 0; q < 8; ++q)
#pragma unroll
                for (int j = 0; j < 2 * T; ++j)
                    p[q][j] = __hip_atomic_load(partial + int64_t(min(sp0 + q, ns - 1)) * k * rows + o[j],
                                                __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
            for (int q = 0; q < 8; ++q)
#pragma unroll
                for (int j = 0; j < 2 * T; ++j) v[j] += sp0 + q < ns ? p[q][j] : 0.f;
        }
#pragma unroll
        for (int j = 0; j < 2 * T; ++j) {
            const int i = lane + 64 * j, nn = i / (16 * T), rr = i % (16 * T);
            if (nn < k && rr < nrow) Y[o[j]] = accumulate ? Y[o[j]] + v[j] : v[j];
        }
    }
}

struct BgemmShape {
    int groups, nc, nsplit, sps;
    int form;      // kOwn (records from the record kernel), kShared or kWide (formed in LDS; nc = 1)
    int64_t cost;
};

// Launch shape: one workgroup of NW waves per CU, in one of the launch
// forms.  The columns are split nc ways between the waves of a workgroup
// (per-wave-record form only: their sums meet in LDS) and/or nsplit ways
// between workgroups (partial sums through the workspace, added by the last
// wave to finish).  The choice minimises (rounds of workgroups over the
// CUs) x (steps per wave + the ring's fill) x the form's cost per step,
// plus a few steps for the cross-workgroup sum, plus, for the
// per-wave-record form, a term for the activation records (waves of one
// column split read the same record at the same step, served once by the
// CU's cache, so a CU reads nc records per step instead of one) and the
// record kernel.  Costs in twentieths of a per-wave-record step of one
// tile; ties go to the earlier form and fewer splits.  The shared and wide
// forms' step costs are measured ratios (k = 8: the wide form took Q4_K
// 28672 x 8192 39.2-39.3 -> 38.2 us and Q6_K 8192 x 28672 53.8-54.0 ->
// 49.8 us, and lost at 8192 x 8192, where it needs eight splits).
template <class F>
BgemmShape bgemm_shape(int64_t rows, int64_t cols) {
    // the cross-workgroup sum: about one one-tile step of one wave, plus a
    // fifth of a step per split, for the tickets the splits of a row set take
    // one after another on the same counter (measured at k = 8: 1024 x 8192
    // split 32 ways 17.5 us, 16 ways 12.4, 8 ways 10.9, on 64 CUs)
    constexpr int kReduceCost = 20;
    constexpr int kRecordCost = 40;   // the record kernel of the per-wave-record forms: about two steps
    BgemmShape b{};
    int64_t best = -1;
    const int ns = int((cols + 255) / 256);
    // one launch form: per-wave records (any nc) or shared records (nc = 1)
    const auto consider = [&](auto geo, int form) {
        using G = decltype(geo);
        const bool shared = form != kOwn;
        const int step_cost = form == kOwn ? 20 : form == kShared ? RingOf<F, kShared>::cost : RingOf<F, kWide>::cost;
        const int64_t tiles = (rows + 16 * G::T - 1) / (16 * G::T);
        for (int sp = 1; sp <= std::min(ns, 64); ++sp) {
            for (int nc = 1; nc <= (shared ? 1 : G::NW); nc *= 2) {
                const int total = nc * sp, sps = (ns + total - 1) / total;
                if ((ns + sps - 1) / sps != total) continue;   // some split would have no step
                const int64_t groups = (tiles + G::NW / nc - 1) / (G::NW / nc);
                if (sp > 1 && groups * (G::NW / nc) > kMaxTickets) continue;   // counters of a split
                const int64_t rounds = (groups * sp + kNumCUs - 1) / kNumCUs;
                // a step of a wave costs in proportion to the tiles it covers; the
                // shared forms have no record kernel and their own cost per step
                // (the wide form's covers twice the rows per workgroup, and its
                // start costs one step more)
                const int64_t cost = int64_t(step_cost) * G::T * rounds * (sps + G::S - 1) +
                                     (sp > 1 ? kReduceCost + 4 * sp : 0) + (form == kWide ? 20 : 0) +
                                     (shared ? 0 : G::T * rounds * sps * (nc - 1) + kRecordCost);
                if (best < 0 || cost < best) {
                    best = cost;
                    b.groups = int(groups);
                    b.nc = nc;
                    b.nsplit = sp;
                    b.sps = sps;
                    b.form = form;
                    b.cost = cost;
                }
            }
        }
    };
    consider(Geo<F, kOwn>{}, kOwn);
    if constexpr (Geo<F, kShared>::kShare) consider(Geo<F, kShared>{}, kShared);
    if constexpr (Geo<F, kWide>::kShare) consider(Geo<F, kWide>{}, kWide);
    return b;
}

// Shared records (formed in LDS by the main kernel) or records written by
// bgemm_prep to the workspace.
template <class F>
bool shared_records(const BgemmShape &b) {
    return b.form != kOwn;
}

template <class F>
size_t workspace_for(int64_t rows, int64_t cols) {
    const BgemmShape b = bgemm_shape<F>(rows, cols);
    const int64_t ns = (cols + 255) / 256;
    return kTicketBytes + (shared_records<F>(b) ? 0 : size_t(ns) * Geo<F>::REC) +
           (b.nsplit > 1 ? size_t(b.nsplit) * 8 * size_t(rows) * 4 : 0);
}

// The main kernel in one of its four forms (shared records or not; columns
// split between workgroups or not).
template <class F, int FORM, bool SPLIT>
hipError_t launch_main(const BgemmShape &b, hipStream_t st, const uint8_t *W, int64_t row_bytes, int64_t rows,
                       int ns, int64_t nblk, const uint8_t *rec, float *Y, int k, int accumulate, float *partial,
                       uint32_t *tickets, const float *X, int64_t cols) {
    using G = Geo<F, FORM>;
    hipLaunchKernelGGL((bgemm<F, FORM, SPLIT>), dim3(unsigned(b.groups), unsigned(b.nsplit)), dim3(64 * G::NW),
                       FORM != kOwn ? G::LDS_SH : G::LDS, st, W, row_bytes, int(rows), ns, int(nblk), rec, b.nc,
                       b.sps, Y, k, accumulate, partial, tickets, X, cols);
    return hipGetLastError();
}

// More than 64 KB of dynamic LDS: allowed once per kernel (both split
// variants of one form).
template <class F, int FORM>
hipError_t allow_lds() {
    using G = Geo<F, FORM>;
    const int bytes = FORM != kOwn ? G::LDS_SH : G::LDS;
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(&bgemm<F, FORM, false>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
    if (e == hipSuccess)
        e = hipFuncSetAttribute(reinterpret_cast<const void *>(&bgemm<F, FORM, true>),
                                hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
    return e;
}

template <class F>
hipError_t run_bgemm(const void *W, int64_t row_bytes, int64_t rows, int64_t cols, int64_t nblk, const float *X,
                     int k, float *Y, int accumulate, void *ws, hipStream_t st) {
    using G = Geo<F>;
    const int ns = int((cols + 255) / 256);
    const BgemmShape b = bgemm_shape<F>(rows, cols);
    const bool split = b.nsplit > 1, share = shared_records<F>(b);
    uint32_t *const tickets = static_cast<uint32_t *>(ws);
    uint8_t *const rec = static_cast<uint8_t *>(ws) + kTicketBytes;
    float *const partial = reinterpret_cast<float *>(rec + (share ? 0 : int64_t(ns) * G::REC));
    // more than 64 KB of dynamic LDS: allowed once per device for each form
    static std::atomic<uint64_t> done{0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
    if (!((done.load(std::memory_order_acquire) >> dev) & 1)) {
        hipError_t e = allow_lds<F, kOwn>();
        if constexpr (Geo<F, kShared>::kShare) {
            if (e == hipSuccess) e = allow_lds<F, kShared>();
        }
        if constexpr (Geo<F, kWide>::kShare) {
            if (e == hipSuccess) e = allow_lds<F, kWide>();
        }
        if (e != hipSuccess) return e;
        done.fetch_or(uint64_t(1) << dev, std::memory_order_release);
    }
    const uint8_t *const w8 = static_cast<const uint8_t *>(W);
    if constexpr (Geo<F, kShared>::kShare) {
        if (b.form == kShared)
            return split ? launch_main<F, kShared, true>(b, st, w8, row_bytes, rows, ns, nblk, rec, Y, k, accumulate,
                                                         partial, tickets, X, cols)
                         : launch_main<F, kShared, false>(b, st, w8, row_bytes, rows, ns, nblk, rec, Y, k, accumulate,
                                                          partial, tickets, X, cols);
    }
    if constexpr (Geo<F, kWide>::kShare) {
        if (b.form == kWide)
            return split ? launch_main<F, kWide, true>(b, st, w8, row_bytes, rows, ns, nblk, rec, Y, k, accumulate,
                                                       partial, tickets, X, cols)
                         : launch_main<F, kWide, false>(b, st, w8, row_bytes, rows, ns, nblk, rec, Y, k, accumulate,
                                                        partial, tickets, X, cols);
    }
    hipLaunchKernelGGL(bgemm_prep<F>, dim3(unsigned(ns)), dim3(256), 0, st, X, cols, k, rec);
    if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
    return split ? launch_main<F, kOwn, true>(b, st, w8, row_bytes, rows, ns, nblk, rec, Y, k, accumulate, partial,
                                              tickets, X, cols)
                 : launch_main<F, kOwn, false>(b, st, w8, row_bytes, rows, ns, nblk, rec, Y, k, accumulate, partial,
                                               tickets, X, cols);
}

}  // namespace

bool gemm_batch_type_ok(nt_qtype t) {
    return t == NT_Q8_0 || t == NT_Q4_0 || t == NT_Q4_K || t == NT_Q5_K || t == NT_Q6_K;
}

size_t gemm_batch_workspace_bytes(nt_qtype t, int64_t rows, int64_t cols) {
    switch (t) {
    case NT_Q8_0: return workspace_for<BQ80>(rows, cols);
    case NT_Q4_0: return workspace_for<BQ40>(rows, cols);
    case NT_Q5_K: return workspace_for<BQ5K>(rows, cols);
    case NT_Q4_K: return workspace_for<BQ4K>(rows, cols);
    case NT_Q6_K: return workspace_for<BQ6K>(rows, cols);
    default: return 0;
    }
}

hipError_t launch_gemm_batch(nt_qtype t, const void *W, int64_t rows, int64_t cols, const float *X, int k, float *Y,
                             int accumulate, void *ws, hipStream_t st) {
    if (rows == 0) return hipSuccess;
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
