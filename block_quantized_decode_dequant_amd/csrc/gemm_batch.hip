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
//    tile, K 16 codes of one scale group (or of one super-block whose scales
//    are folded into the codes).  With N = weight row, every lane applies the
//    scales of its own row to its own accumulators.
//  * weight codes become fp16 exactly: small integers, or (Q4_K) the integer
//    S_j * q scaled by 2^-14, built from the nibble as an fp16 subnormal times
//    an exact fp16 scale.  Nothing about the weights is rounded.
//  * each activation is split into fp16 hi + lo (hi = fp16(x), lo =
//    fp16(x - hi)), which leaves about 2^-22 relative error; the hi parts fill
//    M rows 0-7 and the lo parts rows 8-15, which the padding of k <= 8 to 16
//    would otherwise waste.  Products are exact in fp32; the MFMA sums in fp32.
//  * a prologue kernel writes the split activations once per call in the
//    order the lanes consume them, so each wave reads 128 contiguous bytes
//    per lane per 256 columns.
//  * MFMA lane layout (16x16x16 f16): src0 lane l holds A[l % 16][4(l/16) + i],
//    src1 lane l holds B[4(l/16) + i][l % 16], the result lane l holds
//    D[4(l/16) + i][l % 16], i = 0..3.  Inside one MFMA the order of the 16
//    K slots is free as long as A and B agree, so each lane takes the codes of
//    its row that lie together in memory.
//
// A workgroup of kWaves waves owns 16 rows; its waves take interleaved
// 256-column steps and add their partial sums through LDS in a fixed order.
#include <algorithm>

#include "device_util.h"
#include "nt_internal.h"

namespace nt {
namespace {

typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef uint32_t w2 __attribute__((ext_vector_type(2)));

constexpr int kWaves = 8;

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

// The 32-bit word at a 2-byte-aligned address: two aligned words and a byte
// funnel.  With sh == 0 the second load re-reads the first word, so no word
// wholly past the bytes asked for is touched.
__device__ __forceinline__ uint32_t ldu(const uint8_t *p) {
    const uint32_t sh = uint32_t(reinterpret_cast<uintptr_t>(p) & 3);
    const uint8_t *a = p - sh;
    const uint32_t lo = ld1(a), hi = ld1(a + (sh ? 4 : 0));
    return funnel(hi, lo, shift_sel(sh));
}

// ---- Q8_0: a step is 8 blocks; MFMA m covers block m/2, elements
// 8g + 4(m&1) + perm4(i) for lane group g.
struct BQ80 {
    static constexpr bool kMin = false;
    __host__ __device__ static int elem(int m, int g, int i) { return 32 * (m >> 1) + 8 * g + 4 * (m & 1) + perm4(i); }
    // int8 codes of a word -> two fp16 pairs q (bytes 0,2 and 1,3): 0x64uu is
    // 1024 + uu, the sign bit flipped makes uu = q + 128.
    __device__ static h4 codes(uint32_t w) {
        const uint32_t a = hadd((w & 0x00ff00ffu) ^ 0x64806480u, _Float16(-1152.f));
        const uint32_t b = hadd(((w >> 8) & 0x00ff00ffu) ^ 0x64806480u, _Float16(-1152.f));
        return pack(a, b);
    }
    __device__ static void step(const uint8_t *row, int s, int g, int nblk, const h4 *xa, h4, f4 &acc) {
#pragma unroll
        for (int bb = 0; bb < 8; ++bb) {
            const int blk = 8 * s + bb;
            if (blk >= nblk) break;                       // uniform over the wave
            const uint8_t *b = row + int64_t(blk) * 34;
            const uint32_t w0 = ldu(b + 2 + 8 * g), w1 = ldu(b + 6 + 8 * g);
            const uint32_t dsh = uint32_t(reinterpret_cast<uintptr_t>(b) & 2);
            const float d = h2f(ld1(b - dsh) >> (8 * dsh));
            f4 c = mfma(xa[2 * bb], codes(w0), f4{0.f, 0.f, 0.f, 0.f});
            c = mfma(xa[2 * bb + 1], codes(w1), c);
            acc += d * c;
        }
    }
};

// ---- Q4_K: a step is one super-block; lane group g takes bytes 8g..8g+7 of
// each 32-byte pair chunk p (low nibbles: sub-block 2p, high: 2p+1).  MFMA
// m = 4p + 2*nib + j uses dword j of chunk p.  The codes carry their 6-bit
// scale: (q * 2^-24 or q * 2^-20 as an fp16 subnormal) * fp16(S * 2^10 or
// S * 2^6) = S q 2^-14 exactly (S q <= 945).  The mins go through one more
// MFMA: A = per-sub-block activation sums (hi in K slots 0-7, lo in 8-15),
// B = M_j.
struct BQ4K {
    static constexpr bool kMin = true;
    __host__ __device__ static int elem(int m, int g, int i) {
        const int p = m >> 2, nib = (m >> 1) & 1, j = m & 1;
        return 32 * (2 * p + nib) + 8 * g + 4 * j + perm4(i);
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
    __device__ static void step(const uint8_t *row, int s, int g, int, const h4 *xa, h4 xm, f4 &acc) {
        const uint8_t *b = row + int64_t(s) * 144;
        const u32x4 h = ld4(b);
        w2 q[4];
#pragma unroll
        for (int p = 0; p < 4; ++p) q[p] = *reinterpret_cast<const w2 *>(b + 16 + 32 * p + 8 * g);
        f4 c = {0.f, 0.f, 0.f, 0.f};
        uint32_t Mw[4];
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            uint32_t S0, M0, S1, M1;
            scale_min(h, 2 * p, S0, M0);
            scale_min(h, 2 * p + 1, S1, M1);
            const _Float16 f0 = _Float16(float(S0 * 1024u)), f1 = _Float16(float(S1 * 64u));
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const uint32_t w = q[p][j], t = w >> 8;
                c = mfma(xa[4 * p + j], pack(hmul(w & 0x000f000fu, f0), hmul(t & 0x000f000fu, f0)), c);
                c = mfma(xa[4 * p + 2 + j], pack(hmul(w & 0x00f000f0u, f1), hmul(t & 0x00f000f0u, f1)), c);
            }
            Mw[p] = M0 | (M1 << 16);
        }
        // B of the min MFMA: K slot 4g + i takes M_{(4g + i) & 7}
        const uint32_t ma = (g & 1) ? Mw[2] : Mw[0], mc = (g & 1) ? Mw[3] : Mw[1];
        const h4 mb = {_Float16(float(ma & 0xffffu)), _Float16(float(ma >> 16)), _Float16(float(mc & 0xffffu)),
                       _Float16(float(mc >> 16))};
        const f4 cm = mfma(xm, mb, f4{0.f, 0.f, 0.f, 0.f});
        const float d = h2f(h.x) * 16384.f, dmin = h2f(h.x >> 16);
        acc += d * c - dmin * cm;
    }
};

// ---- Q6_K: a step is one super-block (210 bytes, so only 2-byte aligned).
// MFMA m = 8h + 2k + lh is the 16-value scale group scales[m]: values
// 128h + 32k + 16lh + 4g + perm4(i); the low four bits come from
// ql[64h + 32(k&1) + 16lh + 4g + i] (nibble k>>1), the top two from
// qh[32h + 16lh + 4g + i] (bits 2k, 2k+1).  Codes become q - 32 exactly.
struct BQ6K {
    static constexpr bool kMin = false;
    __host__ __device__ static int elem(int m, int g, int i) {
        const int h = m >> 3, k = (m >> 1) & 3, lh = m & 1;
        return 128 * h + 32 * k + 16 * lh + 4 * g + perm4(i);
    }
    __device__ static h4 codes(uint32_t lo4, uint32_t qh, int k) {
        const uint32_t q = lo4 | (((qh >> (2 * k)) & 0x03030303u) << 4);
        const uint32_t a = hadd((q & 0x00ff00ffu) | 0x64006400u, _Float16(-1056.f));
        const uint32_t b = hadd(((q >> 8) & 0x00ff00ffu) | 0x64006400u, _Float16(-1056.f));
        return pack(a, b);
    }
    __device__ static void step(const uint8_t *row, int s, int g, int, const h4 *xa, h4, f4 &acc) {
        const uint8_t *b = row + int64_t(s) * 210;
        uint32_t ql[2][2][2], qh[2][2];
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int lh = 0; lh < 2; ++lh) {
                ql[h][0][lh] = ldu(b + 64 * h + 16 * lh + 4 * g);
                ql[h][1][lh] = ldu(b + 64 * h + 32 + 16 * lh + 4 * g);
                qh[h][lh] = ldu(b + 128 + 32 * h + 16 * lh + 4 * g);
            }
        // 16 int8 scales and d: words at 192 - sh .. 208 - sh, funnelled
        const uint32_t sh = uint32_t(reinterpret_cast<uintptr_t>(b) & 2);
        const u32x4 sw = ld4(b + 192 - sh);
        const uint32_t tail = ld1(b + 208 - sh);
        const uint32_t sel = shift_sel(sh);
        const uint32_t sc[4] = {funnel(sw.y, sw.x, sel), funnel(sw.z, sw.y, sel), funnel(sw.w, sw.z, sel),
                                funnel(tail, sw.w, sel)};
        const float d = h2f(sh ? tail >> 16 : tail);
        f4 t = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int m = 0; m < 16; ++m) {
            const int h = m >> 3, k = (m >> 1) & 3, lh = m & 1;
            const uint32_t l = ql[h][k & 1][lh];
            const uint32_t lo4 = (k < 2 ? l : l >> 4) & 0x0f0f0f0fu;
            const f4 c = mfma(xa[m], codes(lo4, qh[h][lh], k), f4{0.f, 0.f, 0.f, 0.f});
            const float scm = float(int8_t((sc[m >> 2] >> (8 * (m & 3))) & 0xffu));
            t += scm * c;
        }
        acc += d * t;
    }
};

// Split activations in lane order: xp[((s * 64 + lane) * 16 + m) * 4 + i]
// (fp16) = hi or lo part of x_n[256 s + elem(m, g, i)], n = lane % 8,
// lo for lane % 16 >= 8, zero for n >= k or past cols.  For K-quant mins,
// xm[(s * 64 + lane) * 4 + i]: K slot 4g + i of lane (b, g) is the hi (slots
// 0-7) or lo (8-15) part of the sum of x_b over sub-block (4g + i) & 7;
// zero for b >= 8.
__device__ __forceinline__ uint16_t hbits(float v) { return __half_as_ushort(__float2half_rn(v)); }
__device__ __forceinline__ uint16_t split_part(float v, bool lo) {
    const __half hi = __float2half_rn(v);
    return lo ? hbits(v - __half2float(hi)) : __half_as_ushort(hi);
}

template <class F>
__global__ void __launch_bounds__(256) bgemm_prep(const float *__restrict__ X, int64_t cols, int k, int nsteps,
                                                  uint32_t *__restrict__ xp, uint32_t *__restrict__ xm) {
    const int64_t t = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
    if (t >= int64_t(nsteps) * 1024) return;
    const int m = int(t & 15), lane = int((t >> 4) & 63);
    const int64_t s = t >> 10;
    const int b = lane & 15, g = lane >> 4, n = b & 7;
    const bool lo = b >= 8;
    uint32_t hv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int64_t e = s * 256 + F::elem(m, g, i);
        const float v = (n < k && e < cols) ? X[n * cols + e] : 0.f;
        hv[i] = split_part(v, lo);
    }
    xp[2 * t] = hv[0] | (hv[1] << 16);
    xp[2 * t + 1] = hv[2] | (hv[3] << 16);
    if constexpr (F::kMin) {
        if (m == 0) {
            uint32_t mv[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int kk = 4 * g + i, j = kk & 7;
                float sx = 0.f;
                if (b < 8 && n < k) {
                    const float *p = X + n * cols + s * 256 + 32 * j;
                    for (int u = 0; u < 32; ++u) sx += p[u];
                }
                mv[i] = split_part(sx, kk >= 8);
            }
            const int64_t o = (s * 64 + lane) * 2;
            xm[o] = mv[0] | (mv[1] << 16);
            xm[o + 1] = mv[2] | (mv[3] << 16);
        }
    }
}

template <class F>
__global__ void __launch_bounds__(64 * kWaves) bgemm(const uint8_t *__restrict__ W, int64_t row_bytes, int rows,
                                                      int nsteps, int nblk, const uint32_t *__restrict__ xp,
                                                      const uint32_t *__restrict__ xm, float *__restrict__ Y,
                                                      int k, int accumulate) {
    __shared__ float part[kWaves][16][8];
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6, r = lane & 15, g = lane >> 4;
    const int64_t R = int64_t(blockIdx.x) * 16 + r;
    // rows past the end read row 0 (in bounds); their results are not written
    const uint8_t *row = W + (R < rows ? R : 0) * row_bytes;
    f4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int s = wv; s < nsteps; s += kWaves) {
        const u32x4 *px = reinterpret_cast<const u32x4 *>(xp) + (int64_t(s) * 64 + lane) * 8;
        h4 xa[16];
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            const u32x4 v = px[q];
            xa[2 * q] = pack(v.x, v.y);
            xa[2 * q + 1] = pack(v.z, v.w);
        }
        h4 xmin = {};
        if constexpr (F::kMin) {
            const w2 v = *reinterpret_cast<const w2 *>(xm + (int64_t(s) * 64 + lane) * 2);
            xmin = pack(v.x, v.y);
        }
        F::step(row, s, g, nblk, xa, xmin, acc);
    }
    // lanes g and g + 2 hold the hi and lo parts of outputs n = 4g + i
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float o = acc[i] + __shfl_down(acc[i], 32, 64);
        if (g < 2) part[wv][r][4 * g + i] = o;
    }
    __syncthreads();
    if (threadIdx.x < 128) {
        const int rr = threadIdx.x & 15, n = threadIdx.x >> 4;
        const int64_t R2 = int64_t(blockIdx.x) * 16 + rr;
        if (n < k && R2 < rows) {
            float v = 0.f;
#pragma unroll
            for (int w = 0; w < kWaves; ++w) v += part[w][rr][n];
            float *py = Y + n * int64_t(rows) + R2;
            *py = accumulate ? *py + v : v;
        }
    }
}

}  // namespace

int64_t bgemm_steps(int64_t cols) { return (cols + 255) / 256; }

bool gemm_batch_type_ok(nt_qtype t) { return t == NT_Q8_0 || t == NT_Q4_K || t == NT_Q6_K; }

size_t gemm_batch_workspace_bytes(nt_qtype t, int64_t cols) {
    const int64_t ns = bgemm_steps(cols);
    return size_t(ns) * 8192 + (t == NT_Q4_K ? size_t(ns) * 512 : 0);
}

template <class F>
hipError_t run_bgemm(const void *W, int64_t row_bytes, int64_t rows, int64_t cols, int64_t nblk, const float *X,
                     int k, float *Y, int accumulate, void *ws, hipStream_t st) {
    const int ns = int(bgemm_steps(cols));
    uint32_t *xp = static_cast<uint32_t *>(ws);
    uint32_t *xm = F::kMin ? xp + int64_t(ns) * 2048 : nullptr;
    const int64_t nt = int64_t(ns) * 1024;
    hipLaunchKernelGGL(bgemm_prep<F>, dim3(unsigned((nt + 255) / 256)), dim3(256), 0, st, X, cols, k, ns, xp, xm);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || rows == 0) return e;
    hipLaunchKernelGGL(bgemm<F>, dim3(unsigned((rows + 15) / 16)), dim3(64 * kWaves), 0, st,
                       static_cast<const uint8_t *>(W), row_bytes, int(rows), ns, int(nblk), xp, xm, Y, k, accumulate);
    return hipGetLastError();
}

hipError_t launch_gemm_batch(nt_qtype t, const void *W, int64_t rows, int64_t cols, const float *X, int k, float *Y,
                             int accumulate, void *ws, hipStream_t st) {
    const int64_t nblk = cols / block_elems(t), row_bytes = nblk * block_bytes(t);
    switch (t) {
    case NT_Q8_0: return run_bgemm<BQ80>(W, row_bytes, rows, cols, nblk, X, k, Y, accumulate, ws, st);
    case NT_Q4_K: return run_bgemm<BQ4K>(W, row_bytes, rows, cols, nblk, X, k, Y, accumulate, ws, st);
    case NT_Q6_K: return run_bgemm<BQ6K>(W, row_bytes, rows, cols, nblk, X, k, Y, accumulate, ws, st);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace nt
