// quantize.hip -- fp32 values -> packed blocks on the GPU, one thread per
// block.  Used to build large synthetic models directly in HBM.
//
// The write-up ("Overview") reads GGUF files whose weights were encoded
// offline; it does not say how.  This encoder is the plain one with a
// provable bound |x - decoded| <= step/2, in fp64, every operation rounded
// as written (no contraction), "round" = half away from zero:
//   Q8_0  d = fp16_rne(max|x|/127); q = clamp(round(x/d), -127, 127)
//   Q4_0  d = fp16_rne(max|x|/7);   q = clamp(round(x/d), -8, 7) + 8
//   Q4_K  per 32-value sub-block j: m_j = -min(0, min x);
//         dmin = fp16_up(max m_j / 63); M_j = ceil(m_j/dmin); o_j = dmin*M_j;
//         s_j = (max(max x, -o_j) + o_j)/15; d = fp16_up(max s_j / 63);
//         S_j = ceil(s_j/d); q = clamp(round((x + o_j)/(d*S_j)), 0, 15)
//   Q5_K  as Q4_K with 31 in place of 15 (q in [0, 31]: low 4 bits in qs, the
//         fifth in qh)
//   Q6_K  per 16-value sub-block j: s_j = max|x|/31; d = fp16_up(max s_j/127);
//         S_j = ceil(s_j/d); q = clamp(round(x/(d*S_j)), -32, 31) + 32
// fp16_rne rounds to nearest (ties to even); fp16_up gives the smallest fp16
// >= its argument.  A zero scale gives zero codes.
#include "device_util.h"
#include "nt_internal.h"

#pragma clang fp contract(off)

namespace nt {
namespace {

// IEEE binary16 encoding of v >= 0 with the given rounding of the scaled
// significand (rint: to nearest even; ceil: upward).
template <bool kUp>
__device__ uint32_t f16_encode_pos(double v) {
    if (v == 0.0) return 0;
    if (v < 0x1p-14) {                     // subnormal: multiples of 2^-24
        const double q = kUp ? ceil(v * 0x1p24) : rint(v * 0x1p24);
        return uint32_t(q);                // 1024 is the smallest normal's pattern
    }
    int e2;
    (void)frexp(v, &e2);                   // v in [2^(e2-1), 2^e2)
    int E = e2 - 1;
    double q = ldexp(v, 10 - E);           // [1024, 2048)
    q = kUp ? ceil(q) : rint(q);
    if (q >= 2048.0) { q = 1024.0; E += 1; }
    if (E > 15) return 0x7c00u;
    return uint32_t((E + 15) << 10) | (uint32_t(q) - 1024u);
}

__device__ double f16_value(uint32_t h) {
    const uint32_t e = (h >> 10) & 31, m = h & 1023;
    if (e == 0) return ldexp(double(m), -24);
    return ldexp(double(1024 + m), int(e) - 25);
}

__device__ __forceinline__ void put16(uint8_t *p, uint32_t v) { p[0] = uint8_t(v); p[1] = uint8_t(v >> 8); }

__device__ void enc_q8_0(const float *x, uint8_t *blk) {
    double a = 0.0;
    for (int e = 0; e < 32; ++e) a = fmax(a, fabs(double(x[e])));
    const uint32_t dh = f16_encode_pos<false>(a / 127.0);
    const double d = f16_value(dh);
    put16(blk, dh);
    for (int e = 0; e < 32; ++e) {
        double q = d == 0.0 ? 0.0 : round(double(x[e]) / d);
        q = fmin(127.0, fmax(-127.0, q));
        blk[2 + e] = uint8_t(int8_t(q));
    }
}

__device__ void enc_q4_0(const float *x, uint8_t *blk) {
    double a = 0.0;
    for (int e = 0; e < 32; ++e) a = fmax(a, fabs(double(x[e])));
    const uint32_t dh = f16_encode_pos<false>(a / 7.0);
    const double d = f16_value(dh);
    put16(blk, dh);
    for (int i = 0; i < 16; ++i) {
        double q0 = d == 0.0 ? 0.0 : round(double(x[i]) / d);
        double q1 = d == 0.0 ? 0.0 : round(double(x[i + 16]) / d);
        const int lo = int(fmin(7.0, fmax(-8.0, q0))) + 8;
        const int hi = int(fmin(7.0, fmax(-8.0, q1))) + 8;
        blk[2 + i] = uint8_t(lo | (hi << 4));
    }
}

// Q4_K and Q5_K header: offsets o_j, steps d*S_j and the packed d, dmin and
// scale bytes in blk[0..16); codes take LEVELS + 1 values (15 or 31).
template <int LEVELS>
__device__ void enc_kq_header(const float *x, uint8_t *blk, double o[8], double step[8]) {
    double m[8], s[8], mmax = 0.0, smax = 0.0;
    int S[8], M[8];
    for (int j = 0; j < 8; ++j) {
        double mn = 0.0;
        for (int i = 0; i < 32; ++i) mn = fmin(mn, double(x[32 * j + i]));
        m[j] = -mn;
        mmax = fmax(mmax, m[j]);
    }
    const uint32_t dminh = f16_encode_pos<true>(mmax / 63.0);
    const double dmin = f16_value(dminh);
    for (int j = 0; j < 8; ++j) {
        M[j] = dmin == 0.0 ? 0 : int(ceil(m[j] / dmin));
        o[j] = dmin * double(M[j]);
    }
    for (int j = 0; j < 8; ++j) {
        double mx = -o[j];
        for (int i = 0; i < 32; ++i) mx = fmax(mx, double(x[32 * j + i]));
        s[j] = (mx + o[j]) / double(LEVELS);
        smax = fmax(smax, s[j]);
    }
    const uint32_t dh = f16_encode_pos<true>(smax / 63.0);
    const double d = f16_value(dh);
    for (int j = 0; j < 8; ++j) {
        S[j] = d == 0.0 ? 0 : int(ceil(s[j] / d));
        step[j] = d * double(S[j]);
    }
    put16(blk, dh);
    put16(blk + 2, dminh);
    for (int j = 0; j < 4; ++j) {
        blk[4 + j] = uint8_t((S[j] & 63) | ((S[j + 4] >> 4) << 6));
        blk[8 + j] = uint8_t((M[j] & 63) | ((M[j + 4] >> 4) << 6));
        blk[12 + j] = uint8_t((S[j + 4] & 15) | ((M[j + 4] & 15) << 4));
    }
}

// code of value v in a sub-block with offset o and step st: round((v + o)/st) in [0, LEVELS]
template <int LEVELS>
__device__ __forceinline__ int enc_kq_code(float v, double o, double st) {
    const double q = st == 0.0 ? 0.0 : round((double(v) + o) / st);
    return int(fmin(double(LEVELS), fmax(0.0, q)));
}

__device__ void enc_q4_k(const float *x, uint8_t *blk) {
    double o[8], step[8];
    enc_kq_header<15>(x, blk, o, step);
    for (int p = 0; p < 4; ++p)            // byte 32p + i: sub-block 2p low, 2p+1 high
        for (int i = 0; i < 32; ++i) {
            const int lo = enc_kq_code<15>(x[64 * p + i], o[2 * p], step[2 * p]);
            const int hi = enc_kq_code<15>(x[64 * p + 32 + i], o[2 * p + 1], step[2 * p + 1]);
            blk[16 + 32 * p + i] = uint8_t(lo | (hi << 4));
        }
}

__device__ void enc_q5_k(const float *x, uint8_t *blk) {
    double o[8], step[8];
    enc_kq_header<31>(x, blk, o, step);
    for (int i = 0; i < 32; ++i) blk[16 + i] = 0;   // qh: bit j of qh[i] = fifth bit of value 32j + i
    for (int p = 0; p < 4; ++p)
        for (int i = 0; i < 32; ++i) {
            const int lo = enc_kq_code<31>(x[64 * p + i], o[2 * p], step[2 * p]);
            const int hi = enc_kq_code<31>(x[64 * p + 32 + i], o[2 * p + 1], step[2 * p + 1]);
            blk[48 + 32 * p + i] = uint8_t((lo & 15) | ((hi & 15) << 4));
            blk[16 + i] |= uint8_t(((lo >> 4) << (2 * p)) | ((hi >> 4) << (2 * p + 1)));
        }
}

__device__ void enc_q6_k(const float *x, uint8_t *blk) {
    double s[16], smax = 0.0;
    int S[16];
    for (int j = 0; j < 16; ++j) {
        double a = 0.0;
        for (int i = 0; i < 16; ++i) a = fmax(a, fabs(double(x[16 * j + i])));
        s[j] = a / 31.0;
        smax = fmax(smax, s[j]);
    }
    const uint32_t dh = f16_encode_pos<true>(smax / 127.0);
    const double d = f16_value(dh);
    for (int j = 0; j < 16; ++j) {
        S[j] = d == 0.0 ? 0 : int(ceil(s[j] / d));
        blk[192 + j] = uint8_t(int8_t(S[j]));
    }
    put16(blk + 208, dh);
    // code of value e, 0..63
    auto code = [&](int e) {
        const double st = d * double(S[e >> 4]);
        const double q = st == 0.0 ? 0.0 : round(double(x[e]) / st);
        return int(fmin(31.0, fmax(-32.0, q))) + 32;
    };
    for (int h = 0; h < 2; ++h)
        for (int l = 0; l < 32; ++l) {
            const int q0 = code(128 * h + l), q1 = code(128 * h + 32 + l);
            const int q2 = code(128 * h + 64 + l), q3 = code(128 * h + 96 + l);
            blk[64 * h + l] = uint8_t((q0 & 15) | ((q2 & 15) << 4));
            blk[64 * h + 32 + l] = uint8_t((q1 & 15) | ((q3 & 15) << 4));
            blk[128 + 32 * h + l] =
                uint8_t((q0 >> 4) | ((q1 >> 4) << 2) | ((q2 >> 4) << 4) | ((q3 >> 4) << 6));
        }
}

template <int T>
__global__ void __launch_bounds__(128) quantize_kernel(const float *__restrict__ x, uint8_t *__restrict__ out,
                                                      int64_t nblocks) {
    constexpr int BE = (T == NT_Q8_0 || T == NT_Q4_0) ? 32 : 256;
    constexpr int BB = T == NT_Q8_0 ? 34 : T == NT_Q4_0 ? 18 : T == NT_Q4_K ? 144 : T == NT_Q5_K ? 176 : 210;
    const int64_t stride = int64_t(gridDim.x) * blockDim.x;
    for (int64_t b = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; b < nblocks; b += stride) {
        const float *xb = x + b * BE;
        uint8_t *ob = out + b * BB;
        if constexpr (T == NT_Q8_0) enc_q8_0(xb, ob);
        else if constexpr (T == NT_Q4_0) enc_q4_0(xb, ob);
        else if constexpr (T == NT_Q4_K) enc_q4_k(xb, ob);
        else if constexpr (T == NT_Q5_K) enc_q5_k(xb, ob);
        else enc_q6_k(xb, ob);
    }
}

}  // namespace

hipError_t launch_quantize(nt_qtype t, const float *x, void *blocks, int64_t n, hipStream_t st) {
    const int64_t nb = n / block_elems(t);
    const int threads = 128;
    int64_t want = (nb + threads - 1) / threads;
    const int grid = int(want < 32768 ? want : 32768);
    uint8_t *o = static_cast<uint8_t *>(blocks);
    switch (t) {
    case NT_Q8_0: quantize_kernel<NT_Q8_0><<<grid, threads, 0, st>>>(x, o, nb); break;
    case NT_Q4_0: quantize_kernel<NT_Q4_0><<<grid, threads, 0, st>>>(x, o, nb); break;
    case NT_Q4_K: quantize_kernel<NT_Q4_K><<<grid, threads, 0, st>>>(x, o, nb); break;
    case NT_Q5_K: quantize_kernel<NT_Q5_K><<<grid, threads, 0, st>>>(x, o, nb); break;
    case NT_Q6_K: quantize_kernel<NT_Q6_K><<<grid, threads, 0, st>>>(x, o, nb); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace nt
