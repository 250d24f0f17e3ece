/*
 * formats.c -- the block-quantized weight formats: sizes, decoders and
 * the oracle's own encoders.  Test infrastructure only.
 *
 * Source: the ntransformer write-up (GeekNews topic 26894), "Overview", names
 * the GGUF quantizations the engine reads (Q4_0, Q8_0, Q4_K_M, Q5_K, Q6_K);
 * "Performance" says Q4_K_M keeps 36 instead of 26 of the 70B's layers in
 * 24 GB, and "NVMe direct streaming" gives about 670 MB per 70B Q6_K layer.
 * The pages give no byte layout.  The layouts here are the public GGUF block
 * definitions, restated (all multi-byte fields little-endian):
 *
 *   Q8_0  34 B / 32 values : d (fp16) | qs int8[32]           x_e = d*qs[e]
 *   Q4_0  18 B / 32 values : d (fp16) | qs u8[16]
 *         q = e<16 ? qs[e] & 15 : qs[e-16] >> 4               x_e = d*(q-8)
 *   Q4_K 144 B / 256 values: d, dmin (fp16) | scales u8[12] | qs u8[128]
 *         sub-block j = e/32 has 6-bit scale S_j and 6-bit min M_j;
 *         q = nibble of qs[32*(j/2) + e%32] (low for even j, high for odd j)
 *         x_e = (d*S_j)*q - dmin*M_j
 *   Q5_K 176 B / 256 values: d, dmin (fp16) | scales u8[12] | qh u8[32] | qs u8[128]
 *         scales, mins and low 4 bits as in Q4_K; the fifth bit of value
 *         e = 32j + l is bit j of qh[l]; q in [0,31]
 *         x_e = (d*S_j)*q - dmin*M_j
 *   Q6_K 210 B / 256 values: ql u8[128] | qh u8[64] | scales int8[16] | d (fp16)
 *         half h = e/128, r = e%128, k = r/32, l = r%32;
 *         low 4 bits: nibble of ql[64h + 32(k&1) + l] (low if k<2, else high);
 *         high 2 bits: (qh[32h + l] >> 2k) & 3;  q in [0,63]
 *         x_e = d*scales[e/16]*(q-32)
 *
 * The 70B layer size is the one number on the pages that these layouts can be
 * checked against: 855,638,016 weights per layer at 210/256 bytes each is
 * 701,890,560 B = 669.4 MiB, the "about 670 MB per layer" the NVMe section
 * quotes (a test checks it).
 *
 * Decoders form each value exactly in fp64 (every product here has at most
 * 23 significant bits) and round once to fp32.
 *
 * Q5_K is the next format the write-up lists ("Overview"); it has the same
 * 6-bit scale/min packing as Q4_K plus one bit plane, 5.5 bits per weight.
 */
#include "oracle.h"

#include <math.h>
#include <string.h>

int64_t or_block_elems(int type)
{
    switch (type) {
    case OR_F32: case OR_F16: return 1;
    case OR_Q8_0: case OR_Q4_0: return 32;
    case OR_Q4_K: case OR_Q5_K: case OR_Q6_K: return 256;
    default: return -1;
    }
}

int64_t or_block_bytes(int type)
{
    switch (type) {
    case OR_F32: return 4;
    case OR_F16: return 2;
    case OR_Q8_0: return 34;
    case OR_Q4_0: return 18;
    case OR_Q4_K: return 144;
    case OR_Q5_K: return 176;
    case OR_Q6_K: return 210;
    default: return -1;
    }
}

int64_t or_row_bytes(int type, int64_t cols)
{
    int64_t be = or_block_elems(type);
    if (be <= 0 || cols < 0 || cols % be != 0)
        return -1;
    return cols / be * or_block_bytes(type);
}

static uint16_t rd16(const uint8_t *p) { return (uint16_t)(p[0] | (p[1] << 8)); }
static void wr16(uint8_t *p, uint16_t v) { p[0] = (uint8_t)v; p[1] = (uint8_t)(v >> 8); }

/* Q4_K 6-bit scale and min of sub-block j from the 12 packed bytes b. */
static void q4k_scale_min(const uint8_t *b, int j, int *S, int *M)
{
    if (j < 4) {
        *S = b[j] & 63;
        *M = b[j + 4] & 63;
    } else {
        *S = (b[j + 4] & 15) | ((b[j - 4] >> 6) << 4);
        *M = (b[j + 4] >> 4) | ((b[j] >> 6) << 4);
    }
}

/* ---- decoders ----------------------------------------------------------- */

static void dq_q8_0(const uint8_t *blk, float *out)
{
    double d = or_f16_to_f64(rd16(blk));
    for (int e = 0; e < 32; ++e)
        out[e] = (float)(d * (double)(int8_t)blk[2 + e]);
}

static void dq_q4_0(const uint8_t *blk, float *out)
{
    double d = or_f16_to_f64(rd16(blk));
    const uint8_t *qs = blk + 2;
    for (int e = 0; e < 32; ++e) {
        int q = e < 16 ? (qs[e] & 15) : (qs[e - 16] >> 4);
        out[e] = (float)(d * (double)(q - 8));
    }
}

static void dq_q4_k(const uint8_t *blk, float *out)
{
    double d = or_f16_to_f64(rd16(blk));
    double dmin = or_f16_to_f64(rd16(blk + 2));
    const uint8_t *sc = blk + 4, *qs = blk + 16;
    for (int e = 0; e < 256; ++e) {
        int j = e / 32, S, M;
        q4k_scale_min(sc, j, &S, &M);
        uint8_t byte = qs[32 * (j / 2) + e % 32];
        int q = (j % 2 == 0) ? (byte & 15) : (byte >> 4);
        /* d*S*q and dmin*M are exact in fp64; one rounding to fp32. */
        out[e] = (float)(d * S * q - dmin * M);
    }
}

static void dq_q5_k(const uint8_t *blk, float *out)
{
    double d = or_f16_to_f64(rd16(blk));
    double dmin = or_f16_to_f64(rd16(blk + 2));
    const uint8_t *sc = blk + 4, *qh = blk + 16, *qs = blk + 48;
    for (int e = 0; e < 256; ++e) {
        int j = e / 32, l = e % 32, S, M;
        q4k_scale_min(sc, j, &S, &M);
        uint8_t byte = qs[32 * (j / 2) + l];
        int lo = (j % 2 == 0) ? (byte & 15) : (byte >> 4);
        int q = lo | (((qh[l] >> j) & 1) << 4);
        /* d*S*q (at most 22 bits) and dmin*M are exact; one rounding. */
        out[e] = (float)(d * S * q - dmin * M);
    }
}

static void dq_q6_k(const uint8_t *blk, float *out)
{
    const uint8_t *ql = blk, *qh = blk + 128;
    const int8_t *sc = (const int8_t *)(blk + 192);
    double d = or_f16_to_f64(rd16(blk + 208));
    for (int e = 0; e < 256; ++e) {
        int h = e / 128, r = e % 128, k = r / 32, l = r % 32;
        uint8_t lob = ql[64 * h + 32 * (k & 1) + l];
        int lo = (k < 2) ? (lob & 15) : (lob >> 4);
        int hi = (qh[32 * h + l] >> (2 * k)) & 3;
        int q = lo | (hi << 4);
        out[e] = (float)(d * sc[e / 16] * (q - 32));
    }
}

int or_dequant(int type, const uint8_t *blocks, int64_t n, float *out)
{
    int64_t be = or_block_elems(type), bb = or_block_bytes(type);
    if (be <= 0 || n < 0 || n % be != 0)
        return -1;
    for (int64_t b = 0; b < n / be; ++b) {
        const uint8_t *blk = blocks + b * bb;
        float *o = out + b * be;
        switch (type) {
        case OR_F32: memcpy(o, blk, 4); break;
        case OR_F16: o[0] = (float)or_f16_to_f64(rd16(blk)); break;
        case OR_Q8_0: dq_q8_0(blk, o); break;
        case OR_Q4_0: dq_q4_0(blk, o); break;
        case OR_Q4_K: dq_q4_k(blk, o); break;
        case OR_Q5_K: dq_q5_k(blk, o); break;
        case OR_Q6_K: dq_q6_k(blk, o); break;
        }
    }
    return 0;
}

/* ---- encoders --------------------------------------------------------------
 * Parity is defined on the packed bytes, so any encoder that emits
 * well-formed blocks within a stated error bound will do.  These are the
 * plainest ones with a provable bound (|x - decoded| <= step/2), computed in
 * fp64; "round" is half away from zero. */

static int q_q8_0(const float *x, uint8_t *blk)
{
    double a = 0;
    for (int e = 0; e < 32; ++e)
        a = fmax(a, fabs((double)x[e]));
    uint16_t dh = or_f64_to_f16_rne(a / 127.0);
    double d = or_f16_to_f64(dh);
    wr16(blk, dh);
    for (int e = 0; e < 32; ++e) {
        double q = (d == 0.0) ? 0.0 : round((double)x[e] / d);
        q = fmin(127.0, fmax(-127.0, q));
        blk[2 + e] = (uint8_t)(int8_t)q;
    }
    return 0;
}

static int q_q4_0(const float *x, uint8_t *blk)
{
    double a = 0;
    for (int e = 0; e < 32; ++e)
        a = fmax(a, fabs((double)x[e]));
    uint16_t dh = or_f64_to_f16_rne(a / 7.0);
    double d = or_f16_to_f64(dh);
    wr16(blk, dh);
    memset(blk + 2, 0, 16);
    for (int e = 0; e < 32; ++e) {
        double q = (d == 0.0) ? 0.0 : round((double)x[e] / d);
        int qi = (int)fmin(7.0, fmax(-8.0, q)) + 8;
        if (e < 16)
            blk[2 + e] |= (uint8_t)qi;
        else
            blk[2 + e - 16] |= (uint8_t)(qi << 4);
    }
    return 0;
}

/* Q4_K and Q5_K: the same steps, with codes of `levels` + 1 values (15 or
 * 31).  Returns the per-sub-block offsets o, steps d*S and the packed header
 * (d, dmin, scales) in blk[0..16). */
static void kq_header(const float *x, int levels, uint8_t *blk, double o[8], double step[8])
{
    double m[8], s[8], mmax = 0, smax = 0;
    int S[8], M[8];
    /* 1. Per sub-block offset: the negated minimum, clipped at 0; one shared
     *    fp16 dmin with 6-bit multipliers rounded up, so o_j >= m_j.        */
    for (int j = 0; j < 8; ++j) {
        double mn = 0;
        for (int i = 0; i < 32; ++i)
            mn = fmin(mn, (double)x[32 * j + i]);
        m[j] = -mn;
        mmax = fmax(mmax, m[j]);
    }
    uint16_t dminh = or_f64_to_f16_up(mmax / 63.0);
    double dmin = or_f16_to_f64(dminh);
    for (int j = 0; j < 8; ++j) {
        M[j] = (dmin == 0.0) ? 0 : (int)ceil(m[j] / dmin);
        o[j] = dmin * M[j];
    }
    /* 2. Per sub-block step covering [-o_j, max x] in `levels` steps; one
     *    shared fp16 d with 6-bit multipliers rounded up, so step_j >= s_j. */
    for (int j = 0; j < 8; ++j) {
        double mx = -o[j];
        for (int i = 0; i < 32; ++i)
            mx = fmax(mx, (double)x[32 * j + i]);
        s[j] = (mx + o[j]) / (double)levels;
        smax = fmax(smax, s[j]);
    }
    uint16_t dh = or_f64_to_f16_up(smax / 63.0);
    double d = or_f16_to_f64(dh);
    for (int j = 0; j < 8; ++j) {
        S[j] = (d == 0.0) ? 0 : (int)ceil(s[j] / d);
        step[j] = d * S[j];
    }
    wr16(blk, dh);
    wr16(blk + 2, dminh);
    uint8_t *b = blk + 4;
    memset(b, 0, 12);
    for (int j = 0; j < 4; ++j) {
        b[j] = (uint8_t)((S[j] & 63) | ((S[j + 4] >> 4) << 6));
        b[j + 4] = (uint8_t)((M[j] & 63) | ((M[j + 4] >> 4) << 6));
        b[j + 8] = (uint8_t)((S[j + 4] & 15) | ((M[j + 4] & 15) << 4));
    }
}

/* 3. Code of value x in sub-block j: round((x + o_j) / step_j) in [0, levels]. */
static int kq_code(double x, double o, double step, int levels)
{
    double q = (step == 0.0) ? 0.0 : round((x + o) / step);
    return (int)fmin((double)levels, fmax(0.0, q));
}

static int q_q4_k(const float *x, uint8_t *blk)
{
    double o[8], step[8];
    kq_header(x, 15, blk, o, step);
    uint8_t *qs = blk + 16;
    memset(qs, 0, 128);
    for (int j = 0; j < 8; ++j)
        for (int i = 0; i < 32; ++i) {
            int qi = kq_code((double)x[32 * j + i], o[j], step[j], 15);
            qs[32 * (j / 2) + i] |= (uint8_t)((j % 2 == 0) ? qi : (qi << 4));
        }
    return 0;
}

static int q_q5_k(const float *x, uint8_t *blk)
{
    double o[8], step[8];
    kq_header(x, 31, blk, o, step);
    uint8_t *qh = blk + 16, *qs = blk + 48;
    memset(qh, 0, 32);
    memset(qs, 0, 128);
    for (int j = 0; j < 8; ++j)
        for (int i = 0; i < 32; ++i) {
            int qi = kq_code((double)x[32 * j + i], o[j], step[j], 31);
            qs[32 * (j / 2) + i] |= (uint8_t)((j % 2 == 0) ? (qi & 15) : ((qi & 15) << 4));
            qh[i] |= (uint8_t)((qi >> 4) << j);
        }
    return 0;
}

static int q_q6_k(const float *x, uint8_t *blk)
{
    double s[16], smax = 0;
    int S[16];
    for (int j = 0; j < 16; ++j) {
        double a = 0;
        for (int i = 0; i < 16; ++i)
            a = fmax(a, fabs((double)x[16 * j + i]));
        s[j] = a / 31.0;
        smax = fmax(smax, s[j]);
    }
    uint16_t dh = or_f64_to_f16_up(smax / 127.0);
    double d = or_f16_to_f64(dh);
    for (int j = 0; j < 16; ++j)
        S[j] = (d == 0.0) ? 0 : (int)ceil(s[j] / d);

    uint8_t *ql = blk, *qh = blk + 128;
    memset(blk, 0, 210);
    for (int j = 0; j < 16; ++j)
        blk[192 + j] = (uint8_t)(int8_t)S[j];
    wr16(blk + 208, dh);
    for (int e = 0; e < 256; ++e) {
        double step = d * S[e / 16];
        double q = (step == 0.0) ? 0.0 : round((double)x[e] / step);
        int qi = (int)fmin(31.0, fmax(-32.0, q)) + 32;
        int h = e / 128, r = e % 128, k = r / 32, l = r % 32;
        uint8_t *lob = &ql[64 * h + 32 * (k & 1) + l];
        *lob |= (uint8_t)((k < 2) ? (qi & 15) : ((qi & 15) << 4));
        qh[32 * h + l] |= (uint8_t)(((qi >> 4) & 3) << (2 * k));
    }
    return 0;
}

int or_quantize(int type, const float *x, int64_t n, uint8_t *blocks)
{
    int64_t be = or_block_elems(type), bb = or_block_bytes(type);
    if (be <= 0 || n < 0 || n % be != 0)
        return -1;
    for (int64_t i = 0; i < n; ++i)
        if (!isfinite(x[i]))
            return -2;
    for (int64_t b = 0; b < n / be; ++b) {
        const float *xb = x + b * be;
        uint8_t *blk = blocks + b * bb;
        switch (type) {
        case OR_F32: memcpy(blk, xb, 4); break;
        case OR_F16: wr16(blk, or_f64_to_f16_rne(xb[0])); break;
        case OR_Q8_0: q_q8_0(xb, blk); break;
        case OR_Q4_0: q_q4_0(xb, blk); break;
        case OR_Q4_K: q_q4_k(xb, blk); break;
        case OR_Q5_K: q_q5_k(xb, blk); break;
        case OR_Q6_K: q_q6_k(xb, blk); break;
        }
    }
    return 0;
}

int or_pack_q8_0(const uint16_t *d_bits, const int8_t *qs, int64_t nblocks, uint8_t *blocks)
{
    if (nblocks < 0)
        return -1;
    for (int64_t b = 0; b < nblocks; ++b) {
        wr16(blocks + 34 * b, d_bits[b]);
        memcpy(blocks + 34 * b + 2, qs + 32 * b, 32);
    }
    return 0;
}
