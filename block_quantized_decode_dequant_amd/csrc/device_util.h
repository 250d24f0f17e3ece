// device_util.h -- small device-side helpers shared by the HIP kernel files.
#pragma once

#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>

#include <cstdint>

namespace nt {

// 128/96/64/32-bit loads that need only 4-byte alignment (the kernels build
// these addresses from 2-byte-aligned block starts rounded down to a word).
typedef uint32_t u32x4 __attribute__((ext_vector_type(4), aligned(4)));
typedef uint32_t u32x3 __attribute__((ext_vector_type(3), aligned(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2), aligned(4)));

__device__ __forceinline__ u32x4 ld4(const uint8_t *p) { return *reinterpret_cast<const u32x4 *>(p); }
__device__ __forceinline__ u32x3 ld3(const uint8_t *p) { return *reinterpret_cast<const u32x3 *>(p); }
__device__ __forceinline__ uint32_t ld1(const uint8_t *p) { return *reinterpret_cast<const uint32_t *>(p); }

// Streaming (non-temporal) variants for weights that are read exactly once.
__device__ __forceinline__ u32x4 ld4_nt(const uint8_t *p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
}
__device__ __forceinline__ uint32_t ld1_nt(const uint8_t *p) {
    return __builtin_nontemporal_load(reinterpret_cast<const uint32_t *>(p));
}

// IEEE binary16 bits -> fp32 (exact, subnormals included).
__device__ __forceinline__ float h2f(uint32_t bits16) {
    return __half2float(__ushort_as_half(static_cast<unsigned short>(bits16 & 0xffffu)));
}

// Bytes [sh, sh+4) of the 8-byte value hi:lo, for sh in {0, 2}: v_perm_b32
// with a per-lane selector (selector bytes 0-3 pick lo, 4-7 pick hi).
__device__ __forceinline__ uint32_t shift_sel(uint32_t sh) {
    return sh ? 0x05040302u : 0x03020100u;
}
__device__ __forceinline__ uint32_t funnel(uint32_t hi, uint32_t lo, uint32_t sel) {
    return __builtin_amdgcn_perm(hi, lo, sel);
}

// fp32 value of byte k of w (v_cvt_f32_ubyte{k}).
template <int K>
__device__ __forceinline__ float ubyte(uint32_t w) {
    return static_cast<float>((w >> (8 * K)) & 0xffu);
}

// Sum over the 64 lanes of a wavefront; every lane gets the total.
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
    return v;
}

// DPP-based sum over the 64 lanes: the total lands in lane 63.  Within each
// row of 16 lanes: quad swaps (xor 1, xor 2), half-row and row mirrors; then
// row_bcast:15 / row_bcast:31 carry row totals upward (gfx9 DPP).
template <int CTRL, int ROW_MASK = 0xf>
__device__ __forceinline__ float dpp(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, ROW_MASK, 0xf, false));
}
__device__ __forceinline__ float wave_sum_to_lane63(float v) {
    v += dpp<0xb1>(v);          // quad_perm [1,0,3,2]
    v += dpp<0x4e>(v);          // quad_perm [2,3,0,1]
    v += dpp<0x141>(v);         // row_half_mirror
    v += dpp<0x140>(v);         // row_mirror: every lane holds its row's sum
    v += dpp<0x142, 0xa>(v);    // row_bcast:15 into rows 1 and 3
    v += dpp<0x143, 0xc>(v);    // row_bcast:31 into rows 2 and 3
    return v;
}

// Hide a value from the optimizer (no instruction is emitted), e.g. so a
// masked word still converts with v_cvt_f32_ubyteN instead of a bit-field
// extract plus a conversion, or so a constant lives in a VGPR and can feed
// VOP3 instructions that take no literals.
__device__ __forceinline__ uint32_t opaque(uint32_t v) {
    asm volatile("" : "+v"(v));
    return v;
}

// Low / high fp16 half of a word as fp32 (folds into v_fma_mix_f32 operands).
__device__ __forceinline__ float h_lo(uint32_t w) { return __half2float(__ushort_as_half(static_cast<unsigned short>(w))); }
__device__ __forceinline__ float h_hi(uint32_t w) { return __half2float(__ushort_as_half(static_cast<unsigned short>(w >> 16))); }

// DPP-based max over the 64 lanes: the result lands in lane 63.
template <int CTRL, int ROW_MASK = 0xf>
__device__ __forceinline__ float dpp_keep(float v) {
    // lanes the row mask leaves out keep their own value (bound_ctrl off, old = v)
    return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(v), __float_as_int(v), CTRL, ROW_MASK, 0xf, false));
}
__device__ __forceinline__ float wave_max_to_lane63(float v) {
    v = fmaxf(v, dpp_keep<0xb1>(v));
    v = fmaxf(v, dpp_keep<0x4e>(v));
    v = fmaxf(v, dpp_keep<0x141>(v));
    v = fmaxf(v, dpp_keep<0x140>(v));
    v = fmaxf(v, dpp_keep<0x142, 0xa>(v));
    v = fmaxf(v, dpp_keep<0x143, 0xc>(v));
    return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m, 64));
    return v;
}

// ---- explicit memory waits and asynchronous copies into LDS ----------------
// s_waitcnt immediate that waits until at most n vector-memory operations are
// outstanding (gfx9 encoding: vmcnt bits 3:0 and 15:14; expcnt and lgkmcnt
// fields at their maxima, i.e. no wait on them).
constexpr int vmcnt_imm(int n) { return (n & 15) | (7 << 4) | (15 << 8) | ((n >> 4) << 14); }

typedef __attribute__((address_space(3))) void lds_void;
typedef const __attribute__((address_space(1))) void gbl_void;

// One global_load_lds of V bytes per lane: lane i reads base + off (off is
// per lane, base wave-uniform) and its bytes land at LDS address lds + V*i
// (lds wave-uniform, through M0).  Written as inline assembly on purpose: the
// compiler then does not track these LDS writes, so it adds no conservative
// "wait for every outstanding load" before unrelated LDS reads; every read
// of a ring stage is preceded by an explicit s_waitcnt on the loads that fill
// it.  The "memory" clobber keeps the copies ordered against other memory
// operations in program order.  NT (16-byte copies): the non-temporal cache
// policy, for data read once per token (weights, K/V rows), so the lines it
// brings in do not push out the activations and outputs that the next
// kernels read again.
template <int V, bool NT = false>
__device__ __forceinline__ void dma(const uint8_t *base, uint32_t off, uint32_t lds) {
    int m0_out;   // M0 is declared written (an output), so no value of the compiler's lives in it across the copy
    if constexpr (V == 16 && NT)
        asm volatile("s_mov_b32 m0, %3\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2 nt"
                     : "={m0}"(m0_out) : "v"(off), "s"(base), "s"(lds) : "memory");
    else if constexpr (V == 16)
        asm volatile("s_mov_b32 m0, %3\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
                     : "={m0}"(m0_out) : "v"(off), "s"(base), "s"(lds) : "memory");
    else
        asm volatile("s_mov_b32 m0, %3\n\ts_nop 0\n\tglobal_load_lds_dword %1, %2"
                     : "={m0}"(m0_out) : "v"(off), "s"(base), "s"(lds) : "memory");
    (void)m0_out;
}

// LDS address (32-bit, as M0 takes it) of a wave-uniform LDS location.
__device__ __forceinline__ uint32_t lds_addr(const void *p) {
    return __builtin_amdgcn_readfirstlane(uint32_t(uintptr_t((lds_void *)p)));
}

// s_waitcnt immediate that waits for all LDS operations (lgkmcnt 0) only.
constexpr int kLgkm0 = 15 | (7 << 4) | (0 << 8) | (3 << 14);

}  // namespace nt
