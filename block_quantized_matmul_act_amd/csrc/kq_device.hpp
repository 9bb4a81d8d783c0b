// kq_device.hpp -- device helpers shared by the kq kernels (gfx950 only).
//
// Matrix-core operand conventions used throughout (CDNA3/CDNA4 MFMA):
//   v_mfma_i32_32x32x32_i8: each lane supplies 16 int8 of A and 16 of B.
//   Lane l supplies row (l % 32) of A and column (l % 32) of B; both take
//   the same k-group (l / 32), so any assignment of K indices to (k-group,
//   byte) that is identical on the A and B side gives the same contraction.
//   The 32x32 int32/fp32 result is 16 registers per lane: register r of
//   lane l holds row 8*(r/4) + 4*(l/32) + (r%4), column l % 32.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace kq {

#define KQ_INLINE __attribute__((always_inline))

template <int V>
using IC = std::integral_constant<int, V>;

// f(IC<B>{}), f(IC<B+1>{}), ..., f(IC<E-1>{})
template <int B, int E, class F>
__device__ __forceinline__ void static_for(F &&f) {
    if constexpr (B < E) {
        f(IC<B>{});
        static_for<B + 1, E>(f);
    }
}

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef unsigned short v2u16 __attribute__((ext_vector_type(2)));
typedef short v2i16 __attribute__((ext_vector_type(2)));
typedef unsigned int v2u __attribute__((ext_vector_type(2)));
typedef unsigned int v3u __attribute__((ext_vector_type(3)));

// Row of the 32x32 MFMA result held by register r of lane l.
__device__ __forceinline__ int mfma32_row(int r, int lane) {
    return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
}

__device__ __forceinline__ float f16_bits_to_f32(uint32_t bits) {
    _Float16 h = __builtin_bit_cast(_Float16, (unsigned short)(bits & 0xFFFF));
    return (float)h;
}

// Four bytes, each < 16 (so each product < 128), times an unsigned scale s < 8:
// two packed 16-bit multiplies keep every byte product inside its own byte.
__device__ __forceinline__ uint32_t bytes_times_small(uint32_t four_bytes, uint32_t s) {
    v2u16 a = __builtin_bit_cast(v2u16, four_bytes);
    v2u16 b = {(unsigned short)s, (unsigned short)s};
    return __builtin_bit_cast(uint32_t, (v2u16)(a * b));
}

// Select bytes of {hi:lo} into a dword (v_perm_b32 semantics: selector byte
// values 0..3 pick lo bytes, 4..7 pick hi bytes, 12 gives 0x00).
__device__ __forceinline__ uint32_t perm_b32(uint32_t hi, uint32_t lo, uint32_t sel) {
    return __builtin_amdgcn_perm(hi, lo, sel);
}

// fp32 -> bf16 hi/lo pair so that hi + lo carries ~16 significant bits.
__device__ __forceinline__ void split_bf16(float x, __bf16 &hi, __bf16 &lo) {
    hi = (__bf16)x;
    lo = (__bf16)(x - (float)hi);
}

__device__ __forceinline__ v16i mfma_i8_32x32x32(v4i a, v4i b, v16i c) {
    return __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ v16i mfma_i8_32x32x16(long a, long b, v16i c) {
    return __builtin_amdgcn_mfma_i32_32x32x16_i8(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ v16f mfma_bf16_32x32x16(v8bf a, v8bf b, v16f c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// ---------------------------------------------------------------------------
// Q4_K loader pieces.
//
// The twelve scale bytes are a little-endian 96-bit integer; field f lives in
// bits [6f, 6f+6).  w0..w2 are its three 32-bit words.
__device__ __forceinline__ void q4k_fields(uint32_t w0, uint32_t w1, uint32_t w2, int f_lo,
                                           int count, uint32_t *sc, uint32_t *mn) {
    uint64_t lo = (uint64_t)w0 | ((uint64_t)w1 << 32);  // bits 0..63
    uint64_t hi = (uint64_t)w1 | ((uint64_t)w2 << 32);  // bits 32..95
#pragma unroll
    for (int i = 0; i < count; ++i) {
        int j = f_lo + i;
        sc[i] = (uint32_t)(lo >> (6 * j)) & 63u;
        mn[i] = (uint32_t)(hi >> (16 + 6 * j)) & 63u;
    }
}

// Operand split of the Q4_K product sc*q (up to 945, too wide for int8):
// sc = 8*sh + sl with sh, sl in [0,7], so sh*q and sl*q are both <= 105 and
// sum_k sc*q*a = 8*sum_k (sh*q)*a + sum_k (sl*q)*a.
__device__ __forceinline__ void q4k_digits(uint32_t nib4, uint32_t sc, uint32_t &dh,
                                           uint32_t &dl) {
    dh = bytes_times_small(nib4, sc >> 3);
    dl = bytes_times_small(nib4, sc & 7u);
}

// ---------------------------------------------------------------------------
// Q6_K loader pieces.
//
// q dword (4 weights, bytes in [0,63]) and the sub-block scale sc (int8) ->
// two int8 digit dwords of W = sc*(q-32) in [-4096, 4096]: W = 64*h + l with
// l in [0,63], h in [-64,64].  Products are formed in packed 16-bit lanes as
// 4*W = 256*h + 4*l (|4W| <= 16384 fits a signed 16-bit lane): the high byte
// of each lane is h in two's complement and the low byte 4*l, a multiple of
// 4, so the packed low bytes shifted right by 2 are the four l digits (the
// bits that cross into a byte from its neighbour are zero).
__device__ __forceinline__ void q6k_digits(uint32_t q4, int sc, uint32_t &dh, uint32_t &dl) {
    const uint32_t qe = perm_b32(0u, q4, 0x0c020c00u);   // bytes 0,2 -> 16-bit lanes
    const uint32_t qo = perm_b32(0u, q4, 0x0c030c01u);   // bytes 1,3 -> 16-bit lanes
    const v2i16 s4 = {(short)(4 * sc), (short)(4 * sc)};
    const v2i16 off = {(short)(-128 * sc), (short)(-128 * sc)};
    const uint32_t we = __builtin_bit_cast(uint32_t, (v2i16)(__builtin_bit_cast(v2i16, qe) * s4 + off));
    const uint32_t wo = __builtin_bit_cast(uint32_t, (v2i16)(__builtin_bit_cast(v2i16, qo) * s4 + off));
    // byte order e0, o0, e1, o1: high bytes for h, low bytes for 4*l
    dh = perm_b32(wo, we, 0x07030501u);
    dl = perm_b32(wo, we, 0x06020400u) >> 2;
}

// ---------------------------------------------------------------------------
// Ternary loader pieces.
//
// A byte v <= 242 holds base-3 digits e_0..e_4 (v = sum e_p 3^p).  With the
// 8-bit fixed-point value f = ceil(256*v/243), the fractional part of
// v*3^j/243 sits in the low byte of f*3^j, and
//     e_(4-j) = ((f*3^j mod 256) * 3) >> 8        for j = 0..4,
// exact because 3^5 = 243 < 256 leaves enough guard bits for the rounding of
// f.  Every digit costs the same instructions, whatever the byte holds.
__device__ __forceinline__ uint32_t tq_fixed(uint32_t v) {
    return (v * 256u + 242u) / 243u;
}

// Four trit bytes (as int8 -1/0/+1) from the digits at position p of four
// fixed-point values f0..f3 (each < 256).
template <int P>
__device__ __forceinline__ uint32_t tq_digit(uint32_t f) {
    constexpr uint32_t pow3 = P == 4 ? 1u : P == 3 ? 3u : P == 2 ? 9u : P == 1 ? 27u : 81u;
    return ((((f * pow3) & 255u) * 3u) >> 8);
}

// Digit e in {0,1,2} per byte -> trit e-1 as an int8 byte, for four bytes at
// once: adding 0x7F to each byte never carries (e <= 2), and flipping bit 7
// gives (e - 1) mod 256.
__device__ __forceinline__ uint32_t digits_to_trits(uint32_t e4) {
    return (e4 + 0x7F7F7F7Fu) ^ 0x80808080u;
}

// Ternary decode table entry for byte v: its five base-3 digits minus one as
// int8 in bytes 0..4, zero bytes 5..7.  Digit p is floor(v / 3^p) mod 3, so
// bytes above 242 decode exactly as the plain digit definition gives.
__device__ __forceinline__ void tq_lut_entry(uint32_t v, uint32_t &lo, uint32_t &hi) {
    uint32_t t[5];
#pragma unroll
    for (int p = 0; p < 5; ++p) {
        t[p] = (uint32_t)(int8_t)((int)(v % 3u) - 1) & 0xFFu;
        v /= 3u;
    }
    lo = t[0] | (t[1] << 8) | (t[2] << 16) | (t[3] << 24);
    hi = t[4];
}

}  // namespace kq
