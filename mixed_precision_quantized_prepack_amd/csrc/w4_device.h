// Device helpers for the gfx950 4-bit-weight GEMM kernels: operand
// expansion of prepacked 4-bit words, MFMA wrappers and scalar conversions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "w4.h"
#include "w4_internal.h"

namespace w4 {

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x8 __attribute__((ext_vector_type(8)));

// ---------------------------------------------------------------------------
// 4-bit -> 8-bit expansion for the int8 MFMA (PB-v1, I8 operand class).
//
// A packed word holds k-offsets 0..3 in the low nibbles of its four bytes and
// 4..7 in the high nibbles.  Moving each nibble into the high half of its byte
// turns a two's-complement int4 w into the int8 16*w exactly, so the int32
// accumulator holds 16 * sum(a*w); the factor is removed (exactly: a power of
// two) when the scale is applied.  Three VALU ops per 8 weights.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void expand_i8x16(uint32_t w, uint32_t& k0123, uint32_t& k4567) {
  k0123 = (w << 4) & 0xF0F0F0F0u;
  k4567 = w & 0xF0F0F0F0u;
}

// ---------------------------------------------------------------------------
// 4-bit -> fp8 e4m3fn expansion (I8 operand class).
//
// The sixteen int4 values have no arithmetic relation to their e4m3 codes, so
// this is a 16-entry table lookup done with the byte-permute instruction: the
// low three bits of each nibble index two 8-byte tables (values 0..7 and
// -8..-1) and a third permute picks, byte by byte, one of the two results by
// bit 3.  The same routine with other tables gives any other 8-bit target.
//   e4m3fn codes:   0:00 1:38 2:40 3:44 4:48 5:4A 6:4C 7:4E
//                  -8:D0 -7:CE -6:CC -5:CA -4:C8 -3:C4 -2:C0 -1:B8
// v_perm_b32(hi, lo, sel): selector byte 0..3 picks a byte of lo, 4..7 of hi.
// ---------------------------------------------------------------------------
constexpr uint32_t kFp8PosLo = 0x44403800u;
constexpr uint32_t kFp8PosHi = 0x4E4C4A48u;
constexpr uint32_t kFp8NegLo = 0xCACCCED0u;
constexpr uint32_t kFp8NegHi = 0xB8C0C4C8u;

// A constant the compiler must keep in a scalar (vector) register: the
// three-source VALU encodings of gfx950 take no literal, so (x & c1) | c2
// with both constants as literals costs two instructions; with c1 in a
// scalar and c2 in a vector register it is one v_and_or_b32.  The empty asm
// hides the constant from the compiler; it still sets the two registers once
// per loop iteration (one scalar and one vector move), not once per word.
__device__ __forceinline__ uint32_t in_sgpr(uint32_t v) {
  uint32_t r;
  asm("" : "=s"(r) : "0"(v));
  return r;
}
__device__ __forceinline__ uint32_t in_vgpr(uint32_t v) {
  uint32_t r;
  asm("" : "=v"(r) : "0"(v));
  return r;
}

__device__ __forceinline__ void expand_fp8(uint32_t w, uint32_t& k0123, uint32_t& k4567) {
  // table lookups on the low three bits of each nibble
  const uint32_t w4 = w >> 4;
  const uint32_t sel_lo = w & 0x07070707u;
  const uint32_t sel_hi = w4 & 0x07070707u;
  const uint32_t p_lo = __builtin_amdgcn_perm(kFp8PosHi, kFp8PosLo, sel_lo);
  const uint32_t n_lo = __builtin_amdgcn_perm(kFp8NegHi, kFp8NegLo, sel_lo);
  const uint32_t p_hi = __builtin_amdgcn_perm(kFp8PosHi, kFp8PosLo, sel_hi);
  const uint32_t n_hi = __builtin_amdgcn_perm(kFp8NegHi, kFp8NegLo, sel_hi);
  // per byte, keep byte i of the positive result (selector i) or of the
  // negative one (selector i + 4): bit 3 of the nibble moved to bit 2
  const uint32_t bit2 = in_sgpr(0x04040404u);
  const uint32_t ident = in_vgpr(0x03020100u);
  const uint32_t pick_lo = ((w >> 1) & bit2) | ident;
  const uint32_t pick_hi = ((w4 >> 1) & bit2) | ident;
  k0123 = __builtin_amdgcn_perm(n_lo, p_lo, pick_lo);
  k4567 = __builtin_amdgcn_perm(n_hi, p_hi, pick_hi);
}

// ---------------------------------------------------------------------------
// 4-bit -> fp16 / bf16 expansion (F16 operand class, ExLlama pair order).
//
// (w >> 4i) & 0x000F000F yields the codes of k = 2i (low half) and 2i+1
// (high half).  OR-ing the exponent of 1024 (fp16, 0x6400) or 128 (bf16,
// 0x4300) gives the exact values 1024 + c / 128 + c.
// ---------------------------------------------------------------------------
template <int OP>
__device__ __forceinline__ void expand_f16class(uint32_t w, uint32_t out[4]) {
  constexpr uint32_t kMagic = (OP == OP_F16) ? 0x64006400u : 0x43004300u;
  out[0] = (w & 0x000F000Fu) | kMagic;
  out[1] = ((w >> 4) & 0x000F000Fu) | kMagic;
  out[2] = ((w >> 8) & 0x000F000Fu) | kMagic;
  out[3] = ((w >> 12) & 0x000F000Fu) | kMagic;
}

__device__ __forceinline__ uint32_t f16x2_add(uint32_t a, f16x2 b) {
  f16x2 r = __builtin_bit_cast(f16x2, a) + b;
  return __builtin_bit_cast(uint32_t, r);
}

// ---------------------------------------------------------------------------
// MFMA wrappers.  Operand A carries 16 weight rows (n), operand B 16
// activation rows (m); lane l supplies row l%16 of its operand.  A and B use
// the same assignment of k to (lane group, register position), so feeding both
// from the same logical k-set computes a correct dot product.  Result: lane l,
// element i holds D[n = 4*(l/16) + i][m = l%16].
// ---------------------------------------------------------------------------
__device__ __forceinline__ i32x4 mma_i8(u32x4 a, u32x4 b, i32x4 c) {
  return __builtin_amdgcn_mfma_i32_16x16x64_i8(__builtin_bit_cast(i32x4, a),
                                               __builtin_bit_cast(i32x4, b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma_fp8(u32x8 a, u32x8 b, f32x4 c) {
  // e4m3 x e4m3 (format code 0 for both) with unit block scales (E8M0 127 = 2^0)
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
      __builtin_bit_cast(i32x8, a), __builtin_bit_cast(i32x8, b), c, 0, 0, 0, 127, 0, 127);
}
__device__ __forceinline__ f32x4 mma_f16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma_bf16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// ---------------------------------------------------------------------------
// Scalar conversions.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float f16_bits_to_f32(uint32_t b) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)b);
}
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

__device__ __forceinline__ uint16_t f32_to_f16_bits(float f) {
  return __builtin_bit_cast(uint16_t, (_Float16)f);  // v_cvt_f16_f32, round to nearest even
}
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  // round to nearest even on the 16 dropped bits (finite inputs)
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__device__ __forceinline__ float load_as_f32(const void* p, int dtype, int64_t i) {
  if (dtype == W4_F32) return static_cast<const float*>(p)[i];
  const uint32_t b = static_cast<const uint16_t*>(p)[i];
  return dtype == W4_F16 ? f16_bits_to_f32(b) : bf16_bits_to_f32(b);
}

// ---------------------------------------------------------------------------
// Per-token quantisation of 16-byte chunks (8 fp16 / bf16 elements), shared
// by the quantisation kernels and the small-M GEMM's fused variant.
//
// Quotients x / s must be the correctly rounded fp32 division.  They are
// formed from one correctly rounded reciprocal per row, y = RN(1/s):
// q = RN(x * y), the exact residual r = fma(-q, s, x), and RN(q + r * y), which
// equals RN(x / s) by Markstein's theorem (y within half an ulp of 1/s, q
// within one ulp of x/s, r exact; no overflow or underflow).  Rows whose scale
// is too small for that (bf16 inputs near the bottom of the exponent range)
// use the plain division.
// ---------------------------------------------------------------------------
template <int XT>
__device__ __forceinline__ float elem(const uint4& v, int j) {
  const uint32_t w = (j < 2) ? v.x : (j < 4) ? v.y : (j < 6) ? v.z : v.w;
  const uint32_t b = (j & 1) ? (w >> 16) : (w & 0xFFFFu);
  return XT == W4_F16 ? f16_bits_to_f32(b) : bf16_bits_to_f32(b);
}

template <int XT>
__device__ __forceinline__ float chunk_absmax(float m, const uint4& v) {
#pragma unroll
  for (int j = 0; j < 8; ++j) m = fmaxf(m, fabsf(elem<XT>(v, j)));
  return m;
}

// correctly rounded x / s given y = RN(1 / s) (see above).  The sum q + r*y
// of a zero quotient is +0 even for x = -0, so the sign is taken from x (with
// s > 0 the quotient always has the sign of x).
__device__ __forceinline__ float div_rn(float x, float s, float y) {
  const float q = x * y;
  const float r = fmaf(-q, s, x);
  return copysignf(fmaf(r, y, q), x);
}

template <int XT, int QT, bool FAST>
__device__ __forceinline__ uint2 quant_chunk(const uint4& v, float s, float y) {
  uint32_t out[2];
  if (QT == W4_I8) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      uint32_t word = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float x = elem<XT>(v, 4 * h + j);
        float q = rintf(FAST ? div_rn(x, s, y) : x / s);
        q = fminf(fmaxf(q, -127.0f), 127.0f);
        word |= ((uint32_t)(int)q & 0xFFu) << (8 * j);
      }
      out[h] = word;
    }
  } else {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      float q[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float x = elem<XT>(v, 4 * h + j);
        q[j] = fminf(fmaxf(FAST ? div_rn(x, s, y) : x / s, -448.0f), 448.0f);
      }
      int word = __builtin_amdgcn_cvt_pk_fp8_f32(q[0], q[1], 0, false);
      word = __builtin_amdgcn_cvt_pk_fp8_f32(q[2], q[3], word, true);
      out[h] = (uint32_t)word;
    }
  }
  return make_uint2(out[0], out[1]);
}

}  // namespace w4
