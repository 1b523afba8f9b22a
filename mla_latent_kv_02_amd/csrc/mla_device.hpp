// Device-side building blocks shared by the libmla kernels (gfx950 / CDNA4).
//
// - vector types for the bf16 MFMA operands,
// - round-to-nearest-even fp32 -> bf16, and the two-term bf16 split of softmax weights,
// - the element-wise dequantisation of INT4 / INT2 codes that every decode kernel's
//   in-loop dequant routine (QuantProducer::dequant_task, rows::QuantStage) is built from.
//
// Dequantisation (QuantMLA: unpack and dequantise inside attention): a code q
// of group (scale s, integer zero-point z) becomes RNE_bf16((q - z) * s).  With
// |q - z| <= 15 and an fp16 s the product has at most 15 significant bits, so
// fma(q, s, -(z*s)) returns it exactly in fp32 (z*s is exact as well); the one
// rounding is the final fp32 -> bf16 conversion.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace mla {

typedef __bf16 bf16_t;
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short i16x4;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4;

constexpr int BLOCK_TOKENS = 64;

// Cache formats (values of MLA_FMT_*).
constexpr int FMT_F32 = 0, FMT_BF16 = 1, FMT_INT4 = 2, FMT_INT2 = 3;

// fp32 -> bf16, round to nearest even (v_cvt_pk_bf16_f32 on gfx950)
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)f);
}

// Two floats -> two fp16 (round to nearest even) in one word, the first in the low half.
__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
  const _Float16 a = (_Float16)lo, b = (_Float16)hi;
  return (uint32_t)__builtin_bit_cast(uint16_t, a) | ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2_t;
  const bf16x2_t v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// Softmax weights for the P.V MFMA as two bf16 terms: hi = RNE_bf16(p) and lo = RNE_bf16(p - hi),
// both packed in pairs (p0 in the low half).  p - hi is exact in fp32, so hi + lo keeps about 16
// significant bits of p; one bf16 P (8 bits) moves o_lat by up to ~2^-9 relative, as much as the
// whole error budget of an fp32-accumulated decode.
__device__ __forceinline__ void split_pair(float p0, float p1, uint32_t& hi, uint32_t& lo) {
  hi = pack_bf16x2(p0, p1);
  lo = pack_bf16x2(p0 - __uint_as_float(hi << 16), p1 - __uint_as_float(hi & 0xFFFF0000u));
}

__device__ __forceinline__ float half_bits_to_f32(uint32_t h) {
  _Float16 v = __builtin_bit_cast(_Float16, (uint16_t)h);
  return (float)v;
}

// Byte b of x as a float (v_cvt_f32_ubyte0..3).  The compiler turns (x >> 8b) & 0xFF into a
// bit-field extract plus a byte-0 conversion; the byte-select forms save the extract.
template <int B>
__device__ __forceinline__ float ubyte_f32(uint32_t x) {
  float r;
  if constexpr (B == 0) asm("v_cvt_f32_ubyte0 %0, %1" : "=v"(r) : "v"(x));
  else if constexpr (B == 1) asm("v_cvt_f32_ubyte1 %0, %1" : "=v"(r) : "v"(x));
  else if constexpr (B == 2) asm("v_cvt_f32_ubyte2 %0, %1" : "=v"(r) : "v"(x));
  else asm("v_cvt_f32_ubyte3 %0, %1" : "=v"(r) : "v"(x));
  return r;
}

// Eight INT4 codes of one 32-bit word (element e at bits 4e..4e+3) -> 8 bf16 (as 4 words).
__device__ __forceinline__ u32x4 dequant_int4x8(uint32_t w, float s, float zs) {
  uint32_t lo = w & 0x0F0F0F0Fu;          // elements 0, 2, 4, 6 in bytes 0..3
  uint32_t hi = (w >> 4) & 0x0F0F0F0Fu;   // elements 1, 3, 5, 7
  u32x4 r;
  r[0] = pack_bf16x2(__builtin_fmaf(ubyte_f32<0>(lo), s, -zs), __builtin_fmaf(ubyte_f32<0>(hi), s, -zs));
  r[1] = pack_bf16x2(__builtin_fmaf(ubyte_f32<1>(lo), s, -zs), __builtin_fmaf(ubyte_f32<1>(hi), s, -zs));
  r[2] = pack_bf16x2(__builtin_fmaf(ubyte_f32<2>(lo), s, -zs), __builtin_fmaf(ubyte_f32<2>(hi), s, -zs));
  r[3] = pack_bf16x2(__builtin_fmaf(ubyte_f32<3>(lo), s, -zs), __builtin_fmaf(ubyte_f32<3>(hi), s, -zs));
  return r;
}

// INT2: a group has only four code values, so its four dequantised bf16 values are computed
// once (the same fma + RNE conversion per value) into an 8-byte table {t_hi : t_lo}, code c at
// bytes 2c, 2c + 1, and every output pair is a byte permute of that table.
__device__ __forceinline__ void int2_table(float s, float zs, uint32_t& t_lo, uint32_t& t_hi) {
  t_lo = pack_bf16x2(__builtin_fmaf(0.f, s, -zs), __builtin_fmaf(1.f, s, -zs));
  t_hi = pack_bf16x2(__builtin_fmaf(2.f, s, -zs), __builtin_fmaf(3.f, s, -zs));
}

// Sixteen INT2 codes of a 32-bit word (element e at bits 2e..2e+1) -> 16 bf16 (elements 0..7 in
// lo, 8..15 in hi) through the group's table.  Masking w >> 2j with 0x03030303 puts element
// 4b + j in byte b of m_j; for the pair (4b + j, 4b + j + 1), j even, one permute gathers
// (c, c, c', c') from m_j and m_j+1, 2x + 0x01000100 turns it into the byte selector
// (2c, 2c + 1, 2c', 2c' + 1), and a second permute reads the two bf16 values from the table.
__device__ __forceinline__ void dequant_int2x16(uint32_t w, uint32_t t_lo, uint32_t t_hi, u32x4& lo, u32x4& hi) {
  const uint32_t m0 = w & 0x03030303u, m1 = (w >> 2) & 0x03030303u;
  const uint32_t m2 = (w >> 4) & 0x03030303u, m3 = (w >> 6) & 0x03030303u;
  auto pair = [&](uint32_t ma, uint32_t mb, int b) {
    // byte select: bytes 0..3 of the permute source are its second operand, 4..7 its first
    const uint32_t gsel = (uint32_t)b * 0x0101u + (uint32_t)(4 + b) * 0x01010000u;
    const uint32_t x = __builtin_amdgcn_perm(mb, ma, gsel);
    return __builtin_amdgcn_perm(t_hi, t_lo, (x << 1) + 0x01000100u);
  };
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    u32x4& r = b < 2 ? lo : hi;
    const int k = (b & 1) * 2;   // elements 4b .. 4b + 3 -> words k, k + 1
    r[k] = pair(m0, m1, b);
    r[k + 1] = pair(m2, m3, b);
  }
}

// (scale, zero) fp16 pair packed in a 32-bit word -> (s, z*s) as fp32.
__device__ __forceinline__ void scale_zero(uint32_t sz, float& s, float& zs) {
  s = half_bits_to_f32(sz & 0xFFFFu);
  float z = half_bits_to_f32(sz >> 16);
  zs = z * s;  // exact: z is a small integer, s has 11 significant bits
}

// Byte offsets of the four planes of a quantised block.
struct QuantPlanes {
  int32_t lc, ls, rc, rs;
};

}  // namespace mla
