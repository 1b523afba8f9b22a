// Device-side building blocks shared by the libmla kernels (gfx950 / CDNA4).
//
// - vector types for the bf16 MFMA operands,
// - round-to-nearest-even fp32 -> bf16,
// - the cache-tile reader: loads one 64-token block of a paged cache into
//   registers (bf16 rows, or INT4/INT2 codes with their fp16 scale/zero) and
//   later emits it as bf16 8-element pieces, dequantising codes on the way.
//   The decode kernel and the mla_dequant_blocks kernel both use this reader,
//   so what the debug entry point returns is exactly what attention consumes.
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

// --------------------------------------------------------------------------------------
// Tile reader.  NT threads cooperate on one 64-token block of d_c = 512, d_r = 64.
// load(): issue the global loads into registers (tokens >= valid are not read).
// emit(f): call f(token, col8, u32x4 bf16x8) for every 8-element piece of the block, in
//          the latent-then-rope column order (col8 in 0..71), zeros for tokens >= valid.
// --------------------------------------------------------------------------------------
template <int FMT, int NT>
struct TileReader;

// bf16 rows [c(512) | k_rope(64)] = 72 pieces of 16 bytes per token, 4608 per block.
template <int NT>
struct TileReader<FMT_BF16, NT> {
  static constexpr int PIECES = BLOCK_TOKENS * 72;
  static constexpr int PER = PIECES / NT;
  static_assert(PIECES % NT == 0, "thread count must divide the block");
  u32x4 v[PER];

  __device__ __forceinline__ void load(const uint8_t* blk, int valid, int tid, const QuantPlanes&, int, int) {
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      int p = tid + k * NT;
      int tok = p / 72;
      if (tok < valid) {
        v[k] = __builtin_nontemporal_load((const u32x4*)(blk + (size_t)p * 16));
      } else {
        v[k] = u32x4{0, 0, 0, 0};
      }
    }
  }
  template <class F>
  __device__ __forceinline__ void emit(F&& f, int valid, int tid) {
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      int p = tid + k * NT;
      f(p / 72, p % 72, v[k]);
    }
  }
};

// Quantised latent (INT4 or INT2) + INT4 RoPE key.
// Latent codes are read 16 bytes at a time: 32 INT4 or 64 INT2 elements per piece.
template <int FMT, int NT>
struct QuantTileReader {
  static constexpr int BITS = FMT == FMT_INT4 ? 4 : 2;
  static constexpr int LAT_BYTES = 512 * BITS / 8;              // per token
  static constexpr int LAT_PIECES = BLOCK_TOKENS * LAT_BYTES / 16;
  static constexpr int ELEMS = 128 / BITS;                       // elements per 16-byte piece
  static constexpr int PIECES_PER_TOK = LAT_BYTES / 16;
  static constexpr int PER = LAT_PIECES / NT;
  static constexpr int ROPE_PIECES = BLOCK_TOKENS * 2;           // 64 INT4 codes = 2 pieces/token
  static_assert(LAT_PIECES % NT == 0, "thread count must divide the latent plane");
  static_assert(ROPE_PIECES <= NT, "one rope piece per thread at most");
  u32x4 c[PER];
  uint32_t sz[PER][2];   // (scale, zero) words for the piece's first and second half
  u32x4 rc;
  uint32_t rsz;

  __device__ __forceinline__ void load(const uint8_t* blk, int valid, int tid, const QuantPlanes& pl,
                                       int g_lat, int g_rope) {
    const int groups = 512 / g_lat;
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      int p = tid + k * NT;
      int tok = p / PIECES_PER_TOK;
      int e0 = (p % PIECES_PER_TOK) * ELEMS;
      if (tok < valid) {
        c[k] = __builtin_nontemporal_load((const u32x4*)(blk + pl.lc + (size_t)p * 16));
        const uint32_t* szp = (const uint32_t*)(blk + pl.ls) + tok * groups;
        sz[k][0] = szp[e0 / g_lat];
        sz[k][1] = szp[(e0 + ELEMS / 2) / g_lat];
      } else {
        c[k] = u32x4{0, 0, 0, 0};
        sz[k][0] = sz[k][1] = 0;
      }
    }
    if (tid < ROPE_PIECES) {
      int tok = tid >> 1;
      if (tok < valid) {
        rc = __builtin_nontemporal_load((const u32x4*)(blk + pl.rc + (size_t)tid * 16));
        const uint32_t* szp = (const uint32_t*)(blk + pl.rs) + tok * (64 / g_rope);
        rsz = szp[((tid & 1) * 32) / g_rope];
      } else {
        rc = u32x4{0, 0, 0, 0};
        rsz = 0;
      }
    }
  }

  template <class F>
  __device__ __forceinline__ void emit(F&& f, int valid, int tid) {
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      int p = tid + k * NT;
      int tok = p / PIECES_PER_TOK;
      int col8 = (p % PIECES_PER_TOK) * (ELEMS / 8);
      if (tok >= valid) {
#pragma unroll
        for (int j = 0; j < ELEMS / 8; ++j) f(tok, col8 + j, u32x4{0, 0, 0, 0});
        continue;
      }
      float s0, zs0, s1, zs1;
      scale_zero(sz[k][0], s0, zs0);
      scale_zero(sz[k][1], s1, zs1);
      if (BITS == 4) {
        // 4 words x 8 codes; first two words in the first half of the piece
#pragma unroll
        for (int j = 0; j < 4; ++j) f(tok, col8 + j, dequant_int4x8(c[k][j], j < 2 ? s0 : s1, j < 2 ? zs0 : zs1));
      } else {
        // 4 words x 16 codes; each word gives two 8-element pieces
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          float s = j < 2 ? s0 : s1, zs = j < 2 ? zs0 : zs1;
          uint32_t t_lo, t_hi;
          int2_table(s, zs, t_lo, t_hi);
          u32x4 lo, hi;
          dequant_int2x16(c[k][j], t_lo, t_hi, lo, hi);
          f(tok, col8 + 2 * j, lo);
          f(tok, col8 + 2 * j + 1, hi);
        }
      }
    }
    if (tid < ROPE_PIECES) {
      int tok = tid >> 1;
      int col8 = 64 + (tid & 1) * 4;
      if (tok >= valid) {
#pragma unroll
        for (int j = 0; j < 4; ++j) f(tok, col8 + j, u32x4{0, 0, 0, 0});
      } else {
        float s, zs;
        scale_zero(rsz, s, zs);
#pragma unroll
        for (int j = 0; j < 4; ++j) f(tok, col8 + j, dequant_int4x8(rc[j], s, zs));
      }
    }
  }
};

template <int NT>
struct TileReader<FMT_INT4, NT> : QuantTileReader<FMT_INT4, NT> {};
template <int NT>
struct TileReader<FMT_INT2, NT> : QuantTileReader<FMT_INT2, NT> {};

}  // namespace mla
