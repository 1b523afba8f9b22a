// Cache writer: the new tokens' latent c_KV and RoPE key into their paged slots.
//
// Float caches take the values as they are (fp32) or rounded to bf16 (ties to even).
// Quantised caches take codes from the plain round-to-nearest asymmetric quantiser, per token
// and per group of channels: the pages pair the latent (content) cache at INT4 or INT2 with an
// INT4 RoPE-key cache (QuantMLA English abstract; arxivdaily QuantMLA page) and name
// round-to-nearest as the plain quantiser that the learned transforms are measured against
// (QuantMLA podcast page, comparison part).  Per group, from the exact input values:
//   s = fp16((max - min) / (2^b - 1)), 1 where that is 0;
//   z = clamp(rint(-min / s), 0, 2^b - 1), an integer stored as fp16 (+0 when zero);
//   code = clamp(rint(x / s) + z, 0, 2^b - 1),  rint ties to even.
// Every step is IEEE float64 (inputs are exact in it), so the codes and the (s, z) pairs are
// the ones a float64 evaluation of these formulas gives, bit for bit.
//
// One wavefront per token; lane l owns 8 consecutive channels (chunk l, l + 64, ...), so a
// group of G channels is G / 8 consecutive lanes and its minimum and maximum are two
// butterfly reductions over those lanes.  Codes of a chunk are packed in registers (INT4: one
// 32-bit word, INT2: one 16-bit half-word) and stored with one write; the first lane of a
// group writes its (s, z) pair.
#include <hip/hip_runtime.h>

#include "libmla.h"
#include "mla_device.hpp"
#include "mla_internal.hpp"

namespace mla {
namespace {

constexpr int kWaves = 4;   // tokens per 256-thread workgroup

// IEEE binary16 nearest to x, ties to even, straight from the binary64 bits (one rounding):
// normal results keep 11 significant bits, subnormal ones are multiples of 2^-24, and
// magnitudes from 65520 on become infinity.
__device__ uint16_t f64_to_f16_rne(double x) {
  const uint64_t b = (uint64_t)__double_as_longlong(x);
  const uint16_t sign = (uint16_t)((b >> 48) & 0x8000u);
  const int e = (int)((b >> 52) & 0x7FF);
  const uint64_t frac = b & ((1ull << 52) - 1);
  if (e == 0x7FF) return sign | (frac ? 0x7E00u : 0x7C00u);
  if (e == 0) return sign;                       // below 2^-1022: rounds to zero
  const uint64_t mant = frac | (1ull << 52);     // value = mant * 2^(E - 52)
  int E = e - 1023;
  if (E > 15) return sign | 0x7C00u;
  // the result's unit in the last place: 2^(E - 10) for normal results, 2^-24 below 2^-14
  const int shift = E >= -14 ? 42 : 28 - E;      // bits of mant below that unit
  if (shift > 53) return sign;                   // below half the smallest subnormal
  const uint64_t q = mant >> shift;
  const uint64_t rem = mant & ((1ull << shift) - 1);
  const uint64_t half = 1ull << (shift - 1);
  const uint64_t r = q + ((rem > half || (rem == half && (q & 1))) ? 1 : 0);
  if (E >= -14) {
    // r holds the 11 significant bits (2^10 <= r <= 2^11); a carry to 2^11 moves the exponent
    if (r == (1ull << 11)) {
      ++E;
      if (E > 15) return sign | 0x7C00u;
      return sign | (uint16_t)((E + 15) << 10);
    }
    return sign | (uint16_t)((E + 15) << 10) | (uint16_t)(r & 0x3FFu);
  }
  // subnormal: r multiples of 2^-24; r = 2^10 is the smallest normal, whose encoding is the same
  return sign | (uint16_t)r;
}

__device__ __forceinline__ double f16_to_f64(uint16_t h) {
  const int e = (h >> 10) & 0x1F;
  const int m = h & 0x3FF;
  double v;
  if (e == 31) v = m ? __builtin_nan("") : __builtin_inf();
  else if (e == 0) v = (double)m * 0x1p-24;
  else v = (double)(m | 0x400) * __builtin_ldexp(1.0, e - 25);
  return (h & 0x8000u) ? -v : v;
}

// The 8 input values of chunk k of a token row (bf16 or fp32), as doubles.
__device__ __forceinline__ void load8(const void* row, int k, bool f32, double v[8]) {
  if (f32) {
    const float* f = (const float*)row + 8 * k;
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = (double)f[j];
  } else {
    const uint16_t* h = (const uint16_t*)row + 8 * k;
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = (double)__uint_as_float((uint32_t)h[j] << 16);
  }
}

// Quantise one token's vector of D channels (groups of G) into its code and (s, z) rows.
template <int BITS>
__device__ void quantise_row(const void* src, bool f32, int D, int G, uint8_t* codes, uint8_t* sz, int lane) {
  constexpr int QMAX = (1 << BITS) - 1;
  const int lanes_g = G / 8;                     // a power of two <= 64
  for (int k0 = 0; k0 < D / 8; k0 += 64) {
    const int k = k0 + lane;
    const bool on = k < D / 8;                   // whole groups are on or off together
    double v[8];
    if (on) load8(src, k, f32, v);
    else {
#pragma unroll
      for (int j = 0; j < 8; ++j) v[j] = 0.0;
    }
    double lo = v[0], hi = v[0];
#pragma unroll
    for (int j = 1; j < 8; ++j) {
      lo = fmin(lo, v[j]);
      hi = fmax(hi, v[j]);
    }
    for (int o = 1; o < lanes_g; o <<= 1) {
      lo = fmin(lo, __shfl_xor(lo, o, 64));
      hi = fmax(hi, __shfl_xor(hi, o, 64));
    }
    uint16_t s16 = f64_to_f16_rne((hi - lo) / (double)QMAX);
    if ((s16 & 0x7FFFu) == 0) s16 = 0x3C00u;     // 1.0
    const double s = f16_to_f64(s16);
    // an integer zero-point: a zero is +0 (rint of a small negative quotient gives -0)
    const double z = fmin(fmax(__builtin_rint(-lo / s), 0.0), (double)QMAX) + 0.0;
    uint32_t word = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const double q = fmin(fmax(__builtin_rint(v[j] / s) + z, 0.0), (double)QMAX);
      word |= (uint32_t)q << (BITS * j);
    }
    if (on) {
      if constexpr (BITS == 4) *(uint32_t*)(codes + 4 * k) = word;
      else *(uint16_t*)(codes + 2 * k) = (uint16_t)word;
      if ((lane & (lanes_g - 1)) == 0) {
        const int g = 8 * k / G;
        *(uint32_t*)(sz + 4 * g) = (uint32_t)s16 | ((uint32_t)f64_to_f16_rne(z) << 16);
      }
    }
  }
}

__global__ __launch_bounds__(64 * kWaves) void append_kernel(AppendParams p) {
  const int lane = threadIdx.x & 63;
  const int64_t i = (int64_t)blockIdx.x * kWaves + (threadIdx.x >> 6);
  if (i >= p.n) return;
  const int64_t slot = p.slots[i];
  if (slot < 0 || slot >= p.num_blocks * BLOCK_TOKENS) return;   // padding or not a slot of the pool
  const int64_t blk = slot / BLOCK_TOKENS;
  const int pos = (int)(slot % BLOCK_TOKENS);
  uint8_t* base = p.pool + blk * p.block_bytes;
  const bool f32 = p.in_f32 != 0;
  const void* c = f32 ? (const void*)((const float*)p.c + i * p.c_stride) : (const void*)((const uint16_t*)p.c + i * p.c_stride);
  const void* k = f32 ? (const void*)((const float*)p.k + i * p.k_stride) : (const void*)((const uint16_t*)p.k + i * p.k_stride);
  const int W = p.d_c + p.d_r;
  if (p.fmt_lat == MLA_FMT_F32 || p.fmt_lat == MLA_FMT_BF16) {
    // one row [c | k_rope] per token
    for (int e = lane; e < W; e += 64) {
      const void* src = e < p.d_c ? c : k;
      const int j = e < p.d_c ? e : e - p.d_c;
      const float x = f32 ? ((const float*)src)[j] : __uint_as_float((uint32_t)((const uint16_t*)src)[j] << 16);
      if (p.fmt_lat == MLA_FMT_F32) ((float*)base)[(int64_t)pos * W + e] = x;
      else ((uint16_t*)base)[(int64_t)pos * W + e] = (uint16_t)f32_to_bf16_bits(x);
    }
    return;
  }
  const int lb = p.fmt_lat == MLA_FMT_INT4 ? 4 : 2, rb = p.fmt_rope == MLA_FMT_INT4 ? 4 : 2;
  uint8_t* lc = base + p.off_lc + (int64_t)pos * (p.d_c * lb / 8);
  uint8_t* ls = base + p.off_ls + (int64_t)pos * (p.d_c / p.g_lat) * 4;
  uint8_t* rc = base + p.off_rc + (int64_t)pos * (p.d_r * rb / 8);
  uint8_t* rs = base + p.off_rs + (int64_t)pos * (p.d_r / p.g_rope) * 4;
  if (lb == 4) quantise_row<4>(c, f32, p.d_c, p.g_lat, lc, ls, lane);
  else quantise_row<2>(c, f32, p.d_c, p.g_lat, lc, ls, lane);
  if (rb == 4) quantise_row<4>(k, f32, p.d_r, p.g_rope, rc, rs, lane);
  else quantise_row<2>(k, f32, p.d_r, p.g_rope, rc, rs, lane);
}

}  // namespace

hipError_t launch_append(const AppendParams& p, hipStream_t st) {
  if (p.n <= 0) return hipSuccess;
  const int64_t blocks = (p.n + kWaves - 1) / kWaves;
  hipLaunchKernelGGL(append_kernel, dim3((unsigned)blocks), dim3(64 * kWaves), 0, st, p);
  return hipGetLastError();
}

}  // namespace mla
