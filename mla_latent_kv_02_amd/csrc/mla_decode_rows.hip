// MLA decode for many query rows per sequence (H * s_q >= 96, e.g. 128 heads): the absorbed-MQA
// attention step with each wavefront owning whole query rows (gfx950).
//
// Every head scores the same cached rows [c (512) | k_rope (64)] (GQLA abstract: absorbed MQA
// decoding path), the softmax-weighted sum is taken over the latent itself (RAQ-MLA abstract:
// the latent supplies the values), and INT4/INT2 caches are unpacked and dequantised inside
// the loop (QuantMLA English abstract: native low-bit attention kernel).
//
// Workgroup = 4 wavefronts (one per SIMD, up to 512 registers each) and 128 query rows; wave
// w owns rows 32w .. 32w+31 end to end:
//   * scores S^T = K . Q^T on v_mfma_f32_16x16x32_bf16: K fragments from the LDS stage, Q^T
//     for both 16-row tiles held in registers; each K fragment feeds two MFMAs;
//   * softmax in registers: the 32 scores of a row sit in 4 lane groups, so a row maximum is
//     two lane swaps; the running maximum moves only when a stage exceeds it by more than
//     ROWS_SLACK (log2 units), so rescaling the accumulators is rare;
//   * O^T += V^T . P^T: the score accumulators are already the P^T operand once the token
//     order inside the 32-token step is taken as (4 tokens of tile 0, 4 of tile 1) per lane
//     group, and V^T fragments come from the token-major stage with ds_read_b64_tr_b16 in the
//     same order.  P is split into two bf16 terms (hi + lo, ~16 significant bits), so each
//     V^T fragment feeds four MFMAs (two row tiles x two terms); O^T (32 rows x 512) stays in
//     AGPRs, touched only by inline asm (MFMAs, a rare LDS round-trip rescale, stores).
// There is no cross-wave dependency inside a step: one barrier per 32-token stage guards the
// ring of LDS stages.
//
// Stages stream HBM -> LDS with global_load_lds_dwordx4 (bf16: a 4-deep ring, three stages
// in flight; INT4/INT2: a ring of code stages, dequantised one step ahead into a second bf16
// stage).  The DMA is written as inline asm with precomputed per-lane source offsets: the
// compiler never inserts waits for it, and each step waits with an explicit vmcnt for exactly
// the stage it needs.
//
// Work balance: the batch's cache blocks, sequence after sequence, are cut into n_ranges equal
// ranges (one workgroup per range and row group); a range may cover several sequences or part
// of one.  Each sequence's start is charged a few extra positions, the cost of a piece's store
// and query load, so that ranges which start a sequence in their middle get fewer blocks.  Every piece (a sequence's blocks inside one range) is stored unnormalised with
// 1 / sum(P) and its lse; combine_kernel normalises and merges.
#include <hip/hip_runtime.h>

#include <type_traits>
#include <utility>

#include "mla_device.hpp"
#include "mla_internal.hpp"
#include "mla_stage.hpp"

namespace mla {
namespace rows {

// Piece swizzle of this kernel's bf16 stages: piece c of token t sits at c ^ rsw(t).  The
// P.V operand reads here take tokens 0..7 (and 16..23, 8..15, 24..31) per 32 lanes, in the
// order the score accumulators give P; the shared stage swizzle sw() maps t and t + 4 to the
// same banks for that order.  t & 7 keeps these reads, the score operand reads and the
// dequantised piece stores on 64 distinct banks per cycle (exhaustive check under the
// measured lane-set model), and rsw(t + 16) = rsw(t).
__device__ __forceinline__ int rsw(int t) { return t & 7; }
__device__ __forceinline__ int rst_off(int t, int d) { return t * 576 + (((d >> 3) ^ rsw(t)) << 3) + (d & 7); }

// lambdas of the kernel body are inlined whatever their size: a call would put the accumulator
// array, which they reach by reference, in memory
#define MLA_INLINE __attribute__((always_inline))

// f(integral_constant<int, 0>), ..., f(integral_constant<int, N - 1>) in order: an unrolled
// loop whose index is a compile-time constant in the body
template <typename F, int... I>
__device__ __forceinline__ void static_for_seq(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
// Keeps the computation of x at this point of the instruction stream: an empty volatile asm
// that takes and redefines x is ordered with the MFMA asm around it, so the compiler can
// neither sink the work that produced x to its later uses nor hoist it.
template <typename T>
__device__ __forceinline__ void pin(T& x) {
  asm volatile("" : "+v"(x));
}

// Float maxima as single instructions: fmaxf would first quiet possible signalling NaNs of
// operands the compiler cannot trace (permlane results, pinned values), one instruction each.
__device__ __forceinline__ float vmax(float a, float b) {
  float d;
  asm("v_max_f32 %0, %1, %2" : "=v"(d) : "v"(a), "v"(b));
  return d;
}
__device__ __forceinline__ float vmax3(float a, float b, float c) {
  float d;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(d) : "v"(a), "v"(b), "v"(c));
  return d;
}

template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_seq(f, std::make_integer_sequence<int, N>{});
}

constexpr int NT = 256;                  // 4 wavefronts, one per SIMD
constexpr int ROWS = 128;                // query rows per workgroup
constexpr int RT = 2;                    // 16-row tiles per wavefront
constexpr int MAX_RANGE_BLOCKS = 256;    // cache blocks per range (host planner guarantees it)
constexpr int MAX_ST = 2 * MAX_RANGE_BLOCKS;
constexpr int ST_BYTES = ST_ELEMS * 2;   // one bf16 stage
// Log2 headroom of P before a row's running maximum moves: rescaling the AGPR accumulators
// is slow here, and P <= 2^16 keeps every sum well inside fp32 (at most 2^17 tokens per piece).
constexpr float ROWS_SLACK = 16.f;
static_assert(MAX_RANGE_BLOCKS <= NT, "one thread per block of a range builds the stage table");

// 16 bytes per lane HBM -> LDS from base + off (base wave-uniform, off per lane); lane i writes
// LDS bytes [lds_base + 16 i, lds_base + 16 i + 16).  The addresses are precomputed per lane:
// with one wavefront per SIMD, VALU address arithmetic for each DMA instruction stalls the
// MFMA stream more than the copy itself.  One wait state between the M0 write and the DMA
// that reads it; the kernel makes no other use of M0.
__device__ __forceinline__ void dma16(const uint8_t* base, uint32_t off, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(lds_base), "v"(off), "s"(base)
               : "memory", "m0");
}

// Score MFMAs, v_mfma_f32_16x16x32_bf16 with VGPR accumulators.  The compiler gives every
// MFMA of a function the same accumulator register file, and the O^T accumulators fill the
// 256 AGPRs; written as inline asm, the score MFMAs keep theirs in VGPRs.  The compiler
// inserts no hazard waits around inline asm: the first pair of a step starts with two wait
// states (the VALU may just have written an operand; the other pairs read only LDS loads and
// the query registers), dependent MFMA accumulation is interlocked by the hardware, and the
// last pair waits out the MFMA latency before anything else can read the results.
// c0 += a . q0, c1 += a . q1 (FIRST: c = a . q).
template <bool FIRST, bool NOP, bool DRAIN>
__device__ __forceinline__ void score2(f32x4& c0, f32x4& c1, const bf16x8& a, const bf16x8& q0, const bf16x8& q1) {
#define MLA_S_NOP0 "s_nop 1\n\t"
#define MLA_S_ACC "v_mfma_f32_16x16x32_bf16 %0, %2, %3, %0\n\tv_mfma_f32_16x16x32_bf16 %1, %2, %4, %1"
#define MLA_S_NEW "v_mfma_f32_16x16x32_bf16 %0, %2, %3, 0\n\tv_mfma_f32_16x16x32_bf16 %1, %2, %4, 0"
#define MLA_S_DRAIN "\n\ts_nop 7\n\ts_nop 7\n\ts_nop 3"
  if constexpr (FIRST) {
    if constexpr (NOP)
      asm volatile(MLA_S_NOP0 MLA_S_NEW : "=&v"(c0), "=&v"(c1) : "v"(a), "v"(q0), "v"(q1));
    else
      asm volatile(MLA_S_NEW : "=&v"(c0), "=&v"(c1) : "v"(a), "v"(q0), "v"(q1));
  } else if constexpr (DRAIN) {
    asm volatile(MLA_S_ACC MLA_S_DRAIN : "+v"(c0), "+v"(c1) : "v"(a), "v"(q0), "v"(q1));
  } else {
    asm volatile(MLA_S_ACC : "+v"(c0), "+v"(c1) : "v"(a), "v"(q0), "v"(q1));
  }
#undef MLA_S_NOP0
#undef MLA_S_ACC
#undef MLA_S_NEW
#undef MLA_S_DRAIN
}

// O^T MFMAs on AGPR accumulators, also inline asm, and so is every other access to those
// accumulators: when C code reads them (a rescale, the final store), the compiler moves all
// 256 through VGPRs and spills.  c += v . p (FRESH: c = v . p, the first step of a piece).
// The first MFMA of a step waits two states for the VALU that wrote p; the last waits out
// the MFMA latency before anything else reads the accumulators.
template <bool FRESH, bool NOP, bool DRAIN>
__device__ __forceinline__ void pv1(f32x4& c, const bf16x8& v, const bf16x8& pp) {
#define MLA_PV_NOP0 "s_nop 1\n\t"
#define MLA_PV_ACC "v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0"
#define MLA_PV_NEW "v_mfma_f32_16x16x32_bf16 %0, %1, %2, 0"
#define MLA_PV_DRAIN "\n\ts_nop 7\n\ts_nop 7\n\ts_nop 3"
  if constexpr (FRESH) {
    if constexpr (NOP) asm volatile(MLA_PV_NOP0 MLA_PV_NEW : "=a"(c) : "v"(v), "v"(pp));
    else if constexpr (DRAIN) asm volatile(MLA_PV_NEW MLA_PV_DRAIN : "=a"(c) : "v"(v), "v"(pp));
    else asm volatile(MLA_PV_NEW : "=a"(c) : "v"(v), "v"(pp));
  } else {
    if constexpr (NOP) asm volatile(MLA_PV_NOP0 MLA_PV_ACC : "+a"(c) : "v"(v), "v"(pp));
    else if constexpr (DRAIN) asm volatile(MLA_PV_ACC MLA_PV_DRAIN : "+a"(c) : "v"(v), "v"(pp));
    else asm volatile(MLA_PV_ACC : "+a"(c) : "v"(v), "v"(pp));
  }
#undef MLA_PV_NOP0
#undef MLA_PV_ACC
#undef MLA_PV_NEW
#undef MLA_PV_DRAIN
}

// c = 0 for an AGPR tile: an MFMA of zero operands (z holds zeros).  NOP: two wait states
// first for the VALU that may have just written z; DRAIN: the MFMA latency waited out after.
// The tile is an in-out operand: its registers stay where they are (a fresh output would let
// the register allocator move the accumulators between branches, through copies and spills).
template <bool NOP, bool DRAIN>
__device__ __forceinline__ void zero_tile(f32x4& c, const bf16x8& z) {
  if constexpr (NOP) asm volatile("s_nop 1\n\tv_mfma_f32_16x16x32_bf16 %0, %1, %1, 0" : "+a"(c) : "v"(z));
  else if constexpr (DRAIN) asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %1, 0\n\ts_nop 7\n\ts_nop 7\n\ts_nop 3" : "+a"(c) : "v"(z));
  else asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %1, 0" : "+a"(c) : "v"(z));
}

// c_k *= a (a per lane) for eight AGPR tiles, through 16 bytes per lane of this wave's LDS
// scratch: inline asm cannot name the four registers of a tile one by one, and VALU
// instructions cannot read AGPRs.  A tile goes to the slot, comes back as four VGPRs, is
// scaled, and goes back to its AGPRs by the slot again; the next tile enters the slot right
// behind that read-back (LDS operations of one wave complete in order), so each tile costs one
// wait for an LDS round trip.  Rare: only when a running maximum moves.
#define MLA_SCALE_TILE(T)                     \
  "ds_write_b128 %12, %" #T "\n\t"            \
  "ds_read_b32 %0, %12\n\t"                   \
  "ds_read_b32 %1, %12 offset:4\n\t"          \
  "ds_read_b32 %2, %12 offset:8\n\t"          \
  "ds_read_b32 %3, %12 offset:12\n\t"         \
  "s_waitcnt lgkmcnt(0)\n\t"                  \
  "v_mul_f32 %0, %0, %13\n\t"                 \
  "v_mul_f32 %1, %1, %13\n\t"                 \
  "v_mul_f32 %2, %2, %13\n\t"                 \
  "v_mul_f32 %3, %3, %13\n\t"                 \
  "ds_write_b32 %12, %0\n\t"                  \
  "ds_write_b32 %12, %1 offset:4\n\t"         \
  "ds_write_b32 %12, %2 offset:8\n\t"         \
  "ds_write_b32 %12, %3 offset:12\n\t"        \
  "ds_read_b128 %" #T ", %12\n\t"
__device__ __forceinline__ void scale_tiles8(f32x4& c0, f32x4& c1, f32x4& c2, f32x4& c3, f32x4& c4, f32x4& c5,
                                             f32x4& c6, f32x4& c7, float a, uint32_t lds) {
  float x0, x1, x2, x3;
  asm volatile(MLA_SCALE_TILE(4) MLA_SCALE_TILE(5) MLA_SCALE_TILE(6) MLA_SCALE_TILE(7) MLA_SCALE_TILE(8)
                   MLA_SCALE_TILE(9) MLA_SCALE_TILE(10) MLA_SCALE_TILE(11) "s_waitcnt lgkmcnt(0)"
               : "=&v"(x0), "=&v"(x1), "=&v"(x2), "=&v"(x3), "+a"(c0), "+a"(c1), "+a"(c2), "+a"(c3), "+a"(c4),
                 "+a"(c5), "+a"(c6), "+a"(c7)
               : "v"(lds), "v"(a)
               : "memory");
}
#undef MLA_SCALE_TILE

// 16 bytes of an AGPR tile to global memory (counted by vmcnt like the stage loads)
__device__ __forceinline__ void store_tile(float* dst, const f32x4& c) {
  asm volatile("global_store_dwordx4 %0, %1, off" ::"v"(dst), "a"(c) : "memory");
}

// 16 bytes of an AGPR tile to LDS (the epilogue's way from the accumulators to VGPRs)
template <int OFF>
__device__ __forceinline__ void lds_put_tile(uint32_t addr, const f32x4& c) {
  asm volatile("ds_write_b128 %0, %1 offset:%2" ::"v"(addr), "a"(c), "i"(OFF) : "memory");
}

// Reductions over the four lane groups (lanes l, l ^ 16, l ^ 32, l ^ 48) with the gfx950 lane
// swaps: with both operands equal, permlane32_swap / permlane16_swap return x at l and at l ^ 32
// (l ^ 16), so one max / add per step gives the butterfly without an LDS round trip.
__device__ __forceinline__ float max_lg(float x) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float sum_lg(float x) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) { return (uint32_t)(uintptr_t)(const lds_void*)p; }

__device__ __forceinline__ bf16x8 load_q8(const void* base, size_t elem_off, bool f32) {
  if (!f32) return __builtin_bit_cast(bf16x8, *(const u32x4*)((const bf16_t*)base + elem_off));
  const float* f = (const float*)base + elem_off;
  const f32x4 a = *(const f32x4*)f;
  const f32x4 b = *(const f32x4*)(f + 4);
  u32x4 r;
  r[0] = pack_bf16x2(a[0], a[1]);
  r[1] = pack_bf16x2(a[2], a[3]);
  r[2] = pack_bf16x2(b[0], b[1]);
  r[3] = pack_bf16x2(b[2], b[3]);
  return __builtin_bit_cast(bf16x8, r);
}

// ----------------------------------------------------------------------------------------
// Stage producers: every thread issues LOADS DMA instructions per stage, one call of
// issue_one(i) each, so a wave's count of outstanding stage loads is known exactly.
// ----------------------------------------------------------------------------------------

// bf16 rows: a half block is 32 tokens x 72 pieces = 2304 pieces, 9 per thread.  Slot k of the
// stage receives (token k / 72, logical piece (k mod 72) ^ rsw(token)).  All 32 rows are copied
// (a block is always allocated whole); rows past the sequence end are zeroed before use.
struct BfProducer {
  static constexpr int LOADS = ST_TOK * 72 / NT;
  static_assert(LOADS * NT == ST_TOK * 72, "threads must divide the stage");
  struct Offsets {
    uint32_t o[LOADS];
  };
  __device__ static Offsets offsets(int tid) {
    Offsets r;
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const int slot = i * NT + tid;
      const int t = slot / 72;
      r.o[i] = (uint32_t)(t * 1152 + (((slot - t * 72) ^ rsw(t)) << 4));
    }
    return r;
  }
  __device__ __forceinline__ static void issue_one(int i, const Offsets& off, const uint8_t* half, uint32_t lds) {
    dma16(half, off.o[i], lds + (uint32_t)(i * NT * 16));
  }
};

// Quantised latent (INT4 or INT2) + INT4 rope: the four code planes of a half block are copied
// as they lie in the block (token-major) into a code stage [lc | ls | rc | rs] of SLOTS 16-byte
// slots.
template <int FMT>
struct QuantStage {
  static constexpr int BITS = FMT == FMT_INT4 ? 4 : 2;
  static constexpr int LB = 512 * BITS / 8;        // latent code bytes per token
  static constexpr int LOADS = FMT == FMT_INT4 ? 3 : 2;
  static constexpr int SLOTS = LOADS * NT;         // INT4: 648 used, INT2: 456
  static constexpr int DEPTH = FMT == FMT_INT4 ? 6 : 8;   // code ring slots

  // per-lane source offsets inside a block of DMA instruction i, for the block's two halves;
  // the code stage is the four planes of the half block, token-major, one after the other
  struct Offsets {
    uint32_t o[2][LOADS];
  };
  __device__ static Offsets offsets(const QuantPlanes& pl, int groups, int rgroups, int tid) {
    const int n_lc = ST_TOK * LB / 16;
    const int n_ls = ST_TOK * groups * 4 / 16;
    const int n_rc = ST_TOK * 32 / 16;
    const int n_rs = (ST_TOK * rgroups * 4 + 15) / 16;
    const int n_all = n_lc + n_ls + n_rc + n_rs;
    Offsets r;
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const int slot = i * NT + tid;
      int q = slot < n_all ? slot : slot - n_all;   // padding slots re-load a real piece
      int base, hstride;
      if (q < n_lc) {
        base = pl.lc + q * 16;
        hstride = ST_TOK * LB;
      } else if ((q -= n_lc) < n_ls) {
        base = pl.ls + q * 16;
        hstride = ST_TOK * groups * 4;
      } else if ((q -= n_ls) < n_rc) {
        base = pl.rc + q * 16;
        hstride = ST_TOK * 32;
      } else {
        base = pl.rs + (q - n_rc) * 16;
        hstride = ST_TOK * rgroups * 4;
      }
      r.o[0][i] = (uint32_t)base;
      r.o[1][i] = (uint32_t)(base + hstride);
    }
    return r;
  }
  __device__ __forceinline__ static void issue_one(int i, const Offsets& off, const uint8_t* blk, int half,
                                                   uint32_t lds) {
    dma16(blk, half ? off.o[1][i] : off.o[0][i], lds + (uint32_t)(i * NT * 16));
  }

  // Thread q dequantises latent tasks q and q + 256 (32-element chunks, each inside one
  // quantisation group since groups are multiples of 32) and RoPE task q; the task to (token,
  // chunk) maps keep a wavefront's code reads and bf16 stores free of bank conflicts.  Group
  // sizes are powers of two (gl = log2 latent group, gr = log2 rope group).  load_chunk(h)
  // reads the code words and the raw scale word of latent task q + 256 h, chunk_piece()
  // converts and stores one of its four 8-element pieces (INT2: two); load_rope() and
  // rope_piece() do the same for the RoPE piece.
  struct Chunk {
    uint32_t c[BITS];   // INT4: 16 code bytes, INT2: 8
    uint32_t sz;        // fp16 (scale, zero), 0 for tokens past the end
    int row, p0;        // stage row of the token, physical piece of the chunk's first 8 elements
  };
  __device__ __forceinline__ static Chunk load_chunk(const uint8_t* cst, int valid, int gl, int h, int tid) {
    asm volatile("" : "+v"(tid));
    int t, kk;
    lat_task(tid + 256 * h, t, kk);
    const int ls = ST_TOK * LB;                    // scale plane of the latent codes
    Chunk d;
    const uint32_t sz = *(const uint32_t*)(cst + ls + (((t << (9 - gl)) + ((kk * 32) >> gl)) << 2));
    d.sz = t < valid ? sz : 0u;
    d.row = t * 576;
    d.p0 = (4 * kk) ^ rsw(t);
    const uint8_t* code = cst + t * LB + kk * 4 * BITS;
    if constexpr (BITS == 4) {
      const u32x4 c = *(const u32x4*)code;
      d.c[0] = c[0];
      d.c[1] = c[1];
      d.c[2] = c[2];
      d.c[3] = c[3];
    } else {
      const uint2 c = *(const uint2*)code;
      d.c[0] = c.x;
      d.c[1] = c.y;
    }
    return d;
  }
  __device__ __forceinline__ static void chunk_piece(const Chunk& d, int jj, bf16_t* stage) {
    float sc, zs;
    scale_zero(d.sz, sc, zs);
    if constexpr (BITS == 4) {
      *(u32x4*)&stage[d.row + ((d.p0 ^ jj) << 3)] = dequant_int4x8(d.c[jj], sc, zs);
    } else {
      // INT2: pieces jj and jj + 1 (jj even) from one code word
      uint32_t t_lo, t_hi;
      int2_table(sc, zs, t_lo, t_hi);
      u32x4 lo, hi;
      dequant_int2x16(d.c[jj >> 1], t_lo, t_hi, lo, hi);
      *(u32x4*)&stage[d.row + ((d.p0 ^ jj) << 3)] = lo;
      *(u32x4*)&stage[d.row + ((d.p0 ^ (jj + 1)) << 3)] = hi;
    }
  }
  struct Rope {
    uint32_t c, sz;
    int dst;            // stage element of the piece
  };
  __device__ __forceinline__ static Rope load_rope(const uint8_t* cst, int valid, int gl, int gr, int tid) {
    asm volatile("" : "+v"(tid));
    int t, ri;
    rope_task(tid, t, ri);
    const int rbase = ST_TOK * LB + (ST_TOK << (9 - gl + 2));
    Rope r;
    const uint32_t sz = *(const uint32_t*)(cst + rbase + ST_TOK * 32 + (((t << (6 - gr)) + ((ri * 8) >> gr)) << 2));
    r.sz = t < valid ? sz : 0u;
    r.c = *(const uint32_t*)(cst + rbase + t * 32 + ri * 4);
    r.dst = rst_off(t, 512 + ri * 8);
    return r;
  }
  __device__ __forceinline__ static void rope_piece(const Rope& r, bf16_t* stage) {
    float sc, zs;
    scale_zero(r.sz, sc, zs);
    *(u32x4*)&stage[r.dst] = dequant_int4x8(r.c, sc, zs);
  }
  __device__ __forceinline__ static void dequant(const uint8_t* cst, int valid, int gl, int gr, bf16_t* stage,
                                                 int tid) {
    const Chunk d0 = load_chunk(cst, valid, gl, 0, tid);
    const Chunk d1 = load_chunk(cst, valid, gl, 1, tid);
    const Rope r = load_rope(cst, valid, gl, gr, tid);
    constexpr int STEP = BITS == 4 ? 1 : 2;   // pieces per chunk_piece call
#pragma unroll
    for (int jj = 0; jj < 4; jj += STEP) chunk_piece(d0, jj, stage);
#pragma unroll
    for (int jj = 0; jj < 4; jj += STEP) chunk_piece(d1, jj, stage);
    rope_piece(r, stage);
  }
};

// Stage table entry flags (st_info): sequence index in bits 0..19, valid tokens in 20..25.
constexpr int INFO_START = 1 << 26;   // first stage of a piece (a sequence's blocks inside one range)
constexpr int INFO_END = 1 << 27;     // last stage of a piece
constexpr int INFO_PART = 28;         // mixed histories: the stage's part in bits 28..29 (1: low-bit)

// ----------------------------------------------------------------------------------------
// The kernel
// ----------------------------------------------------------------------------------------
// MIXED: the history of sequence b is a bf16 sink ++ the low-bit middle ++ a bf16 recent
// window (p.hi), decoded as one sequence of blocks: a bf16 block is copied into a bf16 stage by
// DMA where a low-bit block would be dequantised into it, and every step keeps the code ring's
// load count (a bf16 block's ring slot receives a stand-in copy of its first bytes, unread).
template <int FMT, bool QF32, bool MIXED>
__global__ __launch_bounds__(NT, 1) void decode_rows_kernel(RowsParams p) {
  constexpr bool QUANT = FMT != FMT_BF16;
  static_assert(QUANT || !MIXED, "a mixed history has a low-bit middle");
  using QS = QuantStage<FMT == FMT_BF16 ? FMT_INT4 : FMT>;
  // bf16: 4 ring stages.  Quantised: 2 bf16 stages + DEPTH code stages.
  constexpr int DEPTH = QUANT ? QS::DEPTH : 4;
  constexpr int CBYTES = QS::SLOTS * 16;
  constexpr int SMEM = QUANT ? 2 * ST_BYTES + DEPTH * CBYTES : 4 * ST_BYTES;
  __shared__ __attribute__((aligned(16))) uint8_t smem[SMEM];
  __shared__ int st_bid[MAX_ST];
  __shared__ int st_tok[MAX_ST];
  __shared__ int st_info[MAX_ST];
  __shared__ int st_len[MAX_ST];
  __shared__ int sh_scan[NT / 64 + 1];
  __shared__ int sh_scanc[NT / 64];
  __shared__ f32x4 resc[NT];         // per-lane scratch of scale_tiles8

  const int tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63, lr = lane & 15, lg = lane >> 4;
  const float NEG_INF = -__builtin_inff();

  // unit of work; consecutive units sit on one XCD (workgroups are dealt round-robin to 8 XCDs)
  const int u = (int)(blockIdx.x & 7) * p.units_per_xcd + (int)(blockIdx.x >> 3);
  if (u >= p.total_units) return;
  const int rg = u % p.RG;
  const int range = u / p.RG;
  const int B = p.B, R = p.R;
  // mixed histories: the token counts of sequence b's three parts (an absent part has none)
  auto part_lens = [&](int b, int& Ls, int& Lm, int& Lr) {
    auto clamp_len = [b](const int32_t* lens, int mx) {
      if (lens == nullptr) return 0;
      const int L = lens[b];
      return L < 0 ? 0 : (L > mx ? mx : L);
    };
    Ls = clamp_len(p.hi[0].seq_lens, p.hi[0].max_seq_len);
    Lm = clamp_len(p.seq_lens, p.max_seq_len);
    Lr = clamp_len(p.hi[1].seq_lens, p.hi[1].max_seq_len);
  };
  auto nblocks = [](int L) { return (L + BLOCK_TOKENS - 1) / BLOCK_TOKENS; };

  // ---- flattened block space: sequence b owns positions [P_b, P_{b+1}): G positions that
  // stand for the cost of starting a piece (a query load, a piece store), then its n_b cache
  // blocks (an empty sequence owns none).  Ranges cut this space into equal parts, so a range
  // that starts a sequence in its middle gets correspondingly fewer blocks.  G = p.phantom
  // unless every sequence already starts on a range boundary of the plain block space (equal
  // lengths that divide evenly), where no range pays for a start and G = 0.  P, the clamped
  // lengths and the count of non-empty sequences before b live in the (not yet used) stage
  // memory while the stage table is built.
  int* tabP = (int*)smem;            // B + 1 entries
  int* tabL = tabP + (B + 1);        // B entries
  int* tabC = tabL + B;              // B + 1 entries, dead once P includes the charges
  int carry = 0, carry_c = 0;
  for (int base = 0; base < B; base += NT) {
    const int b = base + tid;
    int L = 0, n = 0;
    if (b < B) {
      if constexpr (MIXED) {
        // blocks in joint positions (each part padded to whole blocks); the causal mask of the
        // recent window, which starts at position 64 nsm, as L - s_q + query index, with every
        // sink and middle token visible when the window holds fewer than s_q tokens
        int Ls, Lm, Lr;
        part_lens(b, Ls, Lm, Lr);
        const int nsm = nblocks(Ls) + nblocks(Lm);
        n = nsm + nblocks(Lr);
        L = n > 0 ? BLOCK_TOKENS * nsm + max(Lr, p.s_q - 1) : 0;
      } else {
        L = p.seq_lens[b];
        L = L < 0 ? 0 : (L > p.max_seq_len ? p.max_seq_len : L);
        n = nblocks(L);
      }
    }
    const int c = n > 0 ? 1 : 0;
    int x = n, xc = c;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(x, o, 64);
      const int yc = __shfl_up(xc, o, 64);
      if (lane >= o) {
        x += y;
        xc += yc;
      }
    }
    if (lane == 63) {
      sh_scan[w] = x;
      sh_scanc[w] = xc;
    }
    __syncthreads();
    int woff = 0, tot = 0, woffc = 0, totc = 0;
#pragma unroll
    for (int j = 0; j < NT / 64; ++j) {
      woff += j < w ? sh_scan[j] : 0;
      tot += sh_scan[j];
      woffc += j < w ? sh_scanc[j] : 0;
      totc += sh_scanc[j];
    }
    if (b < B) {
      tabP[b] = carry + woff + x - n;
      tabL[b] = L;
      tabC[b] = carry_c + woffc + xc - c;
    }
    carry += tot;
    carry_c += totc;
    __syncthreads();
  }
  if (tid == 0) {
    tabP[B] = carry;
    tabC[B] = carry_c;
  }
  __syncthreads();
  int G;
  {
    const int per0 = max(1, (carry + p.n_ranges - 1) / p.n_ranges);
    int off = 0;
    for (int b = tid; b < B; b += NT) off |= (tabP[b + 1] > tabP[b] && tabP[b] % per0 != 0) ? 1 : 0;
    G = __syncthreads_or(off) ? p.phantom : 0;
    for (int b = tid; b <= B; b += NT) tabP[b] += G * tabC[b];
  }
  __syncthreads();
  const int total = tabP[B];
  const int per = max(1, (total + p.n_ranges - 1) / p.n_ranges);
  __syncthreads();
  if (u == 0) {
    if (tid == 0) {
      p.meta[0] = per;
      p.meta[B + 2] = G;
    }
    for (int b = tid; b <= B; b += NT) p.meta[1 + b] = tabP[b];
  }
  // empty sequences (no blocks): o = 0 and lse = -inf, written by the workgroups of the range
  // that holds their position in the block space
  {
    int* elist = tabL + B;
    if (tid == 0) sh_scan[NT / 64] = 0;
    __syncthreads();
    for (int b = tid; b < B; b += NT) {
      if (tabP[b + 1] == tabP[b]) {
        const int owner = total > 0 ? min(tabP[b], total - 1) / per : 0;
        if (owner == range) elist[atomicAdd(&sh_scan[NT / 64], 1)] = b;
      }
    }
    __syncthreads();
    const int n_empty = sh_scan[NT / 64];
    for (int e = 0; e < n_empty; ++e) {
      const int b = elist[e];
      for (int q = tid; q < ROWS * 128; q += NT) {
        const int row = rg * ROWS + q / 128;
        if (row >= R) break;
        const size_t o = ((size_t)b * R + row) * 512 + (q % 128) * 4;
        if (p.out_bf16) *(uint2*)((bf16_t*)p.out + o) = uint2{0u, 0u};
        else *(f32x4*)((float*)p.out + o) = f32x4{0.f, 0.f, 0.f, 0.f};
      }
      if (p.out_lse != nullptr && tid < ROWS && rg * ROWS + tid < R) p.out_lse[(size_t)b * R + rg * ROWS + tid] = NEG_INF;
    }
  }
  const int start = range * per;
  const int end = min(total, start + per);
  if (start >= end) return;

  // sequence holding block j: the last b with P_b <= j (P is non-decreasing; j < total)
  auto seq_of = [&](int j) {
    int lo = 0, hi = B;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (tabP[mid] <= j) lo = mid;
      else hi = mid;
    }
    return lo;
  };

  // ---- per-wave state: rows row0 + 16 rt, row0 = rg * 128 + 32 w + lr
  const int row0 = rg * ROWS + 32 * w + lr;
  bf16x8 qreg[RT][18];
  float m_s[RT], l_x[RT];
  int lim[RT];
  int lim_all = -1;   // every query row of the piece attends tokens 0 .. lim_all (L - s_q)
  f32x4 acc[RT][32];

  // new piece: this sequence's queries, fresh softmax state
  int cur_b = -1;
  bool fresh = true;
  auto start_piece = [&](int b, int L, bool wait) MLA_INLINE {
    cur_b = b;
    int r0 = row0, lg_ = lg;
    asm volatile("" : "+v"(r0), "+v"(lg_));   // addresses recomputed here rather than held across the loop
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      const int row = r0 + 16 * rt;
      const bool ok = row < R;
      const size_t qb = (size_t)cur_b * R + (ok ? row : 0);
#pragma unroll
      for (int ks = 0; ks < 16; ++ks)
        qreg[rt][ks] = ok ? load_q8(p.q_lat, qb * 512 + ks * 32 + lg_ * 8, QF32) : bf16x8{};
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
        qreg[rt][16 + ks] = ok ? load_q8(p.q_rope, qb * 64 + ks * 32 + lg_ * 8, QF32) : bf16x8{};
      lim[rt] = ok ? L - p.s_q + row / p.H : -1;
      m_s[rt] = NEG_INF;
      l_x[rt] = 0.f;
    }
    lim_all = L - p.s_q;
    fresh = true;   // the first step's P.V MFMAs start the accumulators from zero
    // wait here, on this rare path: a load the compiler sees pending at the loop's back edge
    // would make it wait for every stage in flight at the top of every step
    if (wait) __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
  };
  // The first piece's queries are loaded now, so that their latency overlaps the block-table
  // loads below, and both are complete before the stage ring starts: the compiler, which does
  // not see the ring's DMA, would otherwise wait for every stage in flight before using Q.
  {
    const int b0 = seq_of(start);
    start_piece(b0, tabL[b0], false);   // completed with the block-table loads below
  }

  // ---- stage table: position j = start + tid -> its sequence and, for a cache block, its
  // rank k among the range's blocks (a workgroup scan), block id and tokens
  {
    const int j = start + tid;
    int b = 0, jb = -1;
    int Ls = 0, Lm = 0, Lr = 0;
    if (j < end) {
      b = seq_of(j);
      int n;
      if constexpr (MIXED) {
        part_lens(b, Ls, Lm, Lr);
        n = nblocks(Ls) + nblocks(Lm) + nblocks(Lr);
      } else {
        n = nblocks(tabL[b]);
      }
      jb = j - (tabP[b + 1] - n);   // < 0: a phantom
    }
    const int is_blk = jb >= 0 ? 1 : 0;
    int x = is_blk;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(x, o, 64);
      if (lane >= o) x += y;
    }
    if (lane == 63) sh_scan[w] = x;
    __syncthreads();
    int woff = 0, tot = 0;
#pragma unroll
    for (int i = 0; i < NT / 64; ++i) {
      woff += i < w ? sh_scan[i] : 0;
      tot += sh_scan[i];
    }
    const int k = woff + x - is_blk;
    if (is_blk) {
      const int L = tabL[b];
      int part = 1, jl = jb, Lp = L;   // the block's part, its index there and the part's tokens
      const int32_t* bt = p.block_table;
      int64_t bts = p.bt_stride, nbp = p.num_blocks;
      if constexpr (MIXED) {
        const int nS = nblocks(Ls), nM = nblocks(Lm);
        if (jb < nS) {
          part = 0;
          Lp = Ls;
        } else if (jb < nS + nM) {
          jl = jb - nS;
          Lp = Lm;
        } else {
          part = 2;
          jl = jb - nS - nM;
          Lp = Lr;
        }
        if (part != 1) {
          // fields picked by selects: a kernel argument indexed at run time goes to scratch
          const bool rec = part == 2;
          bt = rec ? p.hi[1].block_table : p.hi[0].block_table;
          bts = rec ? p.hi[1].bt_stride : p.hi[0].bt_stride;
          nbp = rec ? p.hi[1].num_blocks : p.hi[0].num_blocks;
        }
      }
      int id = bt[(size_t)b * bts + jl];
      int v = min(BLOCK_TOKENS, Lp - jl * BLOCK_TOKENS);
      if (id < 0 || (int64_t)id >= nbp) {
        id = 0;
        v = 0;
      }
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int kk = 2 * k + h;
        const int valid = min(ST_TOK, max(0, v - ST_TOK * h));
        int info = b | (valid << 20) | (MIXED ? part << INFO_PART : 0);
        if (h == 0 && (k == 0 || jb == 0)) info |= INFO_START;
        if (h == 1 && (k == tot - 1 || j == tabP[b + 1] - 1)) info |= INFO_END;
        st_bid[kk] = id;
        st_tok[kk] = jb * BLOCK_TOKENS + ST_TOK * h;
        st_info[kk] = info;
        st_len[kk] = L;
      }
    }
    if (tid == 0) sh_scan[NT / 64] = tot;
  }
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
  __syncthreads();
  const int nblk = sh_scan[NT / 64];   // cache blocks of the range, <= MAX_RANGE_BLOCKS
  if (nblk == 0) return;               // phantom positions only
  const int nst = 2 * nblk;

  // ---- stages
  const uint32_t smem_base = lds_addr(smem);
  const QuantPlanes pl{(int)p.off_lc, (int)p.off_ls, (int)p.off_rc, (int)p.off_rs};
  const int groups = 512 >> p.g_lat_log2, rgroups = 64 >> p.g_rope_log2;
  // ring slot addresses: bf16 stage slot k at k * ST_BYTES; quantised: bf16 stages 0, 1, then
  // code slot k at 2 * ST_BYTES + k * CBYTES
  auto bf_stage = [&](int k) -> bf16_t* { return (bf16_t*)(smem + k * ST_BYTES); };
  auto code_slot = [&](int k) -> int { return 2 * ST_BYTES + k * CBYTES; };
  constexpr int LOADS = QUANT ? QS::LOADS : BfProducer::LOADS;
  // source of stage s: its block and which half (wave-uniform)
  struct Src {
    const uint8_t* blk;
    int half;
  };
  // the cache of a part (mixed histories: 0 sink, 1 middle, 2 recent window)
  auto part_block = [&](int part, int id) -> const uint8_t* {
    if (MIXED && part != 1) {
      const bool rec = part == 2;
      return (rec ? p.hi[1].pool : p.hi[0].pool) + (size_t)id * (size_t)(rec ? p.hi[1].block_bytes : p.hi[0].block_bytes);
    }
    return p.pool + (size_t)id * (size_t)p.block_bytes;
  };
  auto part_of = [](int info) { return MIXED ? (info >> INFO_PART) & 3 : 1; };
  auto src_of = [&](int s) {
    const int id = __builtin_amdgcn_readfirstlane(st_bid[s]);
    const int half = (__builtin_amdgcn_readfirstlane(st_tok[s]) / ST_TOK) & 1;
    if constexpr (MIXED) return Src{part_block(part_of(__builtin_amdgcn_readfirstlane(st_info[s])), id), half};
    else return Src{p.pool + (size_t)id * (size_t)p.block_bytes, half};
  };
  // per-lane DMA source offsets (held for the whole kernel) and this wave's LDS slice
  const uint32_t wlds = (uint32_t)__builtin_amdgcn_readfirstlane((tid & ~63) * 16);
  const auto offs = [&] {
    if constexpr (QUANT) return QS::offsets(pl, groups, rgroups, tid);
    else return BfProducer::offsets(tid);
  }();
  // DMA instruction i of stage s
  auto issue_one = [&](int s, const Src& sr, int i) {
    if constexpr (QUANT) {
      QS::issue_one(i, offs, sr.blk, sr.half, smem_base + code_slot(s % DEPTH) + wlds);
    } else {
      BfProducer::issue_one(i, offs, sr.blk + sr.half * ST_TOK * 1152, smem_base + (s & 3) * ST_BYTES + wlds);
    }
  };
  auto issue = [&](int s) {
    const Src sr = src_of(s);
#pragma unroll
    for (int i = 0; i < LOADS; ++i) issue_one(s, sr, i);
  };
  // wait until a stage has landed, given how many later stages were issued after it
  auto wait_stage = [&](int later) {
    auto wait_k = [&](auto K) {
      constexpr int k = decltype(K)::value;
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(k * LOADS));
    };
    switch (later) {
      case 0: wait_k(std::integral_constant<int, 0>{}); break;
      case 1: wait_k(std::integral_constant<int, 1>{}); break;
      case 2: wait_k(std::integral_constant<int, 2>{}); break;
      case 3: wait_k(std::integral_constant<int, 3>{}); break;
      case 4: wait_k(std::integral_constant<int, 4>{}); break;
      case 5: wait_k(std::integral_constant<int, 5>{}); break;
      case 6: wait_k(std::integral_constant<int, 6>{}); break;
      default: wait_k(std::integral_constant<int, 7>{}); break;
    }
  };
  static_assert((QUANT ? DEPTH - 1 : 2) <= 7 && 7 * LOADS <= 63, "stage waits out of range");

  // ---- shared stage kernels of the two loops below

  // scores S^T[token][row] of the stage at KS for token tiles tt and row tiles rt; hook(ks)
  // runs after k-step ks
  auto score_stage = [&](const bf16_t* KS, f32x4(&sc)[2][RT], auto&& hook) MLA_INLINE {
    const bf16_t* kb[2][2];
    int lr_ = lr;
    asm volatile("" : "+v"(lr_));   // recomputed per stage rather than held across the loop
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      const int t = tt * 16 + lr_;
      const int f = rsw(t);
      kb[tt][0] = KS + t * 576 + (lg ^ f) * 8;
      kb[tt][1] = KS + t * 576 + ((4 + lg) ^ f) * 8 - 32;
    }
    constexpr int KD = 1;   // prefetch depth in k-steps (deeper gains nothing: the loop is MFMA-issue bound)
    bf16x8 a[KD + 1][2];
#pragma unroll
    for (int i = 0; i < KD; ++i)
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) a[i][tt] = *(const bf16x8*)(kb[tt][i & 1] + i * 32);
    // per k-step: read, MFMA pair (token tile 0), read, MFMA pair (token tile 1): reads issued
    // between MFMAs keep the matrix pipe busier than reads grouped before four MFMAs
#pragma unroll
    for (int ks = 0; ks < 18; ++ks) {
      const int nx = (ks + KD) % (KD + 1), cu = ks % (KD + 1);
      if (ks + KD < 18) a[nx][0] = *(const bf16x8*)(kb[0][(ks + KD) & 1] + (ks + KD) * 32);
      if (ks == 0) score2<true, true, false>(sc[0][0], sc[0][1], a[cu][0], qreg[0][ks], qreg[1][ks]);
      else score2<false, false, false>(sc[0][0], sc[0][1], a[cu][0], qreg[0][ks], qreg[1][ks]);
      __builtin_amdgcn_sched_barrier(0);
      if (ks + KD < 18) a[nx][1] = *(const bf16x8*)(kb[1][(ks + KD) & 1] + (ks + KD) * 32);
      if (ks == 0) score2<true, false, false>(sc[1][0], sc[1][1], a[cu][1], qreg[0][ks], qreg[1][ks]);
      else if (ks == 17) score2<false, false, true>(sc[1][0], sc[1][1], a[cu][1], qreg[0][ks], qreg[1][ks]);
      else score2<false, false, false>(sc[1][0], sc[1][1], a[cu][1], qreg[0][ks], qreg[1][ks]);
      __builtin_amdgcn_sched_barrier(0);
      hook(ks);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // O^T[col][row] += V^T[col][token] . P^T[token][row] over the stage at KS (FRESH: the first
  // stage of a piece, the accumulators start from zero); P^T is the pair of bf16 terms pp, ppl.
  // hook(j) (j a compile-time constant) runs after MFMA j of the 128.  The 8 tokens of lane
  // group lg are 4 lg .. 4 lg + 3 (first read) and 16 + 4 lg .. 16 + 4 lg + 3 (second read).
  auto pv_stage = [&](auto FRESH, const bf16_t* KS, const bf16x8(&pp)[RT], const bf16x8(&ppl)[RT], auto&& hook) MLA_INLINE {
    constexpr bool F = decltype(FRESH)::value;
    // column d = 16 nt + 4 (lr & 3) of token t is element rst_off(t, d); with nt = 4 q + r its
    // piece is (2 nt + h) ^ rsw(t) = 8 q + ((2 r + h) ^ rsw(t)), h = (lr & 3) / 2, since
    // rsw < 8: four per-lane bases (r) and an immediate offset of 64 q elements.  Token
    // tb = ta + 16 has rsw(tb) = rsw(ta): its pieces sit exactly 16 rows further on (db).
    int lane_ = lane;
    asm volatile("" : "+v"(lane_));   // recomputed per stage rather than held across the loop
    const int lrp = lane_ & 15, lgp = lane_ >> 4;
    const int ta = 4 * lgp + (lrp >> 2);
    const int h = (lrp & 3) >> 1, fa = rsw(ta);
    constexpr int db = 16 * 576;
    int oa[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) oa[r] = ta * 576 + (((2 * r + h) ^ fa) << 3) + (lrp & 1) * 4;
    // software pipeline: the two halves of the V^T fragment of tile nt + PD are read between
    // the MFMAs of tile nt
    auto rlo = [&](int nt) {
      return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)&KS[oa[nt & 3] + 64 * (nt >> 2)]);
    };
    auto rhi = [&](int nt) {
      return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)&KS[oa[nt & 3] + db + 64 * (nt >> 2)]);
    };
    constexpr int PD = 2;   // prefetch depth
    i16x4 lo[PD + 1], hi[PD + 1];
#pragma unroll
    for (int i = 0; i < PD; ++i) {
      lo[i] = rlo(i);
      hi[i] = rhi(i);
    }
    static_for<32>([&](auto NT_) MLA_INLINE {
      constexpr int nt = decltype(NT_)::value;
      constexpr int cu = nt % (PD + 1), nx = (nt + PD) % (PD + 1);
      const bf16x8 v = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo[cu], hi[cu], 0, 1, 2, 3, 4, 5, 6, 7));
      if constexpr (nt + PD < 32) lo[nx] = rlo(nt + PD);
      pv1<F, nt == 0, false>(acc[0][nt], v, pp[0]);
      hook(std::integral_constant<int, 4 * nt>{});
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (nt + PD < 32) hi[nx] = rhi(nt + PD);
      pv1<F, false, false>(acc[1][nt], v, pp[1]);
      hook(std::integral_constant<int, 4 * nt + 1>{});
      __builtin_amdgcn_sched_barrier(0);
      pv1<false, false, false>(acc[0][nt], v, ppl[0]);
      hook(std::integral_constant<int, 4 * nt + 2>{});
      __builtin_amdgcn_sched_barrier(0);
      pv1<false, false, nt == 31>(acc[1][nt], v, ppl[1]);
      hook(std::integral_constant<int, 4 * nt + 3>{});
      __builtin_amdgcn_sched_barrier(0);
    });
  };
  auto no_hook = [](auto) {};

  // acc[rt] *= a[rt] (a row's running maximum moved)
  auto rescale = [&](const float(&a)[RT]) MLA_INLINE {
    const uint32_t sa = lds_addr(&resc[tid]);
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int q = 0; q < 32; q += 8)
        scale_tiles8(acc[rt][q], acc[rt][q + 1], acc[rt][q + 2], acc[rt][q + 3], acc[rt][q + 4], acc[rt][q + 5],
                     acc[rt][q + 6], acc[rt][q + 7], a[rt], sa);
  };

  // acc = 0 (the bf16 loop starts every piece from zeroed accumulators)
  auto zero_acc = [&]() MLA_INLINE {
    bf16x8 zz{};
    asm volatile("" : "+v"(zz));   // materialised once, here
    static_for<2 * 32>([&](auto K) MLA_INLINE {
      constexpr int k = decltype(K)::value;
      zero_tile<k == 0, k == 63>(acc[k >> 5][k & 31], zz);
    });
  };

  // end of a piece of sequence b: this wave's rows, unnormalised, with 1 / sum(P) and the lse
  // (m: running maximum, l: this lane's share of sum(P)), to slot b + range; the combine
  // normalises (a range's pieces have distinct slots)
  auto store_piece = [&](int b, const float(&m)[RT], const float(&l)[RT]) MLA_INLINE {
    const size_t slot = (size_t)b + range;
    int r0 = row0;
    asm volatile("" : "+v"(r0));   // addresses recomputed here rather than held across the loop
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      const int row = r0 + 16 * rt;
      const float lx = sum_lg(l[rt]);
      if (row < R) {
        float* o = p.part_o + (slot * R + row) * 512 + 4 * lg;
#pragma unroll
        for (int nt = 0; nt < 32; ++nt) store_tile(o + nt * 16, acc[rt][nt]);
        if (lg == 0) {
          p.part_lse[slot * R + row] = lx > 0.f ? (m[rt] + __log2f(lx)) * 0.69314718055994531f : NEG_INF;
          p.part_inv[slot * R + row] = lx > 0.f ? 1.f / lx : 0.f;
        }
      }
    }
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));   // as at a piece start: nothing left pending
  };

  // The range's last piece, after the loop, as fp16: the stage ring is free, so each wave
  // moves a row tile's 32 accumulator tiles through its 32 KB of the ring into VGPRs, reading
  // them back as 8 consecutive columns of its row per 16-byte chunk (lane lg takes chunks
  // lg, lg + 4, ..).  Each row is scaled by 2^-e so that its largest |o / sum(P)| lies in
  // [2^14, 2^15), rounded to fp16 (RNE: error at most 2^-11 of the row's largest value) and
  // stored row-major in the first half of its fp32 row; part_inv holds -2^e (the sign marks
  // the format for the combine).
  auto store_piece16 = [&](int b, const float(&m)[RT], const float(&l)[RT]) MLA_INLINE {
    const size_t slot = (size_t)b + range;
    int r0 = row0;
    asm volatile("" : "+v"(r0));
    const uint32_t wreg = (uint32_t)__builtin_amdgcn_readfirstlane(lds_addr(smem) + (uint32_t)w * 32768u);
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      const uint32_t put = wreg + (uint32_t)lane * 16u;
      static_for<32>([&](auto NT_) MLA_INLINE {
        constexpr int nt = decltype(NT_)::value;
        lds_put_tile<nt * 1024>(put, acc[rt][nt]);
      });
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      // chunk q = 4 j + lg of row lr: columns 8 q .. 8 q + 7 = tile q / 2, lane groups
      // 2 (q & 1) and 2 (q & 1) + 1 of that tile
      f32x4 v[32];
      const uint8_t* reg = smem + (size_t)w * 32768u;
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int q = 4 * j + lg;
        const int t = q >> 1, g0 = 2 * (q & 1);
        v[2 * j] = *(const f32x4*)(reg + t * 1024 + (lr + 16 * g0) * 16);
        v[2 * j + 1] = *(const f32x4*)(reg + t * 1024 + (lr + 16 * (g0 + 1)) * 16);
      }
      float mx = 0.f;
#pragma unroll
      for (int j = 0; j < 32; ++j) mx = fmaxf(mx, fmaxf(fmaxf(fabsf(v[j][0]), fabsf(v[j][1])), fmaxf(fabsf(v[j][2]), fabsf(v[j][3]))));
      mx = max_lg(mx);
      const float lx = sum_lg(l[rt]);
      const float il = lx > 0.f ? 1.f / lx : 0.f;
      const float a = mx * il;
      // e: a 2^-e in [2^14, 2^15) (a > 0), clamped so that 2^-e and 2^e stay normal floats
      int e = a > 0.f ? (int)((__float_as_uint(a) >> 23) & 0xFF) - 127 - 14 : 0;
      e = e < -100 ? -100 : (e > 100 ? 100 : e);
      const float f = il * __uint_as_float((uint32_t)(127 - e) << 23);
      const int row = r0 + 16 * rt;
      if (row < R) {
        uint16_t* o16 = (uint16_t*)(p.part_o + (slot * R + row) * 512);
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          u32x4 h;
          h[0] = pack_f16x2(v[2 * j][0] * f, v[2 * j][1] * f);
          h[1] = pack_f16x2(v[2 * j][2] * f, v[2 * j][3] * f);
          h[2] = pack_f16x2(v[2 * j + 1][0] * f, v[2 * j + 1][1] * f);
          h[3] = pack_f16x2(v[2 * j + 1][2] * f, v[2 * j + 1][3] * f);
          *(u32x4*)(o16 + (4 * j + lg) * 8) = h;
        }
        if (lg == 0) {
          p.part_lse[slot * R + row] = lx > 0.f ? (m[rt] + __log2f(lx)) * 0.69314718055994531f : NEG_INF;
          p.part_inv[slot * R + row] = -__uint_as_float((uint32_t)(127 + e) << 23);
        }
      }
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // every read of the region done before it is reused
    }
  };

  // softmax of rows row0 + 16 rt over one stage's scores sc (this lane holds tokens 16 tt +
  // 4 lg + i) in one piece: P^T operands pt (high bf16 terms) and ptl (low terms), the
  // accumulator factor al, the running maximum m_s and sum l_x updated.  MASK: token k of the
  // stage is kept if k < valid and stok + k <= lim (otherwise every token of the stage is
  // visible to every row).
  auto softmax = [&](auto MASK, f32x4(&sc)[2][RT], int valid, int stok, bf16x8(&pt)[RT], bf16x8(&ptl)[RT],
                     float(&al)[RT]) MLA_INLINE {
    constexpr bool M = decltype(MASK)::value;
    float mt[RT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      const int kb4 = 4 * lg;
      const int lim_k = min(valid - 1, lim[rt] - stok);
      mt[rt] = NEG_INF;
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if constexpr (!M) {
            sc[tt][rt][i] *= p.scale_log2;
          } else {
            const bool ok = kb4 <= lim_k - (16 * tt + i);
            sc[tt][rt][i] = ok ? sc[tt][rt][i] * p.scale_log2 : NEG_INF;
          }
          mt[rt] = fmaxf(mt[rt], sc[tt][rt][i]);
        }
    }
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) mt[rt] = max_lg(mt[rt]);
    // a rescale costs the same however many of the wave's rows move: once one row must move,
    // every row takes its current maximum, which spares the later rescales that rows reaching
    // higher scores one by one would each cost (a piece that opens on low scores)
    bool up = false;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) up |= mt[rt] > m_s[rt] + ROWS_SLACK;
    const bool move = __any(up);
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      const float mn = move && mt[rt] > m_s[rt] ? mt[rt] : m_s[rt];
      const float mu = mn == NEG_INF ? 0.f : mn;
      // while m_s = -inf every P so far was 0 and the accumulators hold zeros: nothing to scale
      al[rt] = (mn == m_s[rt] || m_s[rt] == NEG_INF) ? 1.f : __builtin_amdgcn_exp2f(m_s[rt] - mu);
      l_x[rt] *= al[rt];
      m_s[rt] = mn;
      uint32_t pw[4], pl[4];
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        float pf[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          pf[i] = __builtin_amdgcn_exp2f(sc[tt][rt][i] - mu);
          l_x[rt] += pf[i];
        }
        split_pair(pf[0], pf[1], pw[2 * tt], pl[2 * tt]);
        split_pair(pf[2], pf[3], pw[2 * tt + 1], pl[2 * tt + 1]);
      }
      pt[rt] = __builtin_bit_cast(bf16x8, u32x4{pw[0], pw[1], pw[2], pw[3]});
      ptl[rt] = __builtin_bit_cast(bf16x8, u32x4{pl[0], pl[1], pl[2], pl[3]});
    }
  };
  // rows past the sequence end in ring slot k came from a stand-in address: zero them
  auto zero_tail = [&](int k, int valid) MLA_INLINE {
    bf16_t* Z = bf_stage(k);
    for (int q = tid; q < (ST_TOK - valid) * 72; q += NT)
      *(u32x4*)&Z[(valid + q / 72) * 576 + (q % 72) * 8] = u32x4{0, 0, 0, 0};
    lds_barrier();
  };

  if constexpr (!QUANT) {
    // ---- bf16: a software pipeline over the 4-slot ring.  Step s scores stage s + 1, then
    // takes the P.V products of stage s with the softmax of stage s + 1 spread between its
    // MFMAs: a SIMD issues for one wave here, and vector-ALU work overlaps the matrix pipe
    // only when it sits between independent MFMAs.  Stage s + 3 is issued into the slot of
    // stage s - 1 (free since the barrier closing step s - 1) during the scores; the step
    // ends once stage s + 2 has landed.
    for (int s = 0; s < 3 && s < nst; ++s) issue(s);
    zero_acc();   // while the first stages are in flight
    wait_stage(min(nst - 1, 2));
    lds_barrier();
    int info_c = __builtin_amdgcn_readfirstlane(st_info[0]);
    f32x4 sc[2][RT];
    bf16x8 pt[RT], ptl[RT];
    {
      const int valid0 = (info_c >> 20) & 63;
      const int stok0 = __builtin_amdgcn_readfirstlane(st_tok[0]);
      if (valid0 < ST_TOK) zero_tail(0, valid0);
      score_stage(bf_stage(0), sc, no_hook);
      float al0[RT];   // a piece's first stage: nothing to rescale
      if (valid0 == ST_TOK && stok0 + (ST_TOK - 1) <= lim_all) softmax(std::false_type{}, sc, valid0, stok0, pt, ptl, al0);
      else softmax(std::true_type{}, sc, valid0, stok0, pt, ptl, al0);
    }
    if (nst > 1) wait_stage(min(nst - 1, 2) - 1);
    lds_barrier();
    // stage-table entries of the next step, read at the end of the step before
    int n_info = st_info[min(nst - 1, 1)], n_tok = st_tok[min(nst - 1, 1)];
    int n_bid = st_bid[min(nst - 1, 3)], n_btok = st_tok[min(nst - 1, 3)];
    float m_e[RT], l_e[RT];   // state of the piece ending with stage s
    int fin_b = 0;            // the sequence of the range's last piece
    for (int s = 0; s < nst; ++s) {
      const bool has_n = s + 1 < nst;
      const int info_n = __builtin_amdgcn_readfirstlane(n_info);
      const int valid_n = (info_n >> 20) & 63;
      const int stok_n = __builtin_amdgcn_readfirstlane(n_tok);
      const bool refill = s + 3 < nst;
      const Src sr_new{p.pool + (size_t)__builtin_amdgcn_readfirstlane(n_bid) * (size_t)p.block_bytes,
                       (__builtin_amdgcn_readfirstlane(n_btok) / ST_TOK) & 1};
      if (s > 0 && (info_c & INFO_START)) zero_acc();   // a new piece starts from zero
      if (info_c & INFO_END) {
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
          m_e[rt] = m_s[rt];
          l_e[rt] = l_x[rt];
        }
      }
      if (has_n) {
        if (valid_n < ST_TOK) zero_tail((s + 1) & 3, valid_n);
        // a new piece: its queries and a fresh softmax state (the ending piece's is in m_e, l_e)
        if (info_n & INFO_START) start_piece(info_n & 0xFFFFF, __builtin_amdgcn_readfirstlane(st_len[s + 1]), true);
        score_stage(bf_stage((s + 1) & 3), sc, [&](int ks) {
          if ((ks & 1) && refill) issue_one(s + 3, sr_new, ks >> 1);
        });
      }

      // Softmax of stage s + 1 in steps of one or two vector instructions, step c after P.V
      // MFMA c (MASK: after MFMA c + 1; the masking, when needed, after MFMA 0).  An MFMA holds
      // its wave's issue for most of its cycles: about one vector instruction per MFMA comes for
      // free, so the steps are spread thinly.  Steps 0..7: row maxima (r alternating); 8..15:
      // the lane-group reductions; 16..29: new running maximum and accumulator factor; then six
      // steps per pair of tokens (e0, e1) = (2 jj, 2 jj + 1) of row tile r, pairs in the order
      // (jj, r): two exponentials, the sums and the high term, the residuals, the low term.  A
      // pair's scores die as its P^T words are made, so the register peak stays low.
      float aln[RT], mt[RT], thr[RT], mn[RT], mu[RT], ex[RT], pf0[RT], pf1[RT], d0[RT], d1[RT], sw0[RT], sw1[RT];
      uint32_t pw[RT][4], pl[RT][4];
      auto X = [&](int r, int e) -> float { return sc[e >> 2][r][e & 3]; };
      auto chunk = [&](auto C) MLA_INLINE {
        constexpr int c = decltype(C)::value;
        if constexpr (c < 8) {
          constexpr int r = c & 1, k = c >> 1;
          if constexpr (k == 0) mt[r] = vmax3(X(r, 0), X(r, 1), X(r, 2));
          else if constexpr (k == 1) mt[r] = vmax3(mt[r], X(r, 3), X(r, 4));
          else if constexpr (k == 2) mt[r] = vmax3(mt[r], X(r, 5), X(r, 6));
          else mt[r] = vmax(mt[r], X(r, 7));
          pin(mt[r]);
        } else if constexpr (c < 16) {
          constexpr int r = (c >> 1) & 1, lvl = (c - 8) >> 2;
          if constexpr ((c & 1) == 0) {
            const auto t = lvl == 0 ? __builtin_amdgcn_permlane32_swap(__float_as_uint(mt[r]), __float_as_uint(mt[r]), false, false)
                                    : __builtin_amdgcn_permlane16_swap(__float_as_uint(mt[r]), __float_as_uint(mt[r]), false, false);
            sw0[r] = __uint_as_float(t[0]);
            sw1[r] = __uint_as_float(t[1]);
            pin(sw0[r]);
            pin(sw1[r]);
          } else {
            mt[r] = vmax(sw0[r], sw1[r]);
            pin(mt[r]);
          }
        } else if constexpr (c < 30) {
          constexpr int r = c & 1, k = (c - 16) >> 1;
          if constexpr (k == 0) {
            mt[r] *= p.scale_log2;
            thr[r] = m_s[r] + ROWS_SLACK;
            pin(mt[r]);
            pin(thr[r]);
          } else if constexpr (k == 1) {
            mn[r] = mt[r] > thr[r] ? mt[r] : m_s[r];
            pin(mn[r]);
          } else if constexpr (k == 2) {
            mu[r] = mn[r] == NEG_INF ? 0.f : mn[r];
            pin(mu[r]);
          } else if constexpr (k == 3) {
            ex[r] = __builtin_amdgcn_exp2f(m_s[r] - mu[r]);
            pin(ex[r]);
          } else if constexpr (k == 4) {
            aln[r] = mn[r] == m_s[r] ? 1.f : ex[r];
            pin(aln[r]);
          } else if constexpr (k == 5) {
            // while m_s = -inf every P so far was 0 and the accumulators hold zeros
            aln[r] = m_s[r] == NEG_INF ? 1.f : aln[r];
            pin(aln[r]);
          } else {
            l_x[r] *= aln[r];
            m_s[r] = mn[r];
            pin(l_x[r]);
            pin(m_s[r]);
          }
        } else {
          constexpr int q = (c - 30) / 6, k = (c - 30) % 6;
          constexpr int r = q & 1, jj = q >> 1;
          if constexpr (k == 0) {
            pf0[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(X(r, 2 * jj), p.scale_log2, -mu[r]));
            pin(pf0[r]);
          } else if constexpr (k == 1) {
            pf1[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(X(r, 2 * jj + 1), p.scale_log2, -mu[r]));
            pin(pf1[r]);
          } else if constexpr (k == 2) {
            l_x[r] += pf0[r];
            pw[r][jj] = pack_bf16x2(pf0[r], pf1[r]);
            pin(l_x[r]);
            pin(pw[r][jj]);
          } else if constexpr (k == 3) {
            l_x[r] += pf1[r];
            d0[r] = pf0[r] - __uint_as_float(pw[r][jj] << 16);
            pin(l_x[r]);
            pin(d0[r]);
          } else if constexpr (k == 4) {
            d1[r] = pf1[r] - __uint_as_float(pw[r][jj] & 0xFFFF0000u);
            pin(d1[r]);
          } else {
            pl[r][jj] = pack_bf16x2(d0[r], d1[r]);
            pin(pl[r][jj]);
          }
        }
      };
      constexpr int NCHUNK = 30 + 6 * 8;
      const bool mask_n = !(valid_n == ST_TOK && stok_n + (ST_TOK - 1) <= lim_all);
      auto hook = [&](auto J) MLA_INLINE {
        constexpr int j = decltype(J)::value;
        if constexpr (j == 0) {
          if (mask_n) {
#pragma unroll
            for (int r = 0; r < RT; ++r) {
              const int d = min(valid_n - 1, lim[r] - stok_n) - 4 * lg;
#pragma unroll
              for (int e = 0; e < 8; ++e) sc[e >> 2][r][e & 3] = d >= 16 * (e >> 2) + (e & 3) ? X(r, e) : NEG_INF;
              pin(sc[0][r]);
              pin(sc[1][r]);
            }
          }
        } else if constexpr (j <= NCHUNK) {
          chunk(std::integral_constant<int, j - 1>{});
        }
      };
      pv_stage(std::false_type{}, bf_stage(s & 3), pt, ptl, hook);
      if ((info_c & INFO_END) && s + 1 < nst) store_piece(info_c & 0xFFFFF, m_e, l_e);
      if (s + 1 == nst) fin_b = info_c & 0xFFFFF;
      if (has_n) {
        if (!(info_n & INFO_START) && __any(aln[0] != 1.f || aln[1] != 1.f)) rescale(aln);
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
          pt[rt] = __builtin_bit_cast(bf16x8, u32x4{pw[rt][0], pw[rt][1], pw[rt][2], pw[rt][3]});
          ptl[rt] = __builtin_bit_cast(bf16x8, u32x4{pl[rt][0], pl[rt][1], pl[rt][2], pl[rt][3]});
        }
      }
      info_c = info_n;
      if (s + 2 < nst) {
        n_info = st_info[s + 2];
        n_tok = st_tok[s + 2];
        n_bid = st_bid[min(nst - 1, s + 4)];
        n_btok = st_tok[min(nst - 1, s + 4)];
        // stage s + 2 has landed and nobody reads stage s any more
        wait_stage(min(nst - 1, s + 3) - (s + 2));
      }
      lds_barrier();
    }
    store_piece16(fin_b, m_e, l_e);
  } else {
    // ---- quantised: codes 0..DEPTH-1 in flight, code 0 dequantised into bf16 stage 0, code 1
    // landed.  Step s dequantises code s + 1 into the other bf16 stage, then scores, softmax
    // and P.V of stage s; code s + DEPTH refills the slot of code s.
    // mixed histories: the bf16 rows of stage s by DMA into its bf16 slot (no code to dequantise)
    auto issue_bf = [&](int s) {
      const Src sr = src_of(s);
      const auto bo = BfProducer::offsets(tid);
#pragma unroll
      for (int i = 0; i < BfProducer::LOADS; ++i)
        BfProducer::issue_one(i, bo, sr.blk + sr.half * ST_TOK * 1152, smem_base + (s & 1) * ST_BYTES + wlds);
    };
    for (int s = 0; s < DEPTH && s < nst; ++s) issue(s);
    const int info0 = __builtin_amdgcn_readfirstlane(st_info[0]);
    if (part_of(info0) != 1) {
      issue_bf(0);
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
      lds_barrier();
      if (((info0 >> 20) & 63) < ST_TOK) zero_tail(0, (info0 >> 20) & 63);
    } else {
      wait_stage(min(nst - 1, DEPTH - 1));
      lds_barrier();
      QS::dequant(smem + code_slot(0), (info0 >> 20) & 63, p.g_lat_log2, p.g_rope_log2, bf_stage(0), tid);
      if (nst > 1) wait_stage(min(nst - 1, DEPTH - 1) - 1);
    }
    lds_barrier();

    // stage-table entries of step s, read at the end of step s - 1 so that their LDS latency
    // overlaps the end-of-step wait
    int n_info = st_info[0], n_tok = st_tok[0];
    int n_bid = st_bid[min(nst - 1, DEPTH)], n_btok = st_tok[min(nst - 1, DEPTH)];
    int n_bpart = MIXED ? st_info[min(nst - 1, DEPTH)] : 0;
    for (int s = 0; s < nst; ++s) {
      const int info = __builtin_amdgcn_readfirstlane(n_info);
      const int valid = (info >> 20) & 63;
      const int stok = __builtin_amdgcn_readfirstlane(n_tok);
      if (s > 0 && (info & INFO_START)) start_piece(info & 0xFFFFF, __builtin_amdgcn_readfirstlane(st_len[s]), true);
      const int s_new = s + DEPTH;
      const bool refill = s_new < nst;
      const Src sr_new{MIXED ? part_block(part_of(__builtin_amdgcn_readfirstlane(n_bpart)), __builtin_amdgcn_readfirstlane(n_bid))
                             : p.pool + (size_t)__builtin_amdgcn_readfirstlane(n_bid) * (size_t)p.block_bytes,
                       (__builtin_amdgcn_readfirstlane(n_btok) / ST_TOK) & 1};
      const bf16_t* KS = bf_stage(s & 1);
      // dequantise the next stage while this one is consumed: its code stage has landed and
      // its bf16 slot was last read in step s - 1 (a bf16 block of a mixed history: its DMA
      // into that slot, complete at the end of this step)
      int info1 = 0;
      bool bf_next = false;
      if (s + 1 < nst) {
        info1 = __builtin_amdgcn_readfirstlane(st_info[s + 1]);
        if (MIXED && part_of(info1) != 1) {
          bf_next = true;
          issue_bf(s + 1);
        } else {
          QS::dequant(smem + code_slot((s + 1) % DEPTH), (info1 >> 20) & 63, p.g_lat_log2, p.g_rope_log2,
                      bf_stage((s + 1) & 1), tid);
        }
      }

      f32x4 sc[2][RT];
      score_stage(KS, sc, [](int) {});
      bf16x8 pt[RT], ptl[RT];
      float al[RT];
      if (valid == ST_TOK && stok + (ST_TOK - 1) <= lim_all) softmax(std::false_type{}, sc, valid, stok, pt, ptl, al);
      else softmax(std::true_type{}, sc, valid, stok, pt, ptl, al);
      if (!fresh && __any(al[0] != 1.f || al[1] != 1.f)) rescale(al);
      if (fresh) pv_stage(std::true_type{}, KS, pt, ptl, no_hook);
      else pv_stage(std::false_type{}, KS, pt, ptl, no_hook);
      fresh = false;
      if ((info & INFO_END) && s + 1 < nst) store_piece(cur_b, m_s, l_x);

      if (s + 1 < nst) {
        n_info = st_info[s + 1];
        n_tok = st_tok[s + 1];
        n_bid = st_bid[min(nst - 1, s + 1 + DEPTH)];
        n_btok = st_tok[min(nst - 1, s + 1 + DEPTH)];
        if constexpr (MIXED) n_bpart = st_info[min(nst - 1, s + 1 + DEPTH)];
      }
      // the refill of this step, issued where the wave waits anyway: an issue blocks while many
      // reads are outstanding, and between MFMAs that stalls the matrix pipe
      if (refill) {
#pragma unroll
        for (int i = 0; i < LOADS; ++i) issue_one(s_new, sr_new, i);
      }
      // the next step's stage has landed and nobody reads stage s any more
      if (bf_next) {
        // the bf16 rows of stage s + 1 (issued before this step's refill) and every code stage
        if (refill) __builtin_amdgcn_s_waitcnt(vmcnt_imm(LOADS));
        else __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
        lds_barrier();
        if (((info1 >> 20) & 63) < ST_TOK) zero_tail((s + 1) & 1, (info1 >> 20) & 63);
      } else if (s + 2 < nst) {
        wait_stage(min(nst - 1, s + DEPTH) - (s + 2));
      }
      lds_barrier();
    }
    store_piece16(cur_b, m_s, l_x);
  }
}

// The in-loop dequantisation of this kernel on its own (test/debug): one workgroup per half
// block streams the code planes with QuantStage's DMA (the same per-lane offsets), dequantises
// them with QuantStage::dequant into a bf16 stage of this kernel's swizzle, and copies the
// stage out un-swizzled.  Block ids outside the pool give zero rows (zero scales).
template <int FMT>
__global__ __launch_bounds__(NT) void dequant_stage_rows_kernel(DequantParams p) {
  using QS = QuantStage<FMT>;
  __shared__ __attribute__((aligned(16))) uint8_t cst[QS::SLOTS * 16];
  __shared__ __attribute__((aligned(16))) bf16_t stage[ST_ELEMS];
  const int tid = threadIdx.x;
  const int k = blockIdx.x >> 1, half = blockIdx.x & 1;
  int id = p.ids[k], valid = ST_TOK;
  if (id < 0 || (int64_t)id >= p.num_blocks) {
    id = 0;
    valid = 0;
  }
  id = __builtin_amdgcn_readfirstlane(id);
  valid = __builtin_amdgcn_readfirstlane(valid);
  const QuantPlanes pl{(int)p.off_lc, (int)p.off_ls, (int)p.off_rc, (int)p.off_rs};
  const auto offs = QS::offsets(pl, 512 / p.g_lat, 64 / p.g_rope, tid);
  const uint32_t lds = (uint32_t)__builtin_amdgcn_readfirstlane(lds_addr(cst) + (tid & ~63) * 16);
  const uint8_t* blk = p.pool + (size_t)id * (size_t)p.block_bytes;
#pragma unroll
  for (int i = 0; i < QS::LOADS; ++i) QS::issue_one(i, offs, blk, half, lds);
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
  __syncthreads();
  QS::dequant(cst, valid, 31 - __builtin_clz(p.g_lat), 31 - __builtin_clz(p.g_rope), stage, tid);
  lds_barrier();
  uint16_t* out = p.out + ((size_t)k * BLOCK_TOKENS + half * ST_TOK) * 576;
  for (int q = tid; q < ST_TOK * 72; q += NT) {
    const int t = q / 72, c8 = q % 72;
    *(u32x4*)(out + t * 576 + c8 * 8) = *(const u32x4*)&stage[rst_off(t, c8 * 8)];
  }
}

template <int FMT, bool MIXED = false>
static hipError_t launch_fmt(const RowsParams& p, hipStream_t st) {
  const int grid = 8 * p.units_per_xcd;
  if (p.q_f32)
    hipLaunchKernelGGL((decode_rows_kernel<FMT, true, MIXED>), dim3(grid), dim3(NT), 0, st, p);
  else
    hipLaunchKernelGGL((decode_rows_kernel<FMT, false, MIXED>), dim3(grid), dim3(NT), 0, st, p);
  return hipGetLastError();
}

}  // namespace rows

hipError_t launch_dequant_rows(const DequantParams& p, int fmt, hipStream_t st) {
  if (fmt == FMT_INT4)
    hipLaunchKernelGGL(rows::dequant_stage_rows_kernel<FMT_INT4>, dim3(2 * p.n), dim3(rows::NT), 0, st, p);
  else if (fmt == FMT_INT2)
    hipLaunchKernelGGL(rows::dequant_stage_rows_kernel<FMT_INT2>, dim3(2 * p.n), dim3(rows::NT), 0, st, p);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_decode_rows(const RowsParams& p, int fmt, hipStream_t st) {
  switch (fmt) {
    case FMT_BF16: return rows::launch_fmt<FMT_BF16>(p, st);
    case FMT_INT4: return rows::launch_fmt<FMT_INT4>(p, st);
    case FMT_INT2: return rows::launch_fmt<FMT_INT2>(p, st);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_decode_rows_mixed(const RowsParams& p, int fmt, hipStream_t st) {
  switch (fmt) {
    case FMT_INT4: return rows::launch_fmt<FMT_INT4, true>(p, st);
    case FMT_INT2: return rows::launch_fmt<FMT_INT2, true>(p, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace mla
