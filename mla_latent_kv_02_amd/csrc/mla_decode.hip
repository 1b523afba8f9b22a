// MLA decode over a paged latent cache: the absorbed-MQA attention step (gfx950).
//
// Every head scores the same cached rows [c (512) | k_rope (64)] (GQLA
// abstract: absorbed MQA decoding path), the softmax-weighted sum is taken
// over the latent itself (RAQ-MLA abstract: the latent supplies the values),
// and INT4/INT2 caches are unpacked and dequantised inside this loop
// (QuantMLA English abstract: native low-bit attention kernel).
//
// Work unit = (sequence b, context partition c, row group rg).  A row is one
// (query token i, head h) pair; a workgroup (8 wavefronts) owns 16*RT rows and
// walks its partition in stages of 32 tokens (half a paged block):
//   * stage data streams HBM -> LDS with global_load_lds_dwordx4 through a
//     4-deep ring, so three stages are in flight while one is consumed; no
//     VGPRs are spent on staging.  Quantised caches stream their codes into a
//     code ring and every thread dequantises one piece into a bf16 stage.
//   * the bf16 stage layout is [32 tokens][72 pieces of 16 B], each piece index
//     XOR-swizzled by the token so that both the score operand reads and the
//     transposed reads of the P.C product are free of LDS bank conflicts;
//   * scores S^T = K . Q^T on v_mfma_f32_16x16x32_bf16 (K from LDS, Q^T held in
//     registers for the whole partition), 2*RT waves each own one 16-row x
//     16-token tile; per-row maxima are exchanged through LDS; P = exp2(x - m)
//     is written to LDS as two bf16 terms (hi + lo, ~16 significant bits);
//   * O += P . C on the same MFMA, once per P term: wave w owns latent columns
//     [64w, 64w + 64) of all rows; the C operand comes from the token-major
//     stage with ds_read_b64_tr_b16 and feeds both MFMAs.
// Partials (o, lse) of the partitions are merged by combine_kernel.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "mla_device.hpp"
#include "mla_internal.hpp"
#include "mla_stage.hpp"

namespace mla {

constexpr int NT = 512;                // threads per workgroup (8 waves)
constexpr int PROW = ST_TOK + 8;       // bf16 elements per LDS P row
constexpr int MAX_TPC = 256;           // paged blocks per partition (host planner caps it)

// 16-byte LDS store written as inline asm.  The compiler's wait insertion cannot tell
// which ring slot an LDS store touches once the ring loop's back edge merges its state,
// and would otherwise wait for every DMA in flight (vmcnt(0)) before the store.  The store
// only writes the bf16 stage, which no DMA targets; the next lds_barrier() waits for it.
__device__ __forceinline__ void lds_store16(bf16_t* dst, const u32x4& v) {
  const uint32_t a = (uint32_t)(uintptr_t)(lds_void*)dst;
  asm volatile("ds_write_b128 %0, %1" ::"v"(a), "v"(v) : "memory");
}

__device__ __forceinline__ void dma16(const void* src, lds_void* dst) {
  __builtin_amdgcn_global_load_lds(src, dst, 16, 0, 0);
}

// 16 bytes per lane from a per-lane address to LDS bytes [lds_base + 16 lane, + 16), invisible
// to the compiler's wait insertion (every wait for it is explicit).
__device__ __forceinline__ void dma16a(const void* src, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(
                   __builtin_amdgcn_readfirstlane(lds_base)),
               "v"(src)
               : "memory", "m0");
}

// A wave-uniform pointer held as such (scalar registers), for values that are uniform by
// construction but chosen in ways the compiler cannot follow.
__device__ __forceinline__ const uint8_t* uniform_ptr(const uint8_t* ptr) {
  const uint64_t v = (uint64_t)(uintptr_t)ptr;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return (const uint8_t*)(uintptr_t)(((uint64_t)hi << 32) | lo);
}

__device__ __forceinline__ int64_t uniform_i64(int64_t v) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)(uint64_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)v >> 32));
  return (int64_t)(((uint64_t)hi << 32) | lo);
}

// The fields of a part of a mixed history as values: a choice between parts then selects
// values (a choice between two fields of a kernel argument can become a load from a chosen
// address, which moves the whole argument to scratch memory).
struct MixedLocal {
  const uint8_t* pool;
  int64_t num_blocks, block_bytes;
  const int32_t* block_table;
  int bt_stride;
};
__device__ __forceinline__ MixedLocal mixed_local(const MixedPart& h) {
  return MixedLocal{uniform_ptr(h.pool), uniform_i64(h.num_blocks), uniform_i64(h.block_bytes),
                    (const int32_t*)uniform_ptr((const uint8_t*)h.block_table),
                    (int)__builtin_amdgcn_readfirstlane((uint32_t)h.bt_stride)};
}

// v1, or v0 for part 0 and v2 for part 2, as v1 plus differences: every choice has a constant
// arm (a choice between two loaded variables becomes a load from a chosen address, which keeps
// the variables, and the kernel argument they come from, in scratch memory)
__device__ __forceinline__ int64_t by_part(int part, int64_t v0, int64_t v1, int64_t v2) {
  return v1 + (part == 0 ? v0 - v1 : 0) + (part == 2 ? v2 - v1 : 0);
}

// Mixed histories in joint positions: the part of joint block jb (0 sink, 1 middle, 2 recent
// window) given the sink's and the middle's block counts, and the first block of a part.
__device__ __forceinline__ int mixed_part(int jb, int nS, int nM) { return jb < nS ? 0 : (jb < nS + nM ? 1 : 2); }
__device__ __forceinline__ int mixed_start(int part, int nS, int nM) { return part == 0 ? 0 : (part == 1 ? nS : nS + nM); }

// The same from a wave-uniform base plus a per-lane 32-bit offset (the offset in a VGPR, the
// base in SGPRs): no per-lane 64-bit address arithmetic.
__device__ __forceinline__ void dma16s(const uint8_t* base, uint32_t off, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(
                   __builtin_amdgcn_readfirstlane(lds_base)),
               "v"(off), "s"(base)
               : "memory", "m0");
}

// Reductions over the four lane groups (lanes l, l ^ 16, l ^ 32, l ^ 48) with the gfx950 lane
// swaps: with both operands equal, permlane32_swap / permlane16_swap return x at l and at l ^ 32
// (l ^ 16), so one max / add per step gives the butterfly without an LDS round trip.
__device__ __forceinline__ float wave_max_16_32(float x) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float wave_sum_16_32(float x) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

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
// Stage producers.  Every loader thread issues a fixed number of DMA instructions per stage
// (LOADS), whatever the stage holds, so a wave's outstanding-load count is known exactly.
// ----------------------------------------------------------------------------------------
template <int FMT>
struct Producer;

// bf16 rows: the 2304 pieces of a half block; waves 0-3 issue 5 instructions, waves 4-7 issue 4.
// Slot k receives (token k / 72, logical piece (k mod 72) ^ sw(token)); all 32 rows are copied
// (a block is allocated whole) and rows past the sequence end are zeroed before use.
template <>
struct Producer<FMT_BF16> {
  static constexpr int LOADS_LO = 5;  // waves 0..3
  static constexpr int LOADS_HI = 4;  // waves 4..7
  struct Offsets {
    uint32_t o[LOADS_LO];
  };
  __device__ static Offsets offsets(int tid) {
    Offsets r;
#pragma unroll
    for (int i = 0; i < LOADS_LO; ++i) {
      const int slot = min(i * NT + tid, ST_TOK * 72 - 1);
      const int t = slot / 72;
      r.o[i] = (uint32_t)(t * 1152 + (((slot - t * 72) ^ sw(t)) << 4));
    }
    return r;
  }
  __device__ __forceinline__ static void issue(const uint8_t* half, const Offsets& off, bf16_t* stage, int tid) {
    const int wbase = tid & ~63;
#pragma unroll
    for (int i = 0; i < LOADS_LO; ++i) {
      if (i == LOADS_HI && tid >= 256) break;
      dma16(half + off.o[i], (lds_void*)(stage + (size_t)(i * NT + wbase) * 8));
    }
  }
};

// Quantised latent (INT4 or INT2) + INT4 rope: the four code planes of a half block are
// copied into a flat, token-major code stage [lc | ls | rc | rs], padded to SLOTS pieces.
// A half block holds 256 (INT4) or 128 (INT2) latent code slots, 4096 / latent_group scale
// slots, 64 RoPE code slots and 512 / rope_group RoPE scale slots: at most 720 (INT4) and
// 464 (INT2).  INT4: waves 0 .. WLO-1 issue two DMA instructions per stage, the others one
// (WLO = 4: 768 slots, every layout; WLO = 3: 704 slots, latent groups of 64 or more).
template <int FMT, int WLO = 4>
struct QuantProducer {
  static constexpr int BITS = FMT == FMT_INT4 ? 4 : 2;
  static constexpr int LB = 512 * BITS / 8;        // latent code bytes per token
  static constexpr int LOADS_LO = FMT == FMT_INT4 ? 2 : 1;   // instructions of waves 0 .. WAVES_LO-1
  static constexpr int LOADS_HI = 1;                          // of the other waves
  static constexpr int WAVES_LO = FMT == FMT_INT4 ? WLO : 8;
  static constexpr int SLOTS = 64 * (WAVES_LO * LOADS_LO + (8 - WAVES_LO) * LOADS_HI);
  // code stage slots a layout needs (groups = 512 / latent_group, rgroups = 64 / rope_group)
  __host__ __device__ static constexpr int slots_needed(int groups, int rgroups) {
    return ST_TOK * LB / 16 + ST_TOK * groups * 4 / 16 + ST_TOK * 32 / 16 + (ST_TOK * rgroups * 4 + 15) / 16;
  }
  __device__ __forceinline__ static void issue(const uint8_t* blk, int half, const QuantPlanes& pl, int groups,
                                               int rgroups, uint8_t* cstage, int tid) {
    issue_with(half, pl, groups, rgroups, tid, [&](int off, int i, int wbase) {
      dma16(blk + off, (lds_void*)(cstage + (size_t)(i * NT + wbase) * 16));
    });
  }
  // byte offsets inside the block (first half, second half) of the piece that code-stage slot
  // `slot` receives; padding slots re-load a real piece (spread over the stage, never one
  // shared address)
  __device__ __forceinline__ static uint2 piece_offsets(const QuantPlanes& pl, int groups, int rgroups, int slot) {
    const int n_lc = ST_TOK * LB / 16;
    const int n_ls = ST_TOK * groups * 4 / 16;
    const int n_rc = ST_TOK * 32 / 16;
    const int n_rs = (ST_TOK * rgroups * 4 + 15) / 16;
    const int n_all = n_lc + n_ls + n_rc + n_rs;
    int p = slot < n_all ? slot : slot - n_all;
    int base, hstride;
    if (p < n_lc) {
      base = pl.lc + p * 16;
      hstride = ST_TOK * LB;
    } else if ((p -= n_lc) < n_ls) {
      base = pl.ls + p * 16;
      hstride = ST_TOK * groups * 4;
    } else if ((p -= n_ls) < n_rc) {
      base = pl.rc + p * 16;
      hstride = ST_TOK * 32;
    } else {
      base = pl.rs + (p - n_rc) * 16;
      hstride = ST_TOK * rgroups * 4;
    }
    return uint2{(uint32_t)base, (uint32_t)(base + hstride)};
  }
  // byte offset inside the block of the piece that slot i * NT + tid of a code stage receives:
  // dma(offset, i, first thread of the wave) for each of this thread's DMA instructions
  template <class F>
  __device__ __forceinline__ static void issue_with(int half, const QuantPlanes& pl, int groups, int rgroups, int tid,
                                                    F&& dma) {
    const int n_lc = ST_TOK * LB / 16;
    const int n_ls = ST_TOK * groups * 4 / 16;
    const int n_rc = ST_TOK * 32 / 16;
    const int n_rs = (ST_TOK * rgroups * 4 + 15) / 16;
    const int n_all = n_lc + n_ls + n_rc + n_rs;
    const int wbase = tid & ~63;
#pragma unroll
    for (int i = 0; i < LOADS_LO; ++i) {
      if (i == LOADS_HI && tid >= 64 * WAVES_LO) break;
      const int slot = i * NT + tid;
      // padding slots re-load a real piece (spread over the stage, never one shared address)
      int p = slot < n_all ? slot : slot - n_all;
      int off;
      if (p < n_lc) {
        off = pl.lc + half * ST_TOK * LB + p * 16;
      } else if ((p -= n_lc) < n_ls) {
        off = pl.ls + half * ST_TOK * groups * 4 + p * 16;
      } else if ((p -= n_ls) < n_rc) {
        off = pl.rc + half * ST_TOK * 32 + p * 16;
      } else {
        off = pl.rs + half * ST_TOK * rgroups * 4 + (p - n_rc) * 16;
      }
      dma(off, i, wbase);
    }
  }

  // Latent task k (k < 512) or RoPE task k - 512 of a code stage into the swizzled bf16 stage;
  // tokens >= valid become zeros (scale and zero-point 0).  gl, gr: log2 of the latent and
  // rope group sizes (powers of two: they divide 512 and 64).
  __device__ __forceinline__ static void dequant_task(const uint8_t* cst, int valid, int k, int gl, int gr,
                                                      bf16_t* stage) {
    const int groups_log2 = 9 - gl;
    const int ls = ST_TOK * LB;
    if (k < 512) {
      int t, kk;
      lat_task(k, t, kk);
      uint32_t sz = *(const uint32_t*)(cst + ls + (((t << groups_log2) + ((kk * 32) >> gl)) << 2));
      sz = t < valid ? sz : 0u;
      float sc, zs;
      scale_zero(sz, sc, zs);
      // element 32 kk + 8 j sits at physical piece (4 kk + j) ^ sw(t) = (base piece) ^ j
      const int row = t * 576, p0 = (4 * kk) ^ sw(t);
      const uint8_t* code = cst + t * LB + kk * 4 * BITS;
      if constexpr (BITS == 4) {
        const u32x4 c = *(const u32x4*)code;
#pragma unroll
        for (int j = 0; j < 4; ++j) lds_store16(&stage[row + ((p0 ^ j) << 3)], dequant_int4x8(c[j], sc, zs));
      } else {
        const uint2 c = *(const uint2*)code;
        uint32_t t_lo, t_hi;
        int2_table(sc, zs, t_lo, t_hi);
        u32x4 lo, hi;
        dequant_int2x16(c.x, t_lo, t_hi, lo, hi);
        lds_store16(&stage[row + ((p0 ^ 0) << 3)], lo);
        lds_store16(&stage[row + ((p0 ^ 1) << 3)], hi);
        dequant_int2x16(c.y, t_lo, t_hi, lo, hi);
        lds_store16(&stage[row + ((p0 ^ 2) << 3)], lo);
        lds_store16(&stage[row + ((p0 ^ 3) << 3)], hi);
      }
    } else {
      int t, ri;
      rope_task(k - 512, t, ri);
      const int rbase = ls + (ST_TOK << (groups_log2 + 2));
      uint32_t rsz = *(const uint32_t*)(cst + rbase + ST_TOK * 32 + (((t << (6 - gr)) + ((ri * 8) >> gr)) << 2));
      rsz = t < valid ? rsz : 0u;
      float sc, zs;
      scale_zero(rsz, sc, zs);
      const uint32_t rc = *(const uint32_t*)(cst + rbase + t * 32 + ri * 4);
      lds_store16(&stage[st_off(t, 512 + ri * 8)], dequant_int4x8(rc, sc, zs));
    }
  }
  // every thread's share of a whole stage: latent task tid, RoPE task tid (tid < 256)
  __device__ __forceinline__ static void dequant(const uint8_t* cst, int valid, int gl, int gr, bf16_t* stage,
                                                 int tid) {
    dequant_task(cst, valid, tid, gl, gr, stage);
    if (tid < 256) dequant_task(cst, valid, 512 + tid, gl, gr, stage);
  }
};

template <>
struct Producer<FMT_INT4> : QuantProducer<FMT_INT4> {};
template <>
struct Producer<FMT_INT2> : QuantProducer<FMT_INT2> {};

// ----------------------------------------------------------------------------------------
// The decode kernel
// ----------------------------------------------------------------------------------------
template <int RT, int FMT, bool QF32>
__global__ __launch_bounds__(NT) void decode_mfma_kernel(DecodeParams p) {
  constexpr int ROWS = 16 * RT;
  constexpr bool QUANT = FMT != FMT_BF16;
  using Prod = Producer<FMT>;
  using QP = QuantProducer<FMT == FMT_BF16 ? FMT_INT4 : FMT>;
  constexpr int CBYTES = QUANT ? QP::SLOTS * 16 : 16;

  // bf16 path: a 4-deep ring of bf16 stages.  Quantised path with fewer than 64 rows: the
  // wavefronts that do not score dequantise stage s + 1 into the second of two bf16 stages
  // while stage s is scored, over a 6-deep ring of code stages.  Quantised, 64 rows (every
  // wavefront scores): an 8-deep code ring and one bf16 stage dequantised at each step.
  // Distinct arrays let the compiler see that reading one ring slot does not depend on the
  // DMA into another.
  constexpr bool SPLIT = QUANT && RT < 4;
  constexpr int DEPTH = QUANT ? (SPLIT ? 6 : 8) : 4;
  __shared__ __attribute__((aligned(16))) bf16_t S0[ST_ELEMS];
  __shared__ __attribute__((aligned(16))) bf16_t S1[(QUANT && !SPLIT) ? 8 : ST_ELEMS];
  __shared__ __attribute__((aligned(16))) bf16_t S2[QUANT ? 8 : ST_ELEMS];
  __shared__ __attribute__((aligned(16))) bf16_t S3[QUANT ? 8 : ST_ELEMS];
  __shared__ __attribute__((aligned(16))) uint8_t C0[CBYTES];
  __shared__ __attribute__((aligned(16))) uint8_t C1[CBYTES];
  __shared__ __attribute__((aligned(16))) uint8_t C2[CBYTES];
  __shared__ __attribute__((aligned(16))) uint8_t C3[CBYTES];
  __shared__ __attribute__((aligned(16))) uint8_t C4[CBYTES];
  __shared__ __attribute__((aligned(16))) uint8_t C5[CBYTES];
  __shared__ __attribute__((aligned(16))) uint8_t C6[SPLIT ? 16 : CBYTES];
  __shared__ __attribute__((aligned(16))) uint8_t C7[SPLIT ? 16 : CBYTES];
  __shared__ __attribute__((aligned(16))) bf16_t Ps[ROWS * PROW];   // P, high bf16 term
  __shared__ __attribute__((aligned(16))) bf16_t Pl[ROWS * PROW];   // P, low bf16 term
  __shared__ float red[2][ROWS];
  __shared__ float redx[2][ROWS];   // row sums of P (normalisation and lse)
  __shared__ float mfin[ROWS];
  __shared__ __attribute__((aligned(16))) float alpha[ROWS];
  __shared__ int bids[MAX_TPC];

  const int tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63, lr = lane & 15, lg = lane >> 4;

  // unit of work; consecutive units sit on one XCD (workgroups are dealt round-robin to 8 XCDs)
  const int u = (int)(blockIdx.x & 7) * p.units_per_xcd + (int)(blockIdx.x >> 3);
  if (u >= p.total_units) return;
  const int rg = u % p.RG;
  const int bc = u / p.RG;
  const int b = bc / p.max_chunks, c = bc % p.max_chunks;
  int L = p.seq_lens[b];
  L = L < 0 ? 0 : (L > p.max_seq_len ? p.max_seq_len : L);
  const int nblk = (L + BLOCK_TOKENS - 1) / BLOCK_TOKENS;
  int nch = (nblk + p.tpc - 1) / p.tpc;
  nch = nch < 1 ? 1 : nch;
  if (c >= nch) return;
  const int T0 = c * p.tpc * BLOCK_TOKENS;                      // first token of the partition
  const int T1 = min((c + 1) * p.tpc * BLOCK_TOKENS, L);        // one past its last token
  const int nst = T1 > T0 ? (T1 - T0 + ST_TOK - 1) / ST_TOK : 0;
  const int R = p.R;
  const int r0 = rg * ROWS;

  // score role: waves 0 .. 2*RT-1 own (row tile w/2, token tile w%2) of every stage
  const bool scorer = w < 2 * RT;
  const int sc_rt = (w >> 1) & (RT - 1), sc_tt = w & 1;
  const int row_s = sc_rt * 16 + lr;
  const int qrow = r0 + row_s;
  const bool qvalid = scorer && qrow < R;
  const int lim_s = qvalid ? L - p.s_q + qrow / p.H : -1;

  bf16x8 qreg[18];
  {
    const size_t qbase = (size_t)b * R + (qvalid ? qrow : 0);
#pragma unroll
    for (int ks = 0; ks < 16; ++ks)
      qreg[ks] = qvalid ? load_q8(p.q_lat, qbase * 512 + ks * 32 + lg * 8, QF32) : bf16x8{};
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
      qreg[16 + ks] = qvalid ? load_q8(p.q_rope, qbase * 64 + ks * 32 + lg * 8, QF32) : bf16x8{};
  }

  const float NEG_INF = -__builtin_inff();
  float m_s = NEG_INF, l_x = 0.f;
  f32x4 acc[RT][4];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) acc[rt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  const QuantPlanes pl{(int)p.off_lc, (int)p.off_ls, (int)p.off_rc, (int)p.off_rs};
  const int groups = 512 / p.g_lat, rgroups = 64 / p.g_rope;
  const int32_t* btab = p.block_table + (size_t)b * p.bt_stride;

  // where stage s comes from: block pointer, half, valid tokens
  // The partition's block ids are staged in LDS once: a global load inside the loop would
  // make the compiler wait for vmcnt(0), i.e. for every stage in flight.
  const int blk0 = T0 / BLOCK_TOKENS;
  const int nb_unit = min(p.tpc, nblk - blk0);
  for (int j = tid; j < nb_unit; j += NT) bids[j] = btab[blk0 + j];
  __syncthreads();
  auto stage_src = [&](int s, int& half, int& valid) -> const uint8_t* {
    const int tok = T0 + s * ST_TOK;
    half = (tok / ST_TOK) & 1;
    valid = min(ST_TOK, T1 - tok);
    int id = __builtin_amdgcn_readfirstlane(bids[tok / BLOCK_TOKENS - blk0]);
    if (id < 0 || (int64_t)id >= p.num_blocks) {
      id = 0;
      valid = 0;
    }
    return p.pool + (size_t)id * (size_t)p.block_bytes;
  };
  const auto bf_off = Producer<FMT_BF16>::offsets(tid);
  auto issue = [&](int s, bf16_t* st, uint8_t* cst) {
    int half, valid;
    const uint8_t* blk = stage_src(s, half, valid);
    if constexpr (QUANT)
      Prod::issue(blk, half, pl, groups, rgroups, cst, tid);
    else
      Prod::issue(blk + half * ST_TOK * 1152, bf_off, st, tid);
  };
  // wait until a stage has landed, given how many later stages were issued after it
  // (each loader wave issues a fixed number of DMA instructions per stage)
  auto wait_stage = [&](int later) {
    constexpr int LA = QUANT ? QP::LOADS_LO : Producer<FMT_BF16>::LOADS_LO;
    constexpr int LB = QUANT ? QP::LOADS_HI : Producer<FMT_BF16>::LOADS_HI;
    constexpr int WA = QUANT ? QP::WAVES_LO : 4;   // waves issuing LA instructions per stage
    const int n = w < WA ? LA : LB;
    auto wait_n = [&](auto K) {
      if (n == LA) __builtin_amdgcn_s_waitcnt(vmcnt_imm(decltype(K)::value * LA));
      else __builtin_amdgcn_s_waitcnt(vmcnt_imm(decltype(K)::value * LB));
    };
    switch (later) {
      case 0: wait_n(std::integral_constant<int, 0>{}); break;
      case 1: wait_n(std::integral_constant<int, 1>{}); break;
      case 2: wait_n(std::integral_constant<int, 2>{}); break;
      case 3: wait_n(std::integral_constant<int, 3>{}); break;
      case 4: wait_n(std::integral_constant<int, 4>{}); break;
      case 5: wait_n(std::integral_constant<int, 5>{}); break;
      default: wait_n(std::integral_constant<int, 6>{}); break;
    }
  };
  static_assert(DEPTH - 2 <= 6, "wait_stage covers at most 6 later stages");
  const int gl_log2 = 31 - __builtin_clz(p.g_lat > 0 ? p.g_lat : 1);
  const int gr_log2 = 31 - __builtin_clz(p.g_rope > 0 ? p.g_rope : 1);

  // prologue: stages 0 .. DEPTH-2 in flight; stage 0 landed (split: stages 0 and 1 landed and
  // stage 0 dequantised by every wavefront)
  if constexpr (QUANT) {
    if (0 < nst) issue(0, S0, C0);
    if (1 < nst) issue(1, S0, C1);
    if (2 < nst) issue(2, S0, C2);
    if (3 < nst) issue(3, S0, C3);
    if (4 < nst) issue(4, S0, C4);
    if (!SPLIT && 5 < nst) issue(5, S0, C5);
    if (!SPLIT && 6 < nst) issue(6, S0, C6);
  } else {
    if (0 < nst) issue(0, S0, C0);
    if (1 < nst) issue(1, S1, C0);
    if (2 < nst) issue(2, S2, C0);
  }
  if constexpr (SPLIT) {
    wait_stage(min(nst - 1, DEPTH - 2) - min(nst - 1, 1));
    lds_barrier();
    if (0 < nst) {
      int half_unused, valid0;
      stage_src(0, half_unused, valid0);
      QP::dequant(C0, valid0, gl_log2, gr_log2, S0, tid);
    }
    lds_barrier();
  } else {
    wait_stage(min(nst - 1, DEPTH - 2));
    lds_barrier();
  }
  // ---- the phases of one step
  f32x4 sv = {0.f, 0.f, 0.f, 0.f};   // this scorer's scores of the current stage
  auto score_phase = [&](int s, const bf16_t* KS, int valid) {
    sv = f32x4{0.f, 0.f, 0.f, 0.f};
    // ---- scores for (row tile sc_rt, token tile sc_tt)
    if (scorer) {
      // k-step ks reads logical piece 4 ks + lg, physical 8 (ks / 2) + ((4 (ks & 1) + lg) ^ f):
      // one base register for even and one for odd ks, the rest is an immediate offset of 32
      // elements per ks (k-steps 16 and 17 are the RoPE columns).
      const int t = sc_tt * 16 + lr;
      const int f = sw(t);
      const bf16_t* kev = &KS[t * 576 + (lg ^ f) * 8];
      const bf16_t* kod = &KS[t * 576 + ((4 + lg) ^ f) * 8 - 32];
      const bf16_t* k16 = kev + 16 * 32;
      const bf16_t* k17 = kod + 17 * 32;
      f32x4 a0 = {0.f, 0.f, 0.f, 0.f}, a1 = a0, a2 = a0, a3 = a0;
#pragma unroll
      for (int ks = 0; ks < 16; ks += 4) {
        a0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(*(const bf16x8*)(kev + ks * 32), qreg[ks], a0, 0, 0, 0);
        a1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(*(const bf16x8*)(kod + ks * 32 + 32), qreg[ks + 1], a1, 0, 0, 0);
        a2 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(*(const bf16x8*)(kev + ks * 32 + 64), qreg[ks + 2], a2, 0, 0, 0);
        a3 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(*(const bf16x8*)(kod + ks * 32 + 96), qreg[ks + 3], a3, 0, 0, 0);
      }
      a0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(*(const bf16x8*)k16, qreg[16], a0, 0, 0, 0);
      a1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(*(const bf16x8*)k17, qreg[17], a1, 0, 0, 0);
      sv = (a0 + a1) + (a2 + a3);
      float mx = NEG_INF;
      const int tok0 = T0 + s * ST_TOK + sc_tt * 16 + lg * 4;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        // tokens past the causal limit, and tokens of an out-of-range block (valid = 0), are skipped
        const bool ok = tok0 + i <= lim_s && sc_tt * 16 + lg * 4 + i < valid;
        const float x = ok ? sv[i] * p.scale_log2 : NEG_INF;
        sv[i] = x;
        mx = fmaxf(mx, x);
      }
      mx = wave_max_16_32(mx);
      if (lg == 0) red[sc_tt][row_s] = mx;
    }
  };
  auto softmax_phase = [&]() {
    // ---- running max, P for the scored tile; the scorers of token tile 0 publish the
    // rescale factor of their rows, every wave then rescales the output rows it owns
    if (scorer) {
      // The reference maximum m only moves when the stage maximum exceeds it by more than
      // RESCALE_SLACK (log2 units), so P = exp2(x - m) stays below 2^RESCALE_SLACK and the
      // accumulators are rescaled only on such a move, rare after a partition's first stages.
      // The final division by the row sum cancels the choice of m.
      const float mt = fmaxf(red[0][row_s], red[1][row_s]);
      const float mn = mt > m_s + RESCALE_SLACK ? mt : m_s;
      const float mu = mn == NEG_INF ? 0.f : mn;
      const float al = mn == m_s ? 1.f : __builtin_amdgcn_exp2f(m_s - mu);
      l_x *= al;
      m_s = mn;
      if (sc_tt == 0 && lg == 0) alpha[row_s] = al;
      float pf[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        pf[i] = __builtin_amdgcn_exp2f(sv[i] - mu);
        l_x += pf[i];
      }
      uint32_t h0, l0, h1, l1;
      split_pair(pf[0], pf[1], h0, l0);
      split_pair(pf[2], pf[3], h1, l1);
      *(uint2*)&Ps[row_s * PROW + sc_tt * 16 + lg * 4] = uint2{h0, h1};
      *(uint2*)&Pl[row_s * PROW + sc_tt * 16 + lg * 4] = uint2{l0, l1};
    }
  };
  auto pv_phase = [&](const bf16_t* KS) {
    {
      bool any = false;
      f32x4 al[RT];
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        al[rt] = *(const f32x4*)&alpha[rt * 16 + lg * 4];
        any |= (al[rt][0] != 1.f) | (al[rt][1] != 1.f) | (al[rt][2] != 1.f) | (al[rt][3] != 1.f);
      }
      if (__any(any)) {
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
          for (int nt = 0; nt < 4; ++nt) acc[rt][nt] *= al[rt];
      }
    }

    // ---- O[rows][64w .. 64w+63] += (P_hi + P_lo) . C over the 32 tokens of the stage
    {
      bf16x8 a[RT], al_[RT];
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        a[rt] = *(const bf16x8*)&Ps[(rt * 16 + lr) * PROW + lg * 8];
        al_[rt] = *(const bf16x8*)&Pl[(rt * 16 + lr) * PROW + lg * 8];
      }
      const int t0 = lg * 8 + (lr >> 2);
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        const int d = w * 64 + nt * 16 + (lr & 3) * 4;
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)&KS[st_off(t0, d)]);
        const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)&KS[st_off(t0 + 4, d)]);
        const bf16x8 bv = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
          acc[rt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[rt], bv, acc[rt][nt], 0, 0, 0);
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
          acc[rt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al_[rt], bv, acc[rt][nt], 0, 0, 0);
      }
    }
  };

  // one stage: KS = bf16 stage read by the MFMAs, CCUR = its code stage (quantised formats,
  // not split), NXT/CNXT = ring slot refilled with stage s + DEPTH - 1
  auto step = [&](int s, bf16_t* KS, uint8_t* CCUR, bf16_t* NXT, uint8_t* CNXT) {
    // stage s has landed and every wave is done with stage s-1 (barrier at the end of the
    // previous step), so the ring slot of stage s-1 can take stage s + DEPTH - 1
    if (s + DEPTH - 1 < nst) issue(s + DEPTH - 1, NXT, CNXT);
    int half_unused, valid;
    stage_src(s, half_unused, valid);
    if constexpr (QUANT) {
      QP::dequant(CCUR, valid, gl_log2, gr_log2, KS, tid);
      lds_barrier();
    } else if (valid < ST_TOK) {
      // rows past the sequence end were filled from a dummy address: zero them
      for (int q = tid; q < (ST_TOK - valid) * 72; q += NT)
        *(u32x4*)&KS[(valid + q / 72) * 576 + (q % 72) * 8] = u32x4{0, 0, 0, 0};
      lds_barrier();
    }
    score_phase(s, KS, valid);
    lds_barrier();
    softmax_phase();
    lds_barrier();
    pv_phase(KS);
    // stage s+1 landed, and nobody reads stage s any more
    wait_stage(min(nst - 2 - s, DEPTH - 2));
    lds_barrier();
  };

  // split quantised step: KS = bf16 stage of s, KN = bf16 stage of s + 1, CDQ = code stage of
  // s + 1, CNXT = ring slot refilled with stage s + DEPTH - 1 (the slot of s - 1, dequantised in
  // step s - 2).  The wavefronts that do not score dequantise stage s + 1 meanwhile: tasks
  // q, q + G, ... (G = their thread count), the first half during the scores, the rest during
  // the softmax.
  constexpr int G = SPLIT ? NT - 128 * RT : 1;
  constexpr int N_IT = (768 + G - 1) / G;
  constexpr int IT_A = (N_IT + 1) / 2;
  auto step_split = [&](int s, bf16_t* KS, bf16_t* KN, uint8_t* CDQ, uint8_t* CNXT) {
    if (s + DEPTH - 1 < nst) issue(s + DEPTH - 1, KN, CNXT);
    int half_unused, valid, valid_n = 0;
    stage_src(s, half_unused, valid);
    const bool deq = !scorer && s + 1 < nst;
    if (s + 1 < nst) stage_src(s + 1, half_unused, valid_n);
    const int q = tid - 128 * RT;
    if (scorer) {
      score_phase(s, KS, valid);
    } else if (deq) {
#pragma unroll
      for (int it = 0; it < IT_A; ++it)
        if (it * G + q < 768) QP::dequant_task(CDQ, valid_n, it * G + q, gl_log2, gr_log2, KN);
    }
    lds_barrier();
    if (scorer) {
      softmax_phase();
    } else if (deq) {
#pragma unroll
      for (int it = IT_A; it < N_IT; ++it)
        if (it * G + q < 768) QP::dequant_task(CDQ, valid_n, it * G + q, gl_log2, gr_log2, KN);
    }
    lds_barrier();
    pv_phase(KS);
    // stage s + 2 landed (dequantised in the next step), and nobody reads stage s any more
    if (s + 2 < nst) wait_stage(min(nst - 1, s + DEPTH - 1) - (s + 2));
    lds_barrier();
  };

  if constexpr (!QUANT) {
    for (int s = 0; s < nst; s += 4) {
      step(s, S0, C0, S3, C3);
      if (s + 1 < nst) step(s + 1, S1, C1, S0, C0);
      if (s + 2 < nst) step(s + 2, S2, C2, S1, C1);
      if (s + 3 < nst) step(s + 3, S3, C3, S2, C2);
    }
  } else if constexpr (SPLIT) {
    for (int s = 0; s < nst; s += 6) {
      step_split(s, S0, S1, C1, C5);
      if (s + 1 < nst) step_split(s + 1, S1, S0, C2, C0);
      if (s + 2 < nst) step_split(s + 2, S0, S1, C3, C1);
      if (s + 3 < nst) step_split(s + 3, S1, S0, C4, C2);
      if (s + 4 < nst) step_split(s + 4, S0, S1, C5, C3);
      if (s + 5 < nst) step_split(s + 5, S1, S0, C0, C4);
    }
  } else {
    for (int s = 0; s < nst; s += 8) {
      step(s, S0, C0, S0, C7);
      if (s + 1 < nst) step(s + 1, S0, C1, S0, C0);
      if (s + 2 < nst) step(s + 2, S0, C2, S0, C1);
      if (s + 3 < nst) step(s + 3, S0, C3, S0, C2);
      if (s + 4 < nst) step(s + 4, S0, C4, S0, C3);
      if (s + 5 < nst) step(s + 5, S0, C5, S0, C4);
      if (s + 6 < nst) step(s + 6, S0, C6, S0, C5);
      if (s + 7 < nst) step(s + 7, S0, C7, S0, C6);
    }
  }

  // ---- finish: row sums over lanes and token tiles, normalise, write
  if (scorer) {
    l_x = wave_sum_16_32(l_x);
    if (lg == 0) {
      redx[sc_tt][row_s] = l_x;
      if (sc_tt == 0) mfin[row_s] = m_s;
    }
  }
  lds_barrier();
  const size_t unit_row0 = ((size_t)b * p.max_chunks + c) * R;
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = rt * 16 + lg * 4 + i;
      const int rgl = r0 + row;
      if (rgl >= R) continue;
      const float lt = redx[0][row] + redx[1][row];
      const float inv = lt > 0.f ? 1.f / lt : 0.f;
      const size_t obase = (unit_row0 + rgl) * 512 + w * 64 + lr;
      if (p.out_bf16) {
        bf16_t* o = (bf16_t*)p.out;
#pragma unroll
        for (int nt = 0; nt < 4; ++nt)
          o[obase + nt * 16] = __builtin_bit_cast(bf16_t, (uint16_t)f32_to_bf16_bits(acc[rt][nt][i] * inv));
      } else {
        float* o = (float*)p.out;
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) o[obase + nt * 16] = acc[rt][nt][i] * inv;
      }
    }
  }
  if (p.out_lse != nullptr && tid < ROWS && r0 + tid < R) {
    const float lt = redx[0][tid] + redx[1][tid];
    p.out_lse[unit_row0 + r0 + tid] = lt > 0.f ? (mfin[tid] + __log2f(lt)) * 0.69314718055994531f : NEG_INF;
  }
}

// ---------------------------------------------------------------------------------------
// Pipelined decode for quantised caches and at most 16 query rows (the V2-Lite shapes), one
// barrier per 32-token step.  In step s wavefront 0 scores stage s + 1 and runs its softmax in
// registers (a row's 32 scores sit in its 4 lane groups), every wavefront adds P(s) . C(s) to
// the 64 output columns it owns, and wavefronts 1-7 dequantise stage s + 2 into the third
// bf16 buffer, so the dequantisation (VALU), the scores (MFMA) and the HBM reads of later
// code stages overlap.  Code stage k sits in ring slot k mod 4, bf16 stage k in buffer k mod 3,
// P (two bf16 terms) and the rescale factors of stage k in buffer k mod 2.  The DMA is inline
// asm (each wait for it is explicit), so one LDS array holds every buffer.  The INT4 code
// stages take 704 slots (latent groups of 64 or more; the launcher sends group 32 elsewhere),
// which leaves the LDS room for both P terms.
// ---------------------------------------------------------------------------------------
template <int FMT>
using PipeQP = QuantProducer<FMT, 3>;

// Mixed histories: the bf16 rows of a half block (its first row at `half`) by DMA into a bf16
// stage, and the rows from `valid` on zeroed once landed.  Out of line: the pipelined kernel
// takes this path for a few blocks of a sequence, and inlined it perturbs the scheduling of
// the kernel's every step.
__device__ __attribute__((noinline)) void pipe_issue_bf16(const uint8_t* half, bf16_t* stage, int tid) {
  Producer<FMT_BF16>::issue(half, Producer<FMT_BF16>::offsets(tid), stage, tid);
}
__device__ __attribute__((noinline)) void pipe_zero_rows(bf16_t* stage, int valid, int tid, int nt) {
  for (int q = tid; q < (ST_TOK - valid) * 72; q += nt)
    *(u32x4*)&stage[(valid + q / 72) * 576 + (q % 72) * 8] = u32x4{0, 0, 0, 0};
}

// MIXED: the history of sequence b is a bf16 sink ++ the low-bit middle ++ a bf16 recent
// window (p.hi), each part in whole blocks, partitions cut over that joint list.  A bf16 block
// is copied by DMA into the bf16 buffer that the dequantising wavefronts would fill, and its
// code-ring slot receives a stand-in copy of its first bytes (unread), so every step keeps the
// ring's load count.
template <int FMT, bool QF32, bool MIXED>
__global__ __launch_bounds__(NT) void decode_pipe_kernel(DecodeParams p) {
  using QP = PipeQP<FMT>;
  constexpr int DEPTH = 4;                         // code ring slots
  constexpr int CBYTES = QP::SLOTS * 16;
  constexpr int BF = ST_ELEMS * 2;                 // bytes of a bf16 stage
  constexpr int OFF_C = 3 * BF;
  constexpr int OFF_P = OFF_C + DEPTH * CBYTES;
  constexpr int PBYTES = 16 * PROW * 2;            // one P term of one stage
  constexpr int SMEM = OFF_P + 4 * PBYTES;
  __shared__ __attribute__((aligned(16))) uint8_t smem[SMEM];
  __shared__ __attribute__((aligned(16))) float alpha[2][16];
  __shared__ float fin[2][16];                     // row sums of P, maximum
  // per block of the partition: its address (bits 0..55) and valid tokens (bits 56..63),
  // resolved once before the loop (the host keeps pools below 2^56)
  __shared__ uint2 btab2[MAX_TPC];

  const int tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63, lr = lane & 15, lg = lane >> 4;
  const float NEG_INF = -__builtin_inff();

  const int u = (int)(blockIdx.x & 7) * p.units_per_xcd + (int)(blockIdx.x >> 3);
  if (u >= p.total_units) return;
  const int bc = u / p.RG;                         // RG = 1: at most 16 rows
  const int b = bc / p.max_chunks, c = bc % p.max_chunks;
  auto clamp_len = [b](const int32_t* lens, int mx) {
    if (lens == nullptr) return 0;
    const int v = lens[b];
    return v < 0 ? 0 : (v > mx ? mx : v);
  };
  // L: the length in the causal mask (query i sees positions <= L - s_q + i), Lend: the end of
  // the last part's tokens.  Mixed histories in joint positions (each part padded to whole
  // blocks, the recent window from position 64 (nS + nM)), with every sink and middle token
  // visible when the window holds fewer than s_q tokens.
  const int Ls = MIXED ? clamp_len(p.hi[0].seq_lens, p.hi[0].max_seq_len) : 0;
  int Lm = p.seq_lens[b];
  Lm = Lm < 0 ? 0 : (Lm > p.max_seq_len ? p.max_seq_len : Lm);
  const int Lr = MIXED ? clamp_len(p.hi[1].seq_lens, p.hi[1].max_seq_len) : 0;
  const int nS = (Ls + BLOCK_TOKENS - 1) / BLOCK_TOKENS;
  const int nM = (Lm + BLOCK_TOKENS - 1) / BLOCK_TOKENS;
  const int nR = (Lr + BLOCK_TOKENS - 1) / BLOCK_TOKENS;
  const int nblk = nS + nM + nR;
  const int L = !MIXED ? Lm : (nblk > 0 ? BLOCK_TOKENS * (nS + nM) + max(Lr, p.s_q - 1) : 0);
  const int Lend = !MIXED ? Lm : (nR > 0 ? BLOCK_TOKENS * (nS + nM) + Lr : (nM > 0 ? BLOCK_TOKENS * nS + Lm : Ls));
  // this partition's joint blocks [jb0, jb1) (mixed histories: weighted positions)
  int nch, jb0, jb1;
  if constexpr (MIXED) {
    nch = (mixed_positions(nS, nM, nR) + p.tpc - 1) / p.tpc;
    jb0 = mixed_blocks_before(c * p.tpc, nS, nM, nR);
    jb1 = mixed_blocks_before((c + 1) * p.tpc, nS, nM, nR);
  } else {
    nch = (nblk + p.tpc - 1) / p.tpc;
    jb0 = c * p.tpc;
    jb1 = min(nblk, (c + 1) * p.tpc);
  }
  nch = nch < 1 ? 1 : nch;
  if (c >= nch) return;
  const int T0 = jb0 * BLOCK_TOKENS;
  const int T1 = min(jb1 * BLOCK_TOKENS, Lend);
  const int nst = T1 > T0 ? (T1 - T0 + ST_TOK - 1) / ST_TOK : 0;
  const int R = p.R;

  // wavefront 0: the queries of the 16 rows (row lr) and their softmax state
  const bool qrow = lr < R;
  const int lim = qrow ? L - p.s_q + lr / p.H : -1;
  bf16x8 qreg[18];
  if (w == 0) {
    const size_t qbase = (size_t)b * R + (qrow ? lr : 0);
#pragma unroll
    for (int ks = 0; ks < 16; ++ks)
      qreg[ks] = qrow ? load_q8(p.q_lat, qbase * 512 + ks * 32 + lg * 8, QF32) : bf16x8{};
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
      qreg[16 + ks] = qrow ? load_q8(p.q_rope, qbase * 64 + ks * 32 + lg * 8, QF32) : bf16x8{};
  }
  float m_s = NEG_INF, l_x = 0.f;
  // output columns: wave w owns column group w
  f32x4 acc[4];
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) acc[nt] = f32x4{0.f, 0.f, 0.f, 0.f};

  const QuantPlanes pl{(int)p.off_lc, (int)p.off_ls, (int)p.off_rc, (int)p.off_rs};
  const int groups = 512 / p.g_lat, rgroups = 64 / p.g_rope;
  const int gl_log2 = 31 - __builtin_clz(p.g_lat > 0 ? p.g_lat : 1);
  const int gr_log2 = 31 - __builtin_clz(p.g_rope > 0 ? p.g_rope : 1);
  const int32_t* btab = p.block_table + (size_t)b * p.bt_stride;
  const int blk0 = jb0;
  const int nb_unit = jb1 - jb0;   // at most tpc
  // mixed histories: the fields of the sink (h0), middle (hm) and recent (h1) parts as values
  const MixedLocal h0 = MIXED ? mixed_local(p.hi[0]) : MixedLocal{};
  const MixedLocal h1 = MIXED ? mixed_local(p.hi[1]) : MixedLocal{};
  const MixedLocal hm = MIXED ? mixed_local(MixedPart{p.pool, p.num_blocks, p.block_bytes, p.block_table, p.bt_stride,
                                                      p.seq_lens, p.max_seq_len})
                              : MixedLocal{};
  for (int j = tid; j < nb_unit; j += NT) {
    if constexpr (MIXED) {
      // the block's id in its part's pool, -1 when outside that pool
      const int jb = blk0 + j, part = mixed_part(jb, nS, nM), jl = jb - mixed_start(part, nS, nM);
      const int32_t* ht = (const int32_t*)(uintptr_t)by_part(part, (int64_t)(uintptr_t)h0.block_table,
                                                               (int64_t)(uintptr_t)hm.block_table,
                                                               (int64_t)(uintptr_t)h1.block_table);
      const int hs = (int)by_part(part, h0.bt_stride, hm.bt_stride, h1.bt_stride);
      const int64_t nbp = by_part(part, h0.num_blocks, hm.num_blocks, h1.num_blocks);
      const int id = ht[(size_t)b * hs + jl];
      const bool ok = id >= 0 && (int64_t)id < nbp;
      const int Lp = (int)by_part(part, Ls, Lm, Lr);
      const int vb = ok ? min(BLOCK_TOKENS, max(0, Lp - jl * BLOCK_TOKENS)) : 0;
      const uint8_t* base = (const uint8_t*)(uintptr_t)by_part(part, (int64_t)(uintptr_t)h0.pool,
                                                               (int64_t)(uintptr_t)hm.pool, (int64_t)(uintptr_t)h1.pool);
      const uint64_t a = (uint64_t)(uintptr_t)(base + (size_t)(ok ? id : 0) * (size_t)by_part(part, h0.block_bytes, hm.block_bytes, h1.block_bytes));
      btab2[j] = uint2{(uint32_t)a, (uint32_t)(a >> 32) | ((uint32_t)vb << 24)};
    } else {
      const int id = btab[blk0 + j];
      const bool ok = id >= 0 && (int64_t)id < p.num_blocks;
      const int vb = ok ? min(BLOCK_TOKENS, max(0, Lm - (blk0 + j) * BLOCK_TOKENS)) : 0;
      const uint64_t a = (uint64_t)(uintptr_t)(p.pool + (size_t)(ok ? id : 0) * (size_t)p.block_bytes);
      btab2[j] = uint2{(uint32_t)a, (uint32_t)(a >> 32) | ((uint32_t)vb << 24)};
    }
  }
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));   // queries and block ids, before any DMA
  __syncthreads();

  auto stage_src = [&](int s, int& half, int& valid) __attribute__((always_inline)) -> const uint8_t* {
    const int tok = T0 + s * ST_TOK;
    half = (tok / ST_TOK) & 1;
    // the block's address and valid tokens, resolved once per block before the loop
    const uint2 e = btab2[tok / BLOCK_TOKENS - blk0];
    const uint32_t lo = __builtin_amdgcn_readfirstlane(e.x), hi = __builtin_amdgcn_readfirstlane(e.y);
    valid = min(ST_TOK, max(0, (int)(hi >> 24) - half * ST_TOK));
    return (const uint8_t*)(uintptr_t)(((uint64_t)(hi & 0xFFFFFFu) << 32) | lo);
  };
  const uint32_t sbase = (uint32_t)(uintptr_t)(lds_void*)smem;
  auto bbuf = [&](int k) { return (bf16_t*)(smem + (k % 3) * BF); };
  auto cslot = [&](int k) { return smem + OFF_C + (k % DEPTH) * CBYTES; };
  auto pbuf = [&](int k) { return (bf16_t*)(smem + OFF_P + (k & 1) * 2 * PBYTES); };            // high term
  auto plbuf = [&](int k) { return (bf16_t*)(smem + OFF_P + (k & 1) * 2 * PBYTES + PBYTES); };  // low term
  // every thread issues its LOADS_LO / LOADS_HI pieces of a code stage.  The per-lane source
  // offsets of both halves of a block are computed once: address arithmetic before each DMA
  // instruction would sit in the issue stream of every step.
  // two separate arrays: a select between elements of one 2-D array becomes an indexed load,
  // which puts the array in scratch memory
  uint32_t doff0[QP::LOADS_LO], doff1[QP::LOADS_LO];
#pragma unroll
  for (int i = 0; i < QP::LOADS_LO; ++i) {
    const uint2 o = QP::piece_offsets(pl, groups, rgroups, i * NT + tid);
    doff0[i] = o.x;
    doff1[i] = o.y;
  }
  const uint32_t wslice = (uint32_t)__builtin_amdgcn_readfirstlane((tid & ~63) * 16);
  auto issue = [&](int k) __attribute__((always_inline)) {
    int half, valid;
    const uint8_t* blk = stage_src(k, half, valid);
    const uint32_t cst = sbase + OFF_C + (k % DEPTH) * CBYTES + wslice;
#pragma unroll
    for (int i = 0; i < QP::LOADS_LO; ++i) {
      if (i == QP::LOADS_HI && w >= QP::WAVES_LO) break;
      dma16s(blk, half ? doff1[i] : doff0[i], cst + (uint32_t)(i * NT * 16));
    }
  };
  // wait until code stage k has landed, `later` code stages having been issued after it
  auto wait_later = [&](int later) {
    auto wait_n = [&](auto K) {
      if (w < QP::WAVES_LO)
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(decltype(K)::value * QP::LOADS_LO));
      else
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(decltype(K)::value * QP::LOADS_HI));
    };
    switch (later) {
      case 0: wait_n(std::integral_constant<int, 0>{}); break;
      case 1: wait_n(std::integral_constant<int, 1>{}); break;
      case 2: wait_n(std::integral_constant<int, 2>{}); break;
      default: wait_n(std::integral_constant<int, 3>{}); break;
    }
  };

  // wavefront 0: scores of stage s, softmax, P into pbuf(s), rescale factors into alpha[s & 1]
  auto score_softmax = [&](int s) __attribute__((always_inline)) {
    const bf16_t* KS = bbuf(s);
    int half_unused, valid;
    stage_src(s, half_unused, valid);
    // k-step ks reads logical piece 4 ks + lg of token t, physical 8 (ks / 2) + ((4 (ks & 1) + lg)
    // ^ sw(t)): one base per token tile and k-step parity, the rest an immediate offset.  The
    // fragments of k-step ks + KD are read while k-step ks multiplies; two accumulation chains
    // per token tile keep dependent MFMAs four apart.
    f32x4 sv[2];
    {
      const bf16_t* kb[2][2];
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        const int t = tt * 16 + lr;
        const int f = sw(t);
        kb[tt][0] = &KS[t * 576 + (lg ^ f) * 8];
        kb[tt][1] = &KS[t * 576 + ((4 + lg) ^ f) * 8 - 32];
      }
      constexpr int KD = 4;
      bf16x8 a[KD + 1][2];
#pragma unroll
      for (int i = 0; i < KD; ++i)
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) a[i][tt] = *(const bf16x8*)(kb[tt][i & 1] + i * 32);
      f32x4 ac[2][2] = {};
#pragma unroll
      for (int ks = 0; ks < 18; ++ks) {
        if (ks + KD < 18) {
#pragma unroll
          for (int tt = 0; tt < 2; ++tt)
            a[(ks + KD) % (KD + 1)][tt] = *(const bf16x8*)(kb[tt][(ks + KD) & 1] + (ks + KD) * 32);
        }
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
          ac[tt][ks & 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[ks % (KD + 1)][tt], qreg[ks], ac[tt][ks & 1], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
      sv[0] = ac[0][0] + ac[0][1];
      sv[1] = ac[1][0] + ac[1][1];
    }
    // token 16 tt + 4 lg + i of the stage is kept if it is valid and within the row's limit
    const int tok0 = T0 + s * ST_TOK + 4 * lg;
    float mt = NEG_INF;
    if (valid == ST_TOK && T0 + s * ST_TOK + ST_TOK - 1 <= L - p.s_q) {
      // every token of the stage is visible to every row (rows past R have zero queries)
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          sv[tt][i] *= p.scale_log2;
          mt = fmaxf(mt, sv[tt][i]);
        }
    } else {
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int k = 16 * tt + 4 * lg + i;
          const bool ok = k < valid && tok0 + 16 * tt + i <= lim;
          sv[tt][i] = ok ? sv[tt][i] * p.scale_log2 : NEG_INF;
          mt = fmaxf(mt, sv[tt][i]);
        }
    }
    mt = wave_max_16_32(mt);
    const float mn = mt > m_s + RESCALE_SLACK ? mt : m_s;
    const float mu = mn == NEG_INF ? 0.f : mn;
    const float al = mn == m_s ? 1.f : __builtin_amdgcn_exp2f(m_s - mu);
    l_x *= al;
    m_s = mn;
    bf16_t* P = pbuf(s);
    bf16_t* PL = plbuf(s);
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      float pf[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        pf[i] = __builtin_amdgcn_exp2f(sv[tt][i] - mu);
        l_x += pf[i];
      }
      uint32_t h0, l0, h1, l1;
      split_pair(pf[0], pf[1], h0, l0);
      split_pair(pf[2], pf[3], h1, l1);
      *(uint2*)&P[lr * PROW + tt * 16 + lg * 4] = uint2{h0, h1};
      *(uint2*)&PL[lr * PROW + tt * 16 + lg * 4] = uint2{l0, l1};
    }
    if (lg == 0) alpha[s & 1][lr] = al;
  };

  // O[16 rows][64 cg .. 64 cg + 63] = alpha(s) O + (P_hi(s) + P_lo(s)) . C(s) into accumulators o
  auto pv = [&](int s, int cg, f32x4 (&o)[4]) {
    const bf16_t* KS = bbuf(s);
    const f32x4 al = *(const f32x4*)&alpha[s & 1][lg * 4];
    if (__any(al[0] != 1.f || al[1] != 1.f || al[2] != 1.f || al[3] != 1.f)) {
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) o[nt] *= al;
    }
    f32x4* acc = o;
    const bf16x8 a = *(const bf16x8*)&pbuf(s)[lr * PROW + lg * 8];
    const bf16x8 al_ = *(const bf16x8*)&plbuf(s)[lr * PROW + lg * 8];
    const int t0 = lg * 8 + (lr >> 2);
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      const int d = cg * 64 + nt * 16 + (lr & 3) * 4;
      const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)&KS[st_off(t0, d)]);
      const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)&KS[st_off(t0 + 4, d)]);
      const bf16x8 bv = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bv, acc[nt], 0, 0, 0);
      acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al_, bv, acc[nt], 0, 0, 0);
    }
  };

  // mixed histories: a bf16 block of stage k by DMA into bf16 buffer k (waves 0-3 issue 5
  // instructions, waves 4-7 four), and its rows past the part's end zeroed once landed
  auto is_bf = [&](int k) __attribute__((always_inline)) {
    return MIXED && mixed_part((T0 + k * ST_TOK) / BLOCK_TOKENS, nS, nM) != 1;
  };
  auto issue_bf = [&](int k) __attribute__((always_inline)) {
    int half, valid;
    const uint8_t* blk = stage_src(k, half, valid);
    pipe_issue_bf16(blk + half * ST_TOK * 1152, bbuf(k), tid);
  };
  auto zero_rows = [&](int k) __attribute__((always_inline)) {
    int half_unused, valid;
    stage_src(k, half_unused, valid);
    if (valid < ST_TOK) pipe_zero_rows(bbuf(k), valid, tid, NT);
  };

  if (nst > 0) {
    // prologue: code stages 0..3 issued, 0 and 1 dequantised by every thread, code 4 issued,
    // stage 0 scored, code 2 landed
    for (int k = 0; k < DEPTH && k < nst; ++k) issue(k);
    bool bf_pro = false;
    for (int k = 0; k < 2 && k < nst; ++k)
      if (is_bf(k)) {
        issue_bf(k);
        bf_pro = true;
      }
    if (bf_pro) __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    else wait_later(min(nst - 1, DEPTH - 1) - min(nst - 1, 1));
    lds_barrier();
    for (int k = 0; k < 2 && k < nst; ++k) {
      if (is_bf(k)) {
        zero_rows(k);
      } else {
        int half_unused, valid;
        stage_src(k, half_unused, valid);
        QP::dequant(cslot(k), valid, gl_log2, gr_log2, bbuf(k), tid);
      }
    }
    lds_barrier();
    if (DEPTH < nst) issue(DEPTH);
    if (w == 0) score_softmax(0);
    if (2 < nst) wait_later(min(nst - 1, DEPTH) - 2);
    lds_barrier();

    // step s; BF2: stage s + 2 is a bf16 block of a mixed history
    auto step = [&](int s, auto BF2) __attribute__((always_inline)) {
      constexpr bool bf2 = decltype(BF2)::value;
      // a bf16 block of stage s + 2: its DMA into the buffer of stage s - 1 (read in step s - 1)
      // before this step's code refill
      if constexpr (bf2) issue_bf(s + 2);
      // refill the slot of code s + 1 (dequantised in step s - 1) with code s + 5
      const bool refill = s + DEPTH + 1 < nst;
      if (refill) issue(s + DEPTH + 1);
      if (w == 0 && s + 1 < nst) score_softmax(s + 1);
      pv(s, w, acc);
      // dequantisation by wavefronts 1-7: the 768 tasks over their 448 lanes, lane slot q of
      // wavefront w taking tasks q and 448 + q.  Slots 0..63 get two latent tasks, 64..319 a
      // latent and a RoPE task, 320..447 one latent task; waves are dealt to SIMDs w mod 4, so
      // the slot blocks go to waves (1..7) as 0, 1, 3, 6, 5, 2, 4: the SIMDs that share no
      // wavefront with the scorer carry 3 + 0, 2 + 2 and 2 + 2 latent + RoPE tasks, and
      // wavefront 4, beside the scorer, one latent task
      if constexpr (!bf2) {
        if (w != 0 && s + 2 < nst) {
          int half_unused, valid;
          stage_src(s + 2, half_unused, valid);
          const int q = (int)((0x42563100u >> (4 * w)) & 15u) * 64 + lane;
#pragma unroll
          for (int it = 0; it < 2; ++it)
            if (it * 448 + q < 768) QP::dequant_task(cslot(s + 2), valid, it * 448 + q, gl_log2, gr_log2, bbuf(s + 2));
        }
      }
      // code s + 3 landed (dequantised in the next step); nobody reads the buffers of stage s
      if constexpr (bf2) {
        // the bf16 rows of stage s + 2 (issued before this step's refill) and every code stage
        if (!refill) __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
        else if (w < QP::WAVES_LO) __builtin_amdgcn_s_waitcnt(vmcnt_imm(QP::LOADS_LO));
        else __builtin_amdgcn_s_waitcnt(vmcnt_imm(QP::LOADS_HI));
        lds_barrier();
        zero_rows(s + 2);
      } else if (s + 3 < nst) {
        wait_later(min(nst - 1, s + DEPTH + 1) - (s + 3));
      }
      lds_barrier();
    };
    if constexpr (!MIXED) {
      for (int s = 0; s < nst; ++s) step(s, std::false_type{});
    } else {
      // The partition's stages k < kS are sink blocks and k >= kR recent-window blocks.  The
      // steps run in stretches whose stage s + 2 is low-bit (or past the end), each a loop with
      // no bf16 code in its body (the bf16 path inside every step's code slowed the whole loop
      // by ~6% even where it was never taken), and the steps whose stage s + 2 is a bf16 block
      // one by one in between.
      const int kS = max(0, 2 * (nS - jb0)), kR = max(0, 2 * (nS + nM - jb0));
      int s = 0;
      while (s < nst) {
        int e = s + 2 < kS ? s : max(s, kR - 2);
        e = e + 2 < nst ? e : nst;
        for (; s < e; ++s) step(s, std::false_type{});
        if (s < nst) step(s++, std::true_type{});
      }
    }
  }

  // ---- finish: wavefront 0 publishes the row sums and maxima; every wavefront normalises and
  // writes its 64 columns
  if (w == 0) {
    const float lx = wave_sum_16_32(l_x);
    if (lg == 0) {
      fin[0][lr] = lx;
      fin[1][lr] = m_s;
    }
  }
  lds_barrier();
  const size_t unit_row0 = ((size_t)b * p.max_chunks + c) * R;
  auto write_cols = [&](int cg, const f32x4 (&o4)[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = lg * 4 + i;
      if (row >= R) continue;
      const float lt = fin[0][row];
      const float inv = lt > 0.f ? 1.f / lt : 0.f;
      const size_t obase = (unit_row0 + row) * 512 + cg * 64 + lr;
      if (p.out_bf16) {
        bf16_t* o = (bf16_t*)p.out;
#pragma unroll
        for (int nt = 0; nt < 4; ++nt)
          o[obase + nt * 16] = __builtin_bit_cast(bf16_t, (uint16_t)f32_to_bf16_bits(o4[nt][i] * inv));
      } else {
        float* o = (float*)p.out;
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) o[obase + nt * 16] = o4[nt][i] * inv;
      }
    }
  };
  write_cols(w, acc);
  if (p.out_lse != nullptr && tid < 16 && tid < R) {
    const float lt = fin[0][tid];
    p.out_lse[unit_row0 + tid] = lt > 0.f ? (fin[1][tid] + __log2f(lt)) * 0.69314718055994531f : NEG_INF;
  }
}

// ---------------------------------------------------------------------------------------
// The in-loop dequantisation of the kernels above, on its own (test/debug): one workgroup per
// half block streams the code planes into a code stage with the decode's DMA producer,
// dequantises them with the decode's own QuantProducer::dequant into a swizzled bf16 stage,
// and copies the stage out un-swizzled.  Block ids outside the pool give zero rows, as the
// decode's zero scales for them do.
// ---------------------------------------------------------------------------------------
template <int FMT>
__global__ __launch_bounds__(NT) void dequant_stage_kernel(DequantParams p) {
  using QP = QuantProducer<FMT>;
  __shared__ __attribute__((aligned(16))) uint8_t cst[QP::SLOTS * 16];
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
  QP::issue(p.pool + (size_t)id * (size_t)p.block_bytes, half, pl, 512 / p.g_lat, 64 / p.g_rope, cst, tid);
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
  __syncthreads();
  QP::dequant(cst, valid, 31 - __builtin_clz(p.g_lat), 31 - __builtin_clz(p.g_rope), stage, tid);
  lds_barrier();
  uint16_t* out = p.out + ((size_t)k * BLOCK_TOKENS + half * ST_TOK) * 576;
  for (int q = tid; q < ST_TOK * 72; q += NT) {
    const int t = q / 72, c8 = q % 72;
    *(u32x4*)(out + t * 576 + c8 * 8) = *(const u32x4*)&stage[st_off(t, c8 * 8)];
  }
}

hipError_t launch_dequant_partition(const DequantParams& p, int fmt, hipStream_t st) {
  if (fmt == FMT_INT4)
    hipLaunchKernelGGL(dequant_stage_kernel<FMT_INT4>, dim3(2 * p.n), dim3(NT), 0, st, p);
  else if (fmt == FMT_INT2)
    hipLaunchKernelGGL(dequant_stage_kernel<FMT_INT2>, dim3(2 * p.n), dim3(NT), 0, st, p);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------------------
template <int RT, int FMT>
static hipError_t launch_mfma(const DecodeParams& p, int grid, hipStream_t st) {
  if constexpr (RT == 1 && FMT != FMT_BF16) {
    // quantised cache, at most 16 rows: the pipelined kernel when its code stage holds the
    // layout, else the split kernel with 32-row tiles (same grid: one row group either way)
    // (and when the pool ends beyond the 56 bits of its per-block address table)
    const uint64_t pool_end = (uint64_t)(uintptr_t)p.pool + (uint64_t)p.num_blocks * (uint64_t)p.block_bytes;
    if (PipeQP<FMT>::slots_needed(512 / p.g_lat, 64 / p.g_rope) > PipeQP<FMT>::SLOTS || pool_end >= kPipeAddrLimit)
      return launch_mfma<2, FMT>(p, grid, st);
    if (p.q_f32)
      hipLaunchKernelGGL((decode_pipe_kernel<FMT, true, false>), dim3(grid), dim3(NT), 0, st, p);
    else
      hipLaunchKernelGGL((decode_pipe_kernel<FMT, false, false>), dim3(grid), dim3(NT), 0, st, p);
    return hipGetLastError();
  }
  if (p.q_f32)
    hipLaunchKernelGGL((decode_mfma_kernel<RT, FMT, true>), dim3(grid), dim3(NT), 0, st, p);
  else
    hipLaunchKernelGGL((decode_mfma_kernel<RT, FMT, false>), dim3(grid), dim3(NT), 0, st, p);
  return hipGetLastError();
}

template <int RT>
static hipError_t launch_fmt(const DecodeParams& p, int fmt, int grid, hipStream_t st) {
  switch (fmt) {
    case FMT_BF16: return launch_mfma<RT, FMT_BF16>(p, grid, st);
    case FMT_INT4: return launch_mfma<RT, FMT_INT4>(p, grid, st);
    case FMT_INT2: return launch_mfma<RT, FMT_INT2>(p, grid, st);
  }
  return hipErrorInvalidValue;
}

bool pipe_mixed_fits(int fmt, int g_lat, int g_rope) {
  if (g_lat <= 0 || g_rope <= 0) return false;
  if (fmt == FMT_INT4) return PipeQP<FMT_INT4>::slots_needed(512 / g_lat, 64 / g_rope) <= PipeQP<FMT_INT4>::SLOTS;
  if (fmt == FMT_INT2) return PipeQP<FMT_INT2>::slots_needed(512 / g_lat, 64 / g_rope) <= PipeQP<FMT_INT2>::SLOTS;
  return false;
}

template <int FMT>
static hipError_t launch_pipe_mixed(const DecodeParams& p, hipStream_t st) {
  const int grid = 8 * p.units_per_xcd;
  if (p.q_f32)
    hipLaunchKernelGGL((decode_pipe_kernel<FMT, true, true>), dim3(grid), dim3(NT), 0, st, p);
  else
    hipLaunchKernelGGL((decode_pipe_kernel<FMT, false, true>), dim3(grid), dim3(NT), 0, st, p);
  return hipGetLastError();
}

hipError_t launch_decode_pipe_mixed(const DecodeParams& p, int fmt, hipStream_t st) {
  if (!pipe_mixed_fits(fmt, p.g_lat, p.g_rope) || p.R > 16) return hipErrorInvalidValue;
  if (fmt == FMT_INT4) return launch_pipe_mixed<FMT_INT4>(p, st);
  if (fmt == FMT_INT2) return launch_pipe_mixed<FMT_INT2>(p, st);
  return hipErrorInvalidValue;
}

hipError_t launch_decode_mfma(const DecodeParams& p, int fmt, int rt, hipStream_t st) {
  const int grid = 8 * p.units_per_xcd;
  switch (rt) {
    case 1: return launch_fmt<1>(p, fmt, grid, st);
    case 2: return launch_fmt<2>(p, fmt, grid, st);
    case 4: return launch_fmt<4>(p, fmt, grid, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace mla
