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
//     is written to LDS in bf16;
//   * O += P . C on the same MFMA: wave w owns latent columns [64w, 64w + 64)
//     of all rows; the C operand comes from the token-major stage with
//     ds_read_b64_tr_b16.
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

// 16 bytes per lane from base + off (base wave-uniform, off per lane) to LDS bytes
// [lds_base + 16 lane, + 16).  With the per-lane offsets precomputed, an issue costs no VALU
// work.  One wait state between the M0 write and the DMA; the kernel makes no other use of M0.
__device__ __forceinline__ void dma16s(const uint8_t* base, uint32_t off, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(lds_base), "v"(off), "s"(base)
               : "memory", "m0");
}

__device__ __forceinline__ float wave_max_16_32(float v) {
  v = fmaxf(v, __shfl_xor(v, 16, 64));
  v = fmaxf(v, __shfl_xor(v, 32, 64));
  return v;
}
__device__ __forceinline__ float wave_sum_16_32(float v) {
  v += __shfl_xor(v, 16, 64);
  v += __shfl_xor(v, 32, 64);
  return v;
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
// copied into a flat code stage [lc | ls | rc | rs], padded to SLOTS pieces.
template <int FMT>
struct QuantProducer {
  static constexpr int BITS = FMT == FMT_INT4 ? 4 : 2;
  static constexpr int LB = 512 * BITS / 8;        // latent code bytes per token
  static constexpr int PPT = LB / 16;              // latent code pieces (16 B) per token
  // code stage capacity in 16-byte slots: INT4 waves 0-3 issue 2 instructions, waves 4-7 one
  static constexpr int LOADS_LO = FMT == FMT_INT4 ? 2 : 1;
  static constexpr int LOADS_HI = 1;
  static constexpr int SLOTS = FMT == FMT_INT4 ? 768 : 512;
  __device__ __forceinline__ static void issue(const uint8_t* blk, int half, const QuantPlanes& pl, int groups,
                                               int rgroups, uint8_t* cstage, int tid) {
    const int n_lc = ST_TOK * LB / 16;
    const int n_ls = ST_TOK * groups * 4 / 16;
    const int n_rc = ST_TOK * 32 / 16;
    const int n_rs = (ST_TOK * rgroups * 4 + 15) / 16;
    const int n_all = n_lc + n_ls + n_rc + n_rs;
    const uint8_t* lc = blk + pl.lc + half * ST_TOK * LB;
    const uint8_t* ls = blk + pl.ls + half * ST_TOK * groups * 4;
    const uint8_t* rc = blk + pl.rc + half * ST_TOK * 32;
    const uint8_t* rs = blk + pl.rs + half * ST_TOK * rgroups * 4;
    const int wbase = tid & ~63;
#pragma unroll
    for (int i = 0; i < LOADS_LO; ++i) {
      if (i == LOADS_HI && tid >= 256) break;
      const int slot = i * NT + tid;
      // padding slots re-load a real piece (spread over the stage, never one shared address)
      int p = slot < n_all ? slot : slot - n_all;
      const uint8_t* src;
      if (p < n_lc) {
        // latent code pieces are stored piece-major: slot k * 32 + t holds piece k of token t
        src = lc + ((p % ST_TOK) * PPT + p / ST_TOK) * 16;
      } else if ((p -= n_lc) < n_ls) {
        src = ls + p * 16;
      } else if ((p -= n_ls) < n_rc) {
        src = rc + ((p % ST_TOK) * 2 + p / ST_TOK) * 16;   // rope code halves, also piece-major
      } else {
        src = rs + (p - n_rc) * 16;
      }
      dma16(src, (lds_void*)(cstage + (size_t)(i * NT + wbase) * 16));
    }
  }

  // Per-thread dequantisation work, fixed for the whole partition.  Thread q owns latent
  // chunk kk = q / 32 (32 elements, inside one quantisation group since groups are multiples
  // of 32) of token t = q mod 32: a wavefront's code reads are contiguous and its swizzled
  // bf16 stores spread over all banks.  Threads 0..255 also own 8 RoPE elements
  // (token rt, elements 8 ri .. 8 ri + 7).
  struct Work {
    int t, code, sz, dst;       // latent: token, code byte offset, scale byte offset, stage element
    int rt, rcode, rsz, rdst;   // rope (tid < 256)
  };
  __device__ __forceinline__ static Work plan(int groups, int rgroups, int tid) {
    Work w;
    w.t = tid & 31;
    const int kk = tid >> 5;                      // 0..15
    const int cpiece = (kk * 32 * BITS) / 128;    // 16-byte code piece holding the chunk
    const int cbyte = ((kk * 32 * BITS) / 8) & 15;
    w.code = (cpiece * ST_TOK + w.t) * 16 + cbyte;
    w.sz = ST_TOK * LB + (w.t * groups + (kk * 32) / (512 / groups)) * 4;
    w.dst = st_off(w.t, kk * 32);
    w.rt = tid & 31;
    const int ri = (tid >> 5) & 7;
    w.rcode = ST_TOK * LB + ST_TOK * groups * 4 + ((ri >> 2) * ST_TOK + w.rt) * 16 + (ri & 3) * 4;
    w.rsz = ST_TOK * LB + ST_TOK * groups * 4 + ST_TOK * 32 + (w.rt * rgroups + (ri * 8) / (64 / rgroups)) * 4;
    w.rdst = st_off(w.rt, 512 + ri * 8);
    return w;
  }

  // codes -> swizzled bf16 stage; tokens >= valid become zeros (scale and zero-point 0)
  __device__ __forceinline__ static void dequant(const uint8_t* cst, int valid, const Work& w, bf16_t* stage,
                                                 int tid) {
    uint32_t sz = *(const uint32_t*)(cst + w.sz);
    sz = w.t < valid ? sz : 0u;
    float s, zs;
    scale_zero(sz, s, zs);
    // element 32 kk + 8 j sits at physical piece (4 kk + j) ^ sw(t) = (base piece) ^ j
    const int row = w.t * 576;
    const int p0 = (w.dst - row) >> 3;
    if constexpr (BITS == 4) {
      const u32x4 c = *(const u32x4*)(cst + w.code);
#pragma unroll
      for (int j = 0; j < 4; ++j) lds_store16(&stage[row + ((p0 ^ j) << 3)], dequant_int4x8(c[j], s, zs));
    } else {
      const uint2 c = *(const uint2*)(cst + w.code);
      uint32_t t_lo, t_hi;
      int2_table(s, zs, t_lo, t_hi);
      u32x4 lo, hi;
      dequant_int2x16(c.x, t_lo, t_hi, lo, hi);
      lds_store16(&stage[row + ((p0 ^ 0) << 3)], lo);
      lds_store16(&stage[row + ((p0 ^ 1) << 3)], hi);
      dequant_int2x16(c.y, t_lo, t_hi, lo, hi);
      lds_store16(&stage[row + ((p0 ^ 2) << 3)], lo);
      lds_store16(&stage[row + ((p0 ^ 3) << 3)], hi);
    }
    if (tid < 256) {
      uint32_t rsz = *(const uint32_t*)(cst + w.rsz);
      rsz = w.rt < valid ? rsz : 0u;
      float rsc, rzs;
      scale_zero(rsz, rsc, rzs);
      lds_store16(&stage[w.rdst], dequant_int4x8(*(const uint32_t*)(cst + w.rcode), rsc, rzs));
    }
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

  // bf16 path: a 4-deep ring of bf16 stages.  Quantised path: an 8-deep ring of code stages
  // and one bf16 stage that every step dequantises into.  Distinct arrays let the compiler
  // see that reading one ring slot does not depend on the DMA into another.
  constexpr int DEPTH = QUANT ? 8 : 4;
  __shared__ __attribute__((aligned(16))) bf16_t S0[ST_ELEMS];
  __shared__ __attribute__((aligned(16))) bf16_t S1[QUANT ? 8 : ST_ELEMS];
  __shared__ __attribute__((aligned(16))) bf16_t S2[QUANT ? 8 : ST_ELEMS];
  __shared__ __attribute__((aligned(16))) bf16_t S3[QUANT ? 8 : ST_ELEMS];
  __shared__ __attribute__((aligned(16))) uint8_t C0[CBYTES];
  __shared__ __attribute__((aligned(16))) uint8_t C1[CBYTES];
  __shared__ __attribute__((aligned(16))) uint8_t C2[CBYTES];
  __shared__ __attribute__((aligned(16))) uint8_t C3[CBYTES];
  __shared__ __attribute__((aligned(16))) uint8_t C4[CBYTES];
  __shared__ __attribute__((aligned(16))) uint8_t C5[CBYTES];
  __shared__ __attribute__((aligned(16))) uint8_t C6[CBYTES];
  __shared__ __attribute__((aligned(16))) uint8_t C7[CBYTES];
  __shared__ __attribute__((aligned(16))) bf16_t Ps[ROWS * PROW];
  __shared__ float red[2][ROWS];
  __shared__ float redl[2][ROWS];   // row sums of the bf16-rounded P (normalise o)
  __shared__ float redx[2][ROWS];   // row sums of the unrounded P (lse)
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
  float m_s = NEG_INF, l_s = 0.f, l_x = 0.f;
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
    const int n = w < 4 ? LA : LB;
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

  const typename QP::Work dq = QP::plan(groups, rgroups, tid);

  // prologue: stages 0 .. DEPTH-2 in flight; stage 0 landed
  if constexpr (QUANT) {
    if (0 < nst) issue(0, S0, C0);
    if (1 < nst) issue(1, S0, C1);
    if (2 < nst) issue(2, S0, C2);
    if (3 < nst) issue(3, S0, C3);
    if (4 < nst) issue(4, S0, C4);
    if (5 < nst) issue(5, S0, C5);
    if (6 < nst) issue(6, S0, C6);
  } else {
    if (0 < nst) issue(0, S0, C0);
    if (1 < nst) issue(1, S1, C0);
    if (2 < nst) issue(2, S2, C0);
  }
  wait_stage(min(nst - 1, DEPTH - 2));
  lds_barrier();

  // one stage: KS = bf16 stage read by the MFMAs, CCUR = its code stage (quantised formats),
  // NXT/CNXT = ring slot refilled with stage s + DEPTH - 1
  auto step = [&](int s, bf16_t* KS, uint8_t* CCUR, bf16_t* NXT, uint8_t* CNXT) {
    // stage s has landed and every wave is done with stage s-1 (barrier at the end of the
    // previous step), so the ring slot of stage s-1 can take stage s + DEPTH - 1
    if (s + DEPTH - 1 < nst) issue(s + DEPTH - 1, NXT, CNXT);
    int half_unused, valid;
    stage_src(s, half_unused, valid);
    if constexpr (QUANT) {
      QP::dequant(CCUR, valid, dq, KS, tid);
      lds_barrier();
    } else if (valid < ST_TOK) {
      // rows past the sequence end were filled from a dummy address: zero them
      for (int q = tid; q < (ST_TOK - valid) * 72; q += NT)
        *(u32x4*)&KS[(valid + q / 72) * 576 + (q % 72) * 8] = u32x4{0, 0, 0, 0};
      lds_barrier();
    }

    // ---- scores for (row tile sc_rt, token tile sc_tt)
    f32x4 sv = {0.f, 0.f, 0.f, 0.f};
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
    lds_barrier();

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
      l_s *= al;
      l_x *= al;
      m_s = mn;
      if (sc_tt == 0 && lg == 0) alpha[row_s] = al;
      uint32_t pb[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float pf = __builtin_amdgcn_exp2f(sv[i] - mu);
        pb[i] = f32_to_bf16_bits(pf);
        l_s += bf16_bits_to_f32(pb[i]);
        l_x += pf;
      }
      *(uint2*)&Ps[row_s * PROW + sc_tt * 16 + lg * 4] = uint2{pb[0] | (pb[1] << 16), pb[2] | (pb[3] << 16)};
    }
    lds_barrier();
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

    // ---- O[rows][64w .. 64w+63] += P . C over the 32 tokens of the stage
    {
      bf16x8 a[RT];
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) a[rt] = *(const bf16x8*)&Ps[(rt * 16 + lr) * PROW + lg * 8];
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
      }
    }
    // stage s+1 landed, and nobody reads stage s any more
    wait_stage(min(nst - 2 - s, DEPTH - 2));
    lds_barrier();
  };

  if constexpr (!QUANT) {
    for (int s = 0; s < nst; s += 4) {
      step(s, S0, C0, S3, C3);
      if (s + 1 < nst) step(s + 1, S1, C1, S0, C0);
      if (s + 2 < nst) step(s + 2, S2, C2, S1, C1);
      if (s + 3 < nst) step(s + 3, S3, C3, S2, C2);
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
    l_s = wave_sum_16_32(l_s);
    l_x = wave_sum_16_32(l_x);
    if (lg == 0) {
      redl[sc_tt][row_s] = l_s;
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
      const float lt = redl[0][row] + redl[1][row];
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
// launchers
// ---------------------------------------------------------------------------------------
template <int RT, int FMT>
static hipError_t launch_mfma(const DecodeParams& p, int grid, hipStream_t st) {
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
