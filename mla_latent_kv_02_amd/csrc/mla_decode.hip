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

#include "mla_device.hpp"
#include "mla_internal.hpp"

namespace mla {

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr int NT = 512;                // threads per workgroup (8 waves)
constexpr int ST_TOK = 32;             // tokens per stage
constexpr int ST_PIECES = ST_TOK * 72; // 16-byte pieces per bf16 stage
constexpr int ST_ELEMS = ST_TOK * 576;
constexpr int PROW = ST_TOK + 8;       // bf16 elements per LDS P row
constexpr int MAX_TPC = 256;           // paged blocks per partition (host planner caps it)

// s_waitcnt immediate: wait until at most n vector-memory operations are outstanding
__host__ __device__ constexpr int vmcnt_imm(int n) { return (n & 0xF) | ((n >> 4) << 14) | (7 << 4) | (0xF << 8); }

// All LDS traffic of this wave is complete, then workgroup barrier.  The memory
// clobber keeps the compiler from moving memory operations across it, without
// the release fence that would also wait for the in-flight LDS DMA of later stages.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Stage layout: token row t holds its 72 pieces (8 bf16 each) in 9 groups of 8; piece c sits
// at physical piece c ^ sw(t), an XOR inside its group.  Rows are 288 dwords apart (32 mod 64
// banks).  gfx950 serves a 16-byte LDS access 16 lanes per cycle, a lane set being (lane bit 5,
// parity of lane bits 2..4), and ds_read_b64_tr_b16 32 consecutive lanes per cycle.  sw() is
// the XOR pattern under which all four access patterns of a stage fill 64 distinct banks per
// cycle: the score operand reads (16 tokens x 4 consecutive pieces per wave), the transposed
// P.C operand reads, and the dequantised latent and RoPE piece stores of the quantised formats.
__device__ __forceinline__ int sw(int t) { return (t & 2) | ((t >> 1) & 4) | ((t >> 4) & 1); }
// bf16 element offset of (token t, latent/rope column d) in a stage
__device__ __forceinline__ int st_off(int t, int d) { return t * 576 + (((d >> 3) ^ sw(t)) << 3) + (d & 7); }

__device__ __forceinline__ void dma16(const void* src, lds_void* dst) {
  __builtin_amdgcn_global_load_lds(src, dst, 16, 0, 0);
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
template <>
struct Producer<FMT_BF16> {
  static constexpr int LOADS_LO = 5;  // waves 0..3
  static constexpr int LOADS_HI = 4;  // waves 4..7
  __device__ __forceinline__ static void issue(const uint8_t* half, int valid, bf16_t* stage, int tid) {
    const int wbase = tid & ~63;
#pragma unroll
    for (int i = 0; i < LOADS_LO; ++i) {
      if (i == LOADS_HI && tid >= 256) break;
      const int slot = i * NT + tid;
      const int t = slot / 72;
      const int c = (slot - t * 72) ^ sw(t);  // logical piece held by this physical slot
      const uint8_t* src = t < valid ? half + t * 1152 + c * 16 : half;
      dma16(src, (lds_void*)(stage + (size_t)(i * NT + wbase) * 8));
    }
  }
};

// Quantised latent (INT4 or INT2) + INT4 rope: the four code planes of a half block are
// copied into a flat code stage [lc | ls | rc | rs], padded to SLOTS pieces.
template <int FMT>
struct QuantProducer {
  static constexpr int BITS = FMT == FMT_INT4 ? 4 : 2;
  static constexpr int LB = 512 * BITS / 8;        // latent code bytes per token
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
        // latent code pieces are stored swizzled: slot t*PPT + (k ^ (t & 7)) holds piece k of token t
        constexpr int PPT = LB / 16;
        const int t = p / PPT;
        const int k = (p % PPT) ^ (t & 7);
        src = lc + (t * PPT + k) * 16;
      } else if ((p -= n_lc) < n_ls) {
        src = ls + p * 16;
      } else if ((p -= n_ls) < n_rc) {
        src = rc + p * 16;
      } else {
        src = rs + (p - n_rc) * 16;
      }
      dma16(src, (lds_void*)(cstage + (size_t)(i * NT + wbase) * 16));
    }
  }

  // codes -> swizzled bf16 stage; tokens >= valid become zeros
  __device__ __forceinline__ static void dequant(const uint8_t* cstage, int valid, int groups, int rgroups, bf16_t* stage, int tid) {
    const int g_lat = 512 / groups;
    const uint8_t* lc = cstage;
    const uint32_t* ls = (const uint32_t*)(cstage + ST_TOK * LB);
    const uint8_t* rc = cstage + ST_TOK * LB + ST_TOK * groups * 4;
    const uint32_t* rs = (const uint32_t*)(rc + ST_TOK * 32);
    constexpr int ELEMS = 128 / BITS;          // elements per 16-byte code piece
    constexpr int PPT = LB / 16;               // latent pieces per token
    constexpr int NLP = ST_TOK * PPT;          // latent pieces per stage
    // Thread mapping: 8 consecutive lanes take 8 consecutive tokens and the same code piece k,
    // so the swizzled code reads and the swizzled bf16 writes both spread over all banks.
    for (int q = tid; q < NLP + 2 * ST_TOK; q += NT) {
      if (q < NLP) {
        const int g = q >> 3;
        const int t = (q & 7) + 8 * (g & 3);
        const int k = g >> 2;
        const int e0 = k * ELEMS;
        if (t >= valid) {
#pragma unroll
          for (int j = 0; j < ELEMS / 8; ++j) *(u32x4*)&stage[st_off(t, e0 + 8 * j)] = u32x4{0, 0, 0, 0};
          continue;
        }
        const u32x4 c = *(const u32x4*)(lc + (t * PPT + (k ^ (t & 7))) * 16);
        float s0, zs0, s1, zs1;
        scale_zero(ls[t * groups + e0 / g_lat], s0, zs0);
        scale_zero(ls[t * groups + (e0 + ELEMS / 2) / g_lat], s1, zs1);
        if (BITS == 4) {
#pragma unroll
          for (int j = 0; j < 4; ++j)
            *(u32x4*)&stage[st_off(t, e0 + 8 * j)] = dequant_int4x8(c[j], j < 2 ? s0 : s1, j < 2 ? zs0 : zs1);
        } else {
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const float s = j < 2 ? s0 : s1, zs = j < 2 ? zs0 : zs1;
            *(u32x4*)&stage[st_off(t, e0 + 16 * j)] = dequant_int2x8(c[j] & 0xFFFFu, s, zs);
            *(u32x4*)&stage[st_off(t, e0 + 16 * j + 8)] = dequant_int2x8(c[j] >> 16, s, zs);
          }
        }
      } else {
        const int r = q - NLP;
        const int t = r & 31;
        const int hr = r >> 5;
        const int e0 = 512 + hr * 32;
        if (t >= valid) {
#pragma unroll
          for (int j = 0; j < 4; ++j) *(u32x4*)&stage[st_off(t, e0 + 8 * j)] = u32x4{0, 0, 0, 0};
          continue;
        }
        const u32x4 c = *(const u32x4*)(rc + (t * 2 + hr) * 16);
        float s, zs;
        scale_zero(rs[t * rgroups + (hr * 32) / (64 / rgroups)], s, zs);
#pragma unroll
        for (int j = 0; j < 4; ++j) *(u32x4*)&stage[st_off(t, e0 + 8 * j)] = dequant_int4x8(c[j], s, zs);
      }
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

  // bf16 path: 4 bf16 stages.  quantised path: 4 code stages + 2 bf16 stages.
  __shared__ __attribute__((aligned(16))) bf16_t S0[ST_ELEMS];
  __shared__ __attribute__((aligned(16))) bf16_t S1[ST_ELEMS];
  __shared__ __attribute__((aligned(16))) bf16_t S2[QUANT ? 8 : ST_ELEMS];
  __shared__ __attribute__((aligned(16))) bf16_t S3[QUANT ? 8 : ST_ELEMS];
  __shared__ __attribute__((aligned(16))) uint8_t C0[CBYTES];
  __shared__ __attribute__((aligned(16))) uint8_t C1[CBYTES];
  __shared__ __attribute__((aligned(16))) uint8_t C2[CBYTES];
  __shared__ __attribute__((aligned(16))) uint8_t C3[CBYTES];
  __shared__ __attribute__((aligned(16))) bf16_t Ps[ROWS * PROW];
  __shared__ float red[2][ROWS];
  __shared__ float redl[2][ROWS];
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
  float m_s = NEG_INF, l_s = 0.f;
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
  auto issue = [&](int s, bf16_t* st, uint8_t* cst) {
    int half, valid;
    const uint8_t* blk = stage_src(s, half, valid);
    if constexpr (QUANT)
      Prod::issue(blk, half, pl, groups, rgroups, cst, tid);
    else
      Prod::issue(blk + half * ST_TOK * 1152, valid, st, tid);
  };
  // wait until stage s has landed, given how many later stages were issued after it
  auto wait_stage = [&](int later) {
    constexpr int LA = QUANT ? QP::LOADS_LO : Producer<FMT_BF16>::LOADS_LO;
    constexpr int LB = QUANT ? QP::LOADS_HI : Producer<FMT_BF16>::LOADS_HI;
    if (w < 4) {
      if (later >= 2) __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * LA));
      else if (later == 1) __builtin_amdgcn_s_waitcnt(vmcnt_imm(LA));
      else __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    } else {
      if (later >= 2) __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * LB));
      else if (later == 1) __builtin_amdgcn_s_waitcnt(vmcnt_imm(LB));
      else __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    }
  };

  // prologue: stages 0, 1, 2 in flight; stage 0 landed
  if (0 < nst) issue(0, S0, C0);
  if (1 < nst) issue(1, S1, C1);
  if (2 < nst) issue(2, QUANT ? S0 : S2, C2);
  wait_stage(min(nst - 1, 2));
  lds_barrier();

  // one stage: KS = bf16 stage read by the MFMAs, NXT/CNXT = ring slot refilled with stage s+3
  auto step = [&](int s, bf16_t* KS, uint8_t* CCUR, bf16_t* NXT, uint8_t* CNXT) {
    // stage s has landed and every wave is done with stage s-1 (barrier at the end of the
    // previous step), so the ring slot of stage s-1 can take stage s+3
    if (s + 3 < nst) issue(s + 3, NXT, CNXT);
    int half_unused, valid;
    stage_src(s, half_unused, valid);
    if constexpr (QUANT) {
      Prod::dequant(CCUR, valid, groups, rgroups, KS, tid);
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
        const float x = tok0 + i <= lim_s ? sv[i] * p.scale_log2 : NEG_INF;
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
      const float mn = fmaxf(m_s, fmaxf(red[0][row_s], red[1][row_s]));
      const float mu = mn == NEG_INF ? 0.f : mn;
      const float al = __builtin_amdgcn_exp2f(m_s - mu);
      l_s *= al;
      m_s = mn;
      if (sc_tt == 0 && lg == 0) alpha[row_s] = al;
      uint32_t pb[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        pb[i] = f32_to_bf16_bits(__builtin_amdgcn_exp2f(sv[i] - mu));
        l_s += bf16_bits_to_f32(pb[i]);
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
    wait_stage(min(nst - 2 - s, 2));
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
    for (int s = 0; s < nst; s += 4) {
      step(s, S0, C0, S0, C3);
      if (s + 1 < nst) step(s + 1, S1, C1, S0, C0);
      if (s + 2 < nst) step(s + 2, S0, C2, S0, C1);
      if (s + 3 < nst) step(s + 3, S1, C3, S0, C2);
    }
  }

  // ---- finish: row sums over lanes and token tiles, normalise, write
  if (scorer) {
    l_s = wave_sum_16_32(l_s);
    if (lg == 0) {
      redl[sc_tt][row_s] = l_s;
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
    const float lt = redl[0][tid] + redl[1][tid];
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
