// GQLA's second decode path: grouped-query attention over a per-group expanded cache (gfx950).
//
// GQLA (GQLA abstract, thelatestinai.com paper-cards page) ties the heads of each of G groups to
// one key and one value up-projection, so the same weights also decode as GQA with G key/value
// heads: the latent is expanded once per group, k_nope_g = W_UK^g c and v_g = c W_UV^g, next to
// the shared RoPE key.  The path reads more bytes per token than the absorbed one but does far
// fewer FLOPs per byte; a runtime picks the path that suits the hardware.
//
// Expanded pool, per 64-token block: G planes [64 tokens][k_nope (128) | v (128)] bf16, then one
// RoPE plane [64 tokens][k_rope (64)] bf16 shared by the groups.
//
// gqa_expand_kernel writes new tokens into that pool: workgroup = (16 tokens, group g), four
// waves; wave w computes k_nope^T and v^T for output columns 32w .. 32w+31 as W-fragment x
// latent-fragment MFMAs (the same latent register feeds both), W_UK^g rows straight from memory
// and W_UV^g through LDS with transposed reads; fp32 accumulation, one RNE rounding to bf16.
//
// gqa_decode_kernel: work unit = (sequence b, context partition c, group g); its rows are the
// group's heads for each query token (s_q * H / G <= 64).  Stages of 32 tokens [k_nope | v |
// k_rope] stream HBM -> LDS through a 3-deep ring of inline-asm DMA (two workgroups per CU);
// scores S^T = K . Q^T over 192 columns, softmax with the row maxima exchanged through LDS, P
// as two bf16 terms (hi + lo), O[rows][128] += P . V with V read transposed; partials of the
// partitions are merged by combine_kernel.
#include <hip/hip_runtime.h>

#include "mla_device.hpp"
#include "mla_internal.hpp"
#include "mla_stage.hpp"

namespace mla {
namespace gqa {

constexpr int NT = 256;                    // 4 wavefronts
constexpr int DN = 128, DV = 128, DR = 64; // key (no-RoPE), value and RoPE widths
constexpr int PLANE_ROW = DN + DV;         // elements per token in a group plane
constexpr int ROW = DN + DV + DR;          // elements per token in an LDS stage
constexpr int PIECES = ROW / 8;            // 16-byte pieces per stage row
constexpr int ST_BYTES = ST_TOK * ROW * 2;
constexpr int DEPTH = 3;                   // stage ring
constexpr int LOADS = ST_TOK * PIECES / NT;
constexpr int PROW = ST_TOK + 8;           // bf16 elements per LDS P row
constexpr int MAX_TPC = 256;
static_assert(LOADS * NT == ST_TOK * PIECES, "threads must divide the stage");

// Stage layout: logical pieces 0..15 hold k_nope, 16..31 v, 32..39 k_rope; piece p of token t
// sits at p ^ (t & 7), which stays inside p's aligned group of 8 pieces.
__device__ __forceinline__ int goff(int t, int d) { return t * ROW + ((((d >> 3) ^ (t & 7))) << 3) + (d & 7); }

__device__ __forceinline__ uint32_t lds_addr(const void* p) { return (uint32_t)(uintptr_t)(const lds_void*)p; }

// 16 bytes per lane from a per-lane address to LDS bytes [lds_base + 16 lane, + 16), invisible
// to the compiler's wait insertion (every wait for it is explicit).  lds_base is wave-uniform.
__device__ __forceinline__ void dma16(const void* src, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(lds_base), "v"(src)
               : "memory", "m0");
}

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

// ---------------------------------------------------------------------------------------
// Per-group expansion of new tokens into the pool
// ---------------------------------------------------------------------------------------
__global__ __launch_bounds__(NT) void gqa_expand_kernel(GqaExpandParams p) {
  __shared__ __attribute__((aligned(16))) bf16_t Wv[32 * (DV + 8)];   // W_UV^g rows k0 .. k0+31
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, lr = lane & 15, lg = lane >> 4;
  const int g = blockIdx.x % p.G;
  const int64_t tile = blockIdx.x / p.G;
  const int64_t i = tile * 16 + lr;                   // this lane's token (B operand column)
  const bool tok_ok = i < p.n;
  const bf16_t* c = (const bf16_t*)p.c + (tok_ok ? i : 0) * p.c_stride;
  const bf16_t* wk = (const bf16_t*)p.w_uk + (size_t)g * DN * p.d_c;   // [DN][d_c]
  const bf16_t* wv = (const bf16_t*)p.w_uv + (size_t)g * p.d_c * DV;   // [d_c][DV]
  f32x4 ak[2] = {}, av[2] = {};
  for (int k0 = 0; k0 < p.d_c; k0 += 32) {
    // W_UV^g rows k0 .. k0+31 into LDS (32 rows x 128 columns, 16 bytes per thread and pass)
    for (int q = tid; q < 32 * DV / 8; q += NT) {
      const int r = q >> 4, c8 = q & 15;
      *(u32x4*)&Wv[r * (DV + 8) + c8 * 8] = *(const u32x4*)(wv + (size_t)(k0 + r) * DV + c8 * 8);
    }
    __syncthreads();
    const bf16x8 cf = tok_ok ? *(const bf16x8*)(c + k0 + 8 * lg) : bf16x8{};
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) {
      const int col = 32 * w + 16 * ct;
      // A = W_UK^g [cols x k]: row col + lr, 8 consecutive k
      const bf16x8 a = *(const bf16x8*)(wk + (size_t)(col + lr) * p.d_c + k0 + 8 * lg);
      ak[ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, cf, ak[ct], 0, 0, 0);
      // A = W_UV^g^T [cols x k]: the transposed read of rows k0 .. k0+31
      const int t0 = lg * 8 + (lr >> 2), d = col + (lr & 3) * 4;
      const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)&Wv[t0 * (DV + 8) + d]);
      const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)&Wv[(t0 + 4) * (DV + 8) + d]);
      const bf16x8 b = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      av[ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(b, cf, av[ct], 0, 0, 0);
    }
    __syncthreads();
  }
  // D = out^T [16 columns x 16 tokens]: lane holds columns 4 lg .. 4 lg + 3 of token lr
  const int64_t slot = tok_ok ? p.slots[i] : -1;
  if (slot < 0 || slot >= p.num_blocks * BLOCK_TOKENS) return;
  uint8_t* blk = p.pool + (slot / BLOCK_TOKENS) * p.block_bytes;
  const int t = (int)(slot % BLOCK_TOKENS);
  uint16_t* row = (uint16_t*)(blk + (size_t)g * BLOCK_TOKENS * PLANE_ROW * 2) + t * PLANE_ROW;
#pragma unroll
  for (int ct = 0; ct < 2; ++ct) {
    const int col = 32 * w + 16 * ct + 4 * lg;
    *(uint2*)&row[col] = uint2{pack_bf16x2(ak[ct][0], ak[ct][1]), pack_bf16x2(ak[ct][2], ak[ct][3])};
    *(uint2*)&row[DN + col] = uint2{pack_bf16x2(av[ct][0], av[ct][1]), pack_bf16x2(av[ct][2], av[ct][3])};
  }
  if (g == 0 && w == 0) {
    // the shared RoPE key: lane lg copies 16 of the token's 64 values
    const uint16_t* kr = (const uint16_t*)p.k + i * p.k_stride + 16 * lg;
    uint16_t* dst = (uint16_t*)(blk + (size_t)p.G * BLOCK_TOKENS * PLANE_ROW * 2) + t * DR + 16 * lg;
    *(u32x4*)dst = *(const u32x4*)kr;
    *(u32x4*)(dst + 8) = *(const u32x4*)(kr + 8);
  }
}

// ---------------------------------------------------------------------------------------
// Decode
// ---------------------------------------------------------------------------------------
template <int RT>
__global__ __launch_bounds__(NT, 2) void gqa_decode_kernel(GqaParams p) {
  constexpr int ROWS = 16 * RT;
  constexpr int NRW = (RT + 1) / 2;       // row tiles a scoring wave owns
  __shared__ __attribute__((aligned(16))) uint8_t smem[DEPTH * ST_BYTES];
  __shared__ __attribute__((aligned(16))) bf16_t Ps[ROWS * PROW];   // P, high bf16 term
  __shared__ __attribute__((aligned(16))) bf16_t Pl[ROWS * PROW];   // P, low bf16 term
  __shared__ float red[2][ROWS];
  __shared__ float redx[2][ROWS];
  __shared__ float mfin[ROWS];
  __shared__ __attribute__((aligned(16))) float alpha[ROWS];
  __shared__ int bids[MAX_TPC];

  const int tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63, lr = lane & 15, lg = lane >> 4;
  const float NEG_INF = -__builtin_inff();

  const int u = (int)(blockIdx.x & 7) * p.units_per_xcd + (int)(blockIdx.x >> 3);
  if (u >= p.total_units) return;
  const int g = u % p.G;
  const int bc = u / p.G;
  const int b = bc / p.max_chunks, c = bc % p.max_chunks;
  int L = p.seq_lens[b];
  L = L < 0 ? 0 : (L > p.max_seq_len ? p.max_seq_len : L);
  const int nblk = (L + BLOCK_TOKENS - 1) / BLOCK_TOKENS;
  int nch = (nblk + p.tpc - 1) / p.tpc;
  nch = nch < 1 ? 1 : nch;
  if (c >= nch) return;
  const int T0 = c * p.tpc * BLOCK_TOKENS;
  const int T1 = min((c + 1) * p.tpc * BLOCK_TOKENS, L);
  const int nst = T1 > T0 ? (T1 - T0 + ST_TOK - 1) / ST_TOK : 0;
  const int Hg = p.H / p.G, R = p.s_q * p.H, Rg = p.s_q * Hg;
  // group row r <-> query i = r / Hg, head g Hg + r % Hg, sequence row i H + h
  auto grow = [&](int r) { return (r / Hg) * p.H + g * Hg + r % Hg; };

  // scoring: wave w takes token tile w & 1 of row tiles (w >> 1) + 2 j
  const bool scorer = RT > 1 || w < 2;
  const int tt = w & 1;
  bf16x8 qreg[NRW][6];
  int lim[NRW];
#pragma unroll
  for (int j = 0; j < NRW; ++j) {
    const int r = ((w >> 1) + 2 * j) * 16 + lr;
    const bool ok = scorer && r < Rg;
    const size_t qrow = (size_t)b * R + (ok ? grow(r) : 0);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      qreg[j][ks] = ok ? *(const bf16x8*)((const bf16_t*)p.q_nope + qrow * DN + 32 * ks + 8 * lg) : bf16x8{};
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
      qreg[j][4 + ks] = ok ? *(const bf16x8*)((const bf16_t*)p.q_rope + qrow * DR + 32 * ks + 8 * lg) : bf16x8{};
    lim[j] = ok ? L - p.s_q + r / Hg : -1;
  }
  float m_s[NRW], l_x[NRW];
#pragma unroll
  for (int j = 0; j < NRW; ++j) {
    m_s[j] = NEG_INF;
    l_x[j] = 0.f;
  }
  f32x4 acc[RT][2];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) acc[rt][0] = acc[rt][1] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int32_t* btab = p.block_table + (size_t)b * p.bt_stride;
  const int blk0 = T0 / BLOCK_TOKENS;
  const int nb_unit = min(p.tpc, nblk - blk0);
  for (int j = tid; j < nb_unit; j += NT) bids[j] = btab[blk0 + j];
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));   // queries and block ids, before any DMA
  __syncthreads();

  // per-lane DMA offsets: slot k = i NT + tid of a stage holds token k / 40, physical piece k % 40
  uint32_t off[LOADS];
  bool rope[LOADS];
#pragma unroll
  for (int i = 0; i < LOADS; ++i) {
    const int k = i * NT + tid, t = k / PIECES, pl = (k % PIECES) ^ (t & 7);
    rope[i] = pl >= 32;
    off[i] = rope[i] ? (uint32_t)(t * DR * 2 + (pl - 32) * 16) : (uint32_t)(t * PLANE_ROW * 2 + pl * 16);
  }
  const size_t plane_off = (size_t)g * BLOCK_TOKENS * PLANE_ROW * 2;
  const size_t rope_off = (size_t)p.G * BLOCK_TOKENS * PLANE_ROW * 2;
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
  const uint32_t sbase = lds_addr(smem);
  const uint32_t wslice = (uint32_t)__builtin_amdgcn_readfirstlane((tid & ~63) * 16);
  auto issue = [&](int s) {
    int half, valid;
    const uint8_t* blk = stage_src(s, half, valid);
    const uint8_t* pb = blk + plane_off + (size_t)half * ST_TOK * PLANE_ROW * 2;
    const uint8_t* rb = blk + rope_off + (size_t)half * ST_TOK * DR * 2;
    const uint32_t dst = sbase + (uint32_t)((s % DEPTH) * ST_BYTES) + wslice;
#pragma unroll
    for (int i = 0; i < LOADS; ++i) dma16((rope[i] ? rb : pb) + off[i], dst + (uint32_t)(i * NT * 16));
  };
  auto wait_stage = [&](int later) {
    if (later <= 0) __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    else if (later == 1) __builtin_amdgcn_s_waitcnt(vmcnt_imm(LOADS));
    else __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * LOADS));
  };

  for (int s = 0; s < DEPTH - 1 && s < nst; ++s) issue(s);
  wait_stage(min(nst - 1, DEPTH - 2));
  lds_barrier();

  for (int s = 0; s < nst; ++s) {
    // stage s landed and every wave is done with stage s - 1: its slot takes stage s + 2
    if (s + DEPTH - 1 < nst) issue(s + DEPTH - 1);
    bf16_t* KS = (bf16_t*)(smem + (s % DEPTH) * ST_BYTES);
    int half_unused, valid;
    stage_src(s, half_unused, valid);
    if (valid < ST_TOK) {
      // rows past the sequence end (or of an id outside the pool) hold whatever the block held
      for (int q = tid; q < (ST_TOK - valid) * PIECES; q += NT)
        *(u32x4*)&KS[(valid + q / PIECES) * ROW + (q % PIECES) * 8] = u32x4{0, 0, 0, 0};
      lds_barrier();
    }
    // ---- scores of token tile tt for this wave's row tiles
    f32x4 sv[NRW];
    if (scorer) {
      const int t = tt * 16 + lr;
      const int f = t & 7;
#pragma unroll
      for (int j = 0; j < NRW; ++j) sv[j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 6; ++ks) {
        const int lp = ks < 4 ? 4 * ks + lg : 32 + 4 * (ks - 4) + lg;
        const bf16x8 a = *(const bf16x8*)&KS[t * ROW + ((lp ^ f) << 3)];
#pragma unroll
        for (int j = 0; j < NRW; ++j) sv[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qreg[j][ks], sv[j], 0, 0, 0);
      }
      const int tok0 = T0 + s * ST_TOK + tt * 16 + 4 * lg;
#pragma unroll
      for (int j = 0; j < NRW; ++j) {
        float mx = NEG_INF;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const bool ok = tt * 16 + 4 * lg + i < valid && tok0 + i <= lim[j];
          sv[j][i] = ok ? sv[j][i] * p.scale_log2 : NEG_INF;
          mx = fmaxf(mx, sv[j][i]);
        }
        mx = max_lg(mx);
        const int rt = (w >> 1) + 2 * j;
        if (lg == 0 && rt < RT) red[tt][rt * 16 + lr] = mx;
      }
    }
    lds_barrier();
    // ---- softmax: running maximum (moved only past RESCALE_SLACK), P as hi + lo bf16 terms
    if (scorer) {
#pragma unroll
      for (int j = 0; j < NRW; ++j) {
        const int rt = (w >> 1) + 2 * j;
        if (rt >= RT) continue;
        const int row = rt * 16 + lr;
        const float mt = fmaxf(red[0][row], red[1][row]);
        const float mn = mt > m_s[j] + RESCALE_SLACK ? mt : m_s[j];
        const float mu = mn == NEG_INF ? 0.f : mn;
        const float al = mn == m_s[j] ? 1.f : __builtin_amdgcn_exp2f(m_s[j] - mu);
        l_x[j] *= al;
        m_s[j] = mn;
        if (tt == 0 && lg == 0) alpha[row] = al;
        float pf[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          pf[i] = __builtin_amdgcn_exp2f(sv[j][i] - mu);
          l_x[j] += pf[i];
        }
        uint32_t h0, l0, h1, l1;
        split_pair(pf[0], pf[1], h0, l0);
        split_pair(pf[2], pf[3], h1, l1);
        *(uint2*)&Ps[row * PROW + tt * 16 + 4 * lg] = uint2{h0, h1};
        *(uint2*)&Pl[row * PROW + tt * 16 + 4 * lg] = uint2{l0, l1};
      }
    }
    lds_barrier();
    // ---- O[rows][32 w .. 32 w + 31] = alpha O + (P_hi + P_lo) . V
    {
      bool any = false;
      f32x4 al[RT];
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        al[rt] = *(const f32x4*)&alpha[rt * 16 + 4 * lg];
        any |= (al[rt][0] != 1.f) | (al[rt][1] != 1.f) | (al[rt][2] != 1.f) | (al[rt][3] != 1.f);
      }
      if (__any(any)) {
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
          acc[rt][0] *= al[rt];
          acc[rt][1] *= al[rt];
        }
      }
      bf16x8 ph[RT], pl[RT];
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        ph[rt] = *(const bf16x8*)&Ps[(rt * 16 + lr) * PROW + 8 * lg];
        pl[rt] = *(const bf16x8*)&Pl[(rt * 16 + lr) * PROW + 8 * lg];
      }
      const int t0 = lg * 8 + (lr >> 2);
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) {
        const int d = DN + 32 * w + 16 * ct + (lr & 3) * 4;
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)&KS[goff(t0, d)]);
        const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)&KS[goff(t0 + 4, d)]);
        const bf16x8 bv = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) acc[rt][ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ph[rt], bv, acc[rt][ct], 0, 0, 0);
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) acc[rt][ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pl[rt], bv, acc[rt][ct], 0, 0, 0);
      }
    }
    // the next stage landed and nobody reads stage s any more
    if (s + 1 < nst) wait_stage(min(nst - 1, s + DEPTH - 1) - (s + 1));
    lds_barrier();
  }

  // ---- finish: row sums over lanes and token tiles, normalise, write
  if (scorer) {
#pragma unroll
    for (int j = 0; j < NRW; ++j) {
      const int rt = (w >> 1) + 2 * j;
      const float lx = sum_lg(l_x[j]);
      if (lg == 0 && rt < RT) {
        redx[tt][rt * 16 + lr] = lx;
        if (tt == 0) mfin[rt * 16 + lr] = m_s[j];
      }
    }
  }
  lds_barrier();
  const size_t unit_row0 = ((size_t)b * p.max_chunks + c) * R;
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = rt * 16 + 4 * lg + i;
      if (r >= Rg) continue;
      const float lt = redx[0][r] + redx[1][r];
      const float inv = lt > 0.f ? 1.f / lt : 0.f;
      float* o = p.out + (unit_row0 + grow(r)) * DV + 32 * w + lr;
      o[0] = acc[rt][0][i] * inv;
      o[16] = acc[rt][1][i] * inv;
    }
  }
  if (p.out_lse != nullptr && tid < Rg) {
    const float lt = redx[0][tid] + redx[1][tid];
    p.out_lse[unit_row0 + grow(tid)] = lt > 0.f ? (mfin[tid] + __log2f(lt)) * 0.69314718055994531f : NEG_INF;
  }
}

}  // namespace gqa

hipError_t launch_gqa_expand(const GqaExpandParams& p, hipStream_t st) {
  if (p.n <= 0) return hipSuccess;
  const int64_t grid = (p.n + 15) / 16 * p.G;
  hipLaunchKernelGGL(gqa::gqa_expand_kernel, dim3((unsigned)grid), dim3(gqa::NT), 0, st, p);
  return hipGetLastError();
}

hipError_t launch_gqa_decode(const GqaParams& p, int rt, hipStream_t st) {
  const int grid = 8 * p.units_per_xcd;
  switch (rt) {
    case 1: hipLaunchKernelGGL(gqa::gqa_decode_kernel<1>, dim3(grid), dim3(gqa::NT), 0, st, p); break;
    case 2: hipLaunchKernelGGL(gqa::gqa_decode_kernel<2>, dim3(grid), dim3(gqa::NT), 0, st, p); break;
    case 4: hipLaunchKernelGGL(gqa::gqa_decode_kernel<4>, dim3(grid), dim3(gqa::NT), 0, st, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace mla
