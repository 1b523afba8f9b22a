// MLA decode over a paged latent cache: the absorbed-MQA attention step.
//
// Every head scores the same cached rows [c (512) | k_rope (64)] (GQLA
// abstract: absorbed MQA decoding path), the softmax-weighted sum is taken
// over the latent itself (RAQ-MLA abstract: the latent supplies the values),
// and INT4/INT2 caches are unpacked and dequantised inside this loop
// (QuantMLA English abstract: native low-bit kernel).
//
// Work unit = (sequence b, context partition c, row group rg).  A row is one
// (query token i, head h) pair; a workgroup owns 16*RT rows.  Per 64-token
// block the workgroup (4 wavefronts):
//   1. writes the block, dequantised to bf16, into LDS from registers that
//      were loaded while the previous block was being processed;
//   2. scores: S^T = K . Q^T with v_mfma_f32_16x16x32_bf16 (K from LDS, Q^T
//      held in registers for the whole partition); wave w scores one row tile
//      and 4/RT... token tiles so every row's 64 scores are covered once;
//   3. online softmax in the log2 domain: per-row tile maxima are exchanged
//      through LDS, P = exp2(x - m) goes to LDS in bf16;
//   4. O += P . C with the same MFMA: wave w owns latent columns
//      [128w, 128w + 128) for all rows; C^T operands come straight from the
//      token-major tile with ds_read_b64_tr_b16.
// Partial (o, lse) per partition are merged by combine_kernel (log-sum-exp).
#include <hip/hip_runtime.h>

#include "mla_device.hpp"
#include "mla_internal.hpp"

namespace mla {

constexpr int KROW = 576 + 8;  // bf16 elements per LDS key row (1168 bytes)
constexpr int PROW = 64 + 8;   // bf16 elements per LDS P row

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
  if (!f32) {
    u32x4 v = *(const u32x4*)((const bf16_t*)base + elem_off);
    return __builtin_bit_cast(bf16x8, v);
  }
  const float* f = (const float*)base + elem_off;
  f32x4 a = *(const f32x4*)f;
  f32x4 b = *(const f32x4*)(f + 4);
  u32x4 r;
  r[0] = pack_bf16x2(a[0], a[1]);
  r[1] = pack_bf16x2(a[2], a[3]);
  r[2] = pack_bf16x2(b[0], b[1]);
  r[3] = pack_bf16x2(b[2], b[3]);
  return __builtin_bit_cast(bf16x8, r);
}

typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

__device__ __forceinline__ i16x4 lds_tr16(const bf16_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p));
}

template <int RT, int FMT, bool QF32>
__global__ __launch_bounds__(256) void decode_mfma_kernel(DecodeParams p) {
  constexpr int NT = 256;
  constexpr int ROWS = 16 * RT;
  constexpr int SLOTS = 4 / RT;
  __shared__ __attribute__((aligned(16))) bf16_t Ks[BLOCK_TOKENS * KROW];
  __shared__ __attribute__((aligned(16))) bf16_t Ps[ROWS * PROW];
  __shared__ float red[4][ROWS];
  __shared__ float redl[4][ROWS];
  __shared__ float mfin[ROWS];

  const int tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63, lr = lane & 15, lg = lane >> 4;

  // unit of work: consecutive units sit on one XCD (workgroups are dealt round-robin to the 8 XCDs)
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
  const int t_begin = c * p.tpc;
  const int t_end = min(t_begin + p.tpc, nblk);
  const int R = p.R;
  const int r0 = rg * ROWS;

  // score role of this wave: one row tile, RT token tiles of each 64-token block
  const int sc_rt = w / SLOTS, sc_ts = w % SLOTS;
  const int row_s = sc_rt * 16 + lr;          // row within the group scored by this lane
  const int qrow = r0 + row_s;
  const bool qvalid = qrow < R;
  const int lim_s = qvalid ? L - p.s_q + qrow / p.H : -1;  // last attended token

  bf16x8 qreg[18];
  {
    const size_t qbase = ((size_t)b * R + (qvalid ? qrow : 0));
#pragma unroll
    for (int ks = 0; ks < 16; ++ks) {
      qreg[ks] = qvalid ? load_q8(p.q_lat, qbase * 512 + ks * 32 + lg * 8, QF32) : bf16x8{};
    }
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      qreg[16 + ks] = qvalid ? load_q8(p.q_rope, qbase * 64 + ks * 32 + lg * 8, QF32) : bf16x8{};
    }
  }

  const float NEG_INF = -__builtin_inff();
  float m_s = NEG_INF, l_s = 0.f;
  float m_p[RT][4];
  f32x4 acc[RT][8];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
#pragma unroll
    for (int i = 0; i < 4; ++i) m_p[rt][i] = NEG_INF;
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) acc[rt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  const QuantPlanes pl{(int)p.off_lc, (int)p.off_ls, (int)p.off_rc, (int)p.off_rs};
  const int32_t* btab = p.block_table + (size_t)b * p.bt_stride;
  auto tile_src = [&](int t, int& valid) -> const uint8_t* {
    int id = btab[t];
    valid = min(BLOCK_TOKENS, L - t * BLOCK_TOKENS);
    if (id < 0 || (int64_t)id >= p.num_blocks) {
      valid = 0;
      id = 0;
    }
    return p.pool + (size_t)id * (size_t)p.block_bytes;
  };

  TileReader<FMT, NT> rd;
  int valid_next = 0;
  if (t_begin < t_end) {
    const uint8_t* src = tile_src(t_begin, valid_next);
    rd.load(src, valid_next, tid, pl, p.g_lat, p.g_rope);
  }

  for (int t = t_begin; t < t_end; ++t) {
    const int valid = valid_next;
    __syncthreads();  // every wave is done reading the previous block from LDS
    rd.emit([&](int tok, int col8, u32x4 v) { *(u32x4*)&Ks[tok * KROW + col8 * 8] = v; }, valid, tid);
    if (t + 1 < t_end) {
      const uint8_t* src = tile_src(t + 1, valid_next);
      rd.load(src, valid_next, tid, pl, p.g_lat, p.g_rope);
    }
    __syncthreads();

    // ---- scores S^T[token][row] for this wave's row tile and token tiles
    f32x4 s[RT];
#pragma unroll
    for (int j = 0; j < RT; ++j) {
      const int tt = sc_ts * RT + j;
      const bf16_t* krow = &Ks[(tt * 16 + lr) * KROW + lg * 8];
      f32x4 a0 = {0.f, 0.f, 0.f, 0.f}, a1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 18; ks += 2) {
        bf16x8 k0 = *(const bf16x8*)(krow + ks * 32);
        bf16x8 k1 = *(const bf16x8*)(krow + ks * 32 + 32);
        a0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k0, qreg[ks], a0, 0, 0, 0);
        a1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k1, qreg[ks + 1], a1, 0, 0, 0);
      }
      s[j] = a0 + a1;
    }
    float mx = NEG_INF;
    const int tok0 = t * BLOCK_TOKENS + lg * 4;
#pragma unroll
    for (int j = 0; j < RT; ++j) {
      const int tt = sc_ts * RT + j;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int tok = tok0 + tt * 16 + i;
        float x = tok <= lim_s ? s[j][i] * p.scale_log2 : NEG_INF;
        s[j][i] = x;
        mx = fmaxf(mx, x);
      }
    }
    mx = wave_max_16_32(mx);
    if (lg == 0) red[sc_ts][row_s] = mx;
    __syncthreads();

    // ---- new running max; P for the scored tokens
    {
      float tm = red[0][row_s];
#pragma unroll
      for (int sl = 1; sl < SLOTS; ++sl) tm = fmaxf(tm, red[sl][row_s]);
      const float mn = fmaxf(m_s, tm);
      const float mu = mn == NEG_INF ? 0.f : mn;
      l_s *= exp2f(m_s - mu);
      m_s = mn;
#pragma unroll
      for (int j = 0; j < RT; ++j) {
        const int tt = sc_ts * RT + j;
        uint32_t pb[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          pb[i] = f32_to_bf16_bits(exp2f(s[j][i] - mu));
          l_s += bf16_bits_to_f32(pb[i]);
        }
        uint2 pk = {pb[0] | (pb[1] << 16), pb[2] | (pb[3] << 16)};
        *(uint2*)&Ps[row_s * PROW + tt * 16 + lg * 4] = pk;
      }
    }
    // rescale the output rows this wave accumulates
    {
      bool any = false;
      float al[RT][4];
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int row = rt * 16 + lg * 4 + i;
          float tm = red[0][row];
#pragma unroll
          for (int sl = 1; sl < SLOTS; ++sl) tm = fmaxf(tm, red[sl][row]);
          const float mn = fmaxf(m_p[rt][i], tm);
          const float mu = mn == NEG_INF ? 0.f : mn;
          al[rt][i] = exp2f(m_p[rt][i] - mu);
          any |= al[rt][i] != 1.f;
          m_p[rt][i] = mn;
        }
      }
      if (__any(any)) {
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
          for (int nt = 0; nt < 8; ++nt)
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[rt][nt][i] *= al[rt][i];
      }
    }
    __syncthreads();

    // ---- O[rows][128w .. 128w+127] += P . C
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      bf16x8 a[RT];
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) a[rt] = *(const bf16x8*)&Ps[(rt * 16 + lr) * PROW + kk * 32 + lg * 8];
      const bf16_t* cb = &Ks[(kk * 32 + lg * 8 + (lr >> 2)) * KROW + w * 128 + (lr & 3) * 4];
#pragma unroll
      for (int nt = 0; nt < 8; ++nt) {
        i16x4 lo = lds_tr16(cb + nt * 16);
        i16x4 hi = lds_tr16(cb + 4 * KROW + nt * 16);
        bf16x8 bv = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
          acc[rt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[rt], bv, acc[rt][nt], 0, 0, 0);
      }
    }
  }

  // ---- finish: row sums over lanes and token slots, normalise, write
  l_s = wave_sum_16_32(l_s);
  __syncthreads();
  if (lg == 0) {
    redl[sc_ts][row_s] = l_s;
    if (sc_ts == 0) mfin[row_s] = m_s;
  }
  __syncthreads();
  const size_t unit_row0 = ((size_t)b * p.max_chunks + c) * R;
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = rt * 16 + lg * 4 + i;
      const int rgl = r0 + row;
      if (rgl >= R) continue;
      float lt = redl[0][row];
#pragma unroll
      for (int sl = 1; sl < SLOTS; ++sl) lt += redl[sl][row];
      const float inv = lt > 0.f ? 1.f / lt : 0.f;
      const size_t obase = (unit_row0 + rgl) * 512 + w * 128 + lr;
      if (p.out_bf16) {
        bf16_t* o = (bf16_t*)p.out;
#pragma unroll
        for (int nt = 0; nt < 8; ++nt)
          o[obase + nt * 16] = __builtin_bit_cast(bf16_t, (uint16_t)f32_to_bf16_bits(acc[rt][nt][i] * inv));
      } else {
        float* o = (float*)p.out;
#pragma unroll
        for (int nt = 0; nt < 8; ++nt) o[obase + nt * 16] = acc[rt][nt][i] * inv;
      }
    }
  }
  if (p.out_lse != nullptr && tid < ROWS && r0 + tid < R) {
    float lt = redl[0][tid];
#pragma unroll
    for (int sl = 1; sl < SLOTS; ++sl) lt += redl[sl][tid];
    const float m = mfin[tid];
    p.out_lse[unit_row0 + r0 + tid] = lt > 0.f ? (m + __log2f(lt)) * 0.69314718055994531f : NEG_INF;
  }
}

// ---------------------------------------------------------------------------------------
// fp32 cache path: plain fp32 arithmetic, one workgroup (128 threads) per (b, partition, row).
// Any d_c <= 1024, d_r <= 256.  Same partial layout as the MFMA kernel.
// ---------------------------------------------------------------------------------------
__global__ __launch_bounds__(128) void decode_f32_kernel(DecodeParams p) {
  constexpr int NT = 128;
  __shared__ float qs[1024 + 256];
  __shared__ float sc[16];
  const int tid = threadIdx.x;
  const int u = blockIdx.x;
  if (u >= p.total_units) return;
  const int R = p.R;
  const int r = u % R;
  const int bc = u / R;
  const int b = bc / p.max_chunks, c = bc % p.max_chunks;
  int L = p.seq_lens[b];
  L = L < 0 ? 0 : (L > p.max_seq_len ? p.max_seq_len : L);
  const int nblk = (L + BLOCK_TOKENS - 1) / BLOCK_TOKENS;
  int nch = (nblk + p.tpc - 1) / p.tpc;
  nch = nch < 1 ? 1 : nch;
  if (c >= nch) return;
  const int d_c = p.d_c, d_r = p.d_r, dk = d_c + d_r;
  const int lim = L - p.s_q + r / p.H;
  const int tok_begin = c * p.tpc * BLOCK_TOKENS;
  const int tok_end = min(min((c + 1) * p.tpc * BLOCK_TOKENS, L), lim + 1);
  const float* ql = (const float*)p.q_lat + ((size_t)b * R + r) * d_c;
  const float* qr = (const float*)p.q_rope + ((size_t)b * R + r) * d_r;
  for (int d = tid; d < d_c; d += NT) qs[d] = ql[d];
  for (int d = tid; d < d_r; d += NT) qs[d_c + d] = qr[d];
  __syncthreads();
  const int32_t* btab = p.block_table + (size_t)b * p.bt_stride;
  float o[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) o[k] = 0.f;
  float m = -__builtin_inff(), l = 0.f;
  const float scale = p.scale_log2 * 0.69314718055994531f;  // natural-log scale
  for (int t0 = tok_begin; t0 < tok_end; t0 += 16) {
    const int tok = t0 + (tid >> 3), sub = tid & 7;
    float part = 0.f;
    if (tok < tok_end) {
      int id = btab[tok / BLOCK_TOKENS];
      if (id >= 0 && (int64_t)id < p.num_blocks) {
        const float* row = (const float*)(p.pool + (size_t)id * p.block_bytes) + (size_t)(tok % BLOCK_TOKENS) * dk;
        for (int d = sub; d < dk; d += 8) part += qs[d] * row[d];
      }
    }
    part += __shfl_xor(part, 1, 8);
    part += __shfl_xor(part, 2, 8);
    part += __shfl_xor(part, 4, 8);
    if (sub == 0) sc[tid >> 3] = tok < tok_end ? part * scale : -__builtin_inff();
    __syncthreads();
    float tm = sc[0];
    for (int j = 1; j < 16; ++j) tm = fmaxf(tm, sc[j]);
    const float mn = fmaxf(m, tm);
    const float alpha = expf(m - mn);
    l *= alpha;
#pragma unroll
    for (int k = 0; k < 8; ++k) o[k] *= alpha;
    m = mn;
    for (int j = 0; j < 16 && t0 + j < tok_end; ++j) {
      const float pj = expf(sc[j] - mn);
      l += pj;
      const int tk = t0 + j;
      int id = btab[tk / BLOCK_TOKENS];
      if (id < 0 || (int64_t)id >= p.num_blocks) continue;
      const float* row = (const float*)(p.pool + (size_t)id * p.block_bytes) + (size_t)(tk % BLOCK_TOKENS) * dk;
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int d = tid + k * NT;
        if (d < d_c) o[k] += pj * row[d];
      }
    }
    __syncthreads();
  }
  const size_t unit_row = ((size_t)b * p.max_chunks + c) * R + r;
  const float inv = l > 0.f ? 1.f / l : 0.f;
  for (int k = 0; k < 8; ++k) {
    const int d = tid + k * NT;
    if (d >= d_c) break;
    if (p.out_bf16)
      ((bf16_t*)p.out)[unit_row * d_c + d] = __builtin_bit_cast(bf16_t, (uint16_t)f32_to_bf16_bits(o[k] * inv));
    else
      ((float*)p.out)[unit_row * d_c + d] = o[k] * inv;
  }
  if (p.out_lse != nullptr && tid == 0) p.out_lse[unit_row] = l > 0.f ? m + logf(l) : -__builtin_inff();
}

// ---------------------------------------------------------------------------------------
// Combine: o = sum_c exp(lse_c - lse) o_c, lse = log sum_c exp(lse_c), over the partitions
// a sequence was split into.  One workgroup of 128 threads per (b, row); 4 columns/thread
// for d_c = 512 (generic d_c handled by striding).
// ---------------------------------------------------------------------------------------
__global__ __launch_bounds__(128) void combine_kernel(CombineParams p) {
  const int idx = blockIdx.x;
  const int R = p.R;
  const int b = idx / R, r = idx % R;
  int L = p.seq_lens[b];
  L = L < 0 ? 0 : (L > p.max_seq_len ? p.max_seq_len : L);
  const int nblk = (L + BLOCK_TOKENS - 1) / BLOCK_TOKENS;
  int nch = (nblk + p.tpc - 1) / p.tpc;
  nch = nch < 1 ? 1 : (nch > p.max_chunks ? p.max_chunks : nch);
  const size_t u0 = (size_t)b * p.max_chunks;
  float m = -__builtin_inff();
  for (int c = 0; c < nch; ++c) m = fmaxf(m, p.part_lse[(u0 + c) * R + r]);
  float wsum = 0.f;
  for (int c = 0; c < nch; ++c) {
    const float lc = p.part_lse[(u0 + c) * R + r];
    wsum += (m == -__builtin_inff()) ? 0.f : expf(lc - m);
  }
  const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
  const int d_c = p.d_c;
  for (int d = threadIdx.x * 4; d < d_c; d += 128 * 4) {
    f32x4 accv = {0.f, 0.f, 0.f, 0.f};
    for (int c = 0; c < nch; ++c) {
      const float lc = p.part_lse[(u0 + c) * R + r];
      const float wc = (m == -__builtin_inff()) ? 0.f : expf(lc - m);
      const f32x4 v = *(const f32x4*)(p.part_o + ((u0 + c) * R + r) * (size_t)d_c + d);
      accv += wc * v;
    }
    accv *= inv;
    const size_t ob = ((size_t)b * R + r) * d_c + d;
    if (p.out_bf16) {
      uint2 pk = {pack_bf16x2(accv[0], accv[1]), pack_bf16x2(accv[2], accv[3])};
      *(uint2*)((bf16_t*)p.out + ob) = pk;
    } else {
      *(f32x4*)((float*)p.out + ob) = accv;
    }
  }
  if (p.out_lse != nullptr && threadIdx.x == 0)
    p.out_lse[(size_t)b * R + r] = wsum > 0.f ? m + logf(wsum) : -__builtin_inff();
}

// ---------------------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------------------
template <int RT, int FMT>
static hipError_t launch_mfma(const DecodeParams& p, int grid, hipStream_t st) {
  if (p.q_f32)
    hipLaunchKernelGGL((decode_mfma_kernel<RT, FMT, true>), dim3(grid), dim3(256), 0, st, p);
  else
    hipLaunchKernelGGL((decode_mfma_kernel<RT, FMT, false>), dim3(grid), dim3(256), 0, st, p);
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

hipError_t launch_decode_f32(const DecodeParams& p, hipStream_t st) {
  hipLaunchKernelGGL(decode_f32_kernel, dim3(p.total_units), dim3(128), 0, st, p);
  return hipGetLastError();
}

hipError_t launch_combine(const CombineParams& p, int batch, hipStream_t st) {
  hipLaunchKernelGGL(combine_kernel, dim3(batch * p.R), dim3(128), 0, st, p);
  return hipGetLastError();
}

}  // namespace mla
