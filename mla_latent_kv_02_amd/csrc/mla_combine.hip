// The fp32-cache decode kernel and the log-sum-exp combine of split partitions.
#include <hip/hip_runtime.h>

#include "mla_device.hpp"
#include "mla_internal.hpp"

namespace mla {

// ---------------------------------------------------------------------------------------
// fp32 cache path: plain fp32 arithmetic, one workgroup (128 threads) per (b, partition, row).
// Any d_c <= 1024, d_r <= 256.  Writes the same partial layout as the MFMA kernel.
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
    bool live = false;   // a token past the range, or of a block-table entry outside the pool, is not attended
    if (tok < tok_end) {
      const int id = btab[tok / BLOCK_TOKENS];
      if (id >= 0 && (int64_t)id < p.num_blocks) {
        live = true;
        const float* row = (const float*)(p.pool + (size_t)id * p.block_bytes) + (size_t)(tok % BLOCK_TOKENS) * dk;
        for (int d = sub; d < dk; d += 8) part += qs[d] * row[d];
      }
    }
    part += __shfl_xor(part, 1, 8);
    part += __shfl_xor(part, 2, 8);
    part += __shfl_xor(part, 4, 8);
    if (sub == 0) sc[tid >> 3] = live ? part * scale : -__builtin_inff();
    __syncthreads();
    float tm = sc[0];
    for (int j = 1; j < 16; ++j) tm = fmaxf(tm, sc[j]);
    const float mn = fmaxf(m, tm);
    // while nothing has been attended (mn = -inf) there is nothing to rescale
    const float alpha = mn == -__builtin_inff() ? 1.f : expf(m - mn);
    l *= alpha;
#pragma unroll
    for (int k = 0; k < 8; ++k) o[k] *= alpha;
    m = mn;
    for (int j = 0; j < 16 && t0 + j < tok_end; ++j) {
      if (sc[j] == -__builtin_inff()) continue;
      const float pj = expf(sc[j] - mn);
      l += pj;
      const int tk = t0 + j;
      const int id = btab[tk / BLOCK_TOKENS];
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
// Combine: lse = log sum_c exp(lse_c), o = sum_c exp(lse_c - lse) o_c over the partials of one
// (b, row), o_c = part_o_c (partition mode) or part_o_c * part_inv_c (range mode).  One
// workgroup of 128 threads per (b, row), each thread owning 4 columns (of every 512).  The
// partials are taken in batches of CB (8, or 32 when rows usually hold more than 16
// partials): all loads of a batch (lse, 1/sum and the thread's columns) are issued together,
// so a (b, row) with at most CB partials costs one memory round trip; batches merge with a
// running maximum.  Weights use the hardware exp2 (relative error
// ~1e-7 for the lse differences that occur, far inside the fp32 tolerance).
// ---------------------------------------------------------------------------------------
template <int CB>
__global__ __launch_bounds__(128) void combine_kernel(CombineParams p) {
  constexpr float LOG2E = 1.4426950408889634f;
  const int tid = threadIdx.x;
  const int R = p.R;
  const int b = blockIdx.x / R, r = blockIdx.x % R;
  const float NEG_INF = -__builtin_inff();
  int nch;
  size_t base, step = (size_t)R;   // partial c of this (b, row) is row base + c * step
  if (p.chunk_major) {
    // parts of one decode over several caches: every (b, row) has max_chunks partials,
    // partial c at row (c * B + b) * R + r
    nch = p.max_chunks;
    base = (size_t)b * R + r;
    step = (size_t)p.B * R;
  } else if (p.meta == nullptr) {
    int L = p.seq_lens[b];
    L = L < 0 ? 0 : (L > p.max_seq_len ? p.max_seq_len : L);
    int nblk = (L + BLOCK_TOKENS - 1) / BLOCK_TOKENS;
    if (p.mixed) {
      // a mixed history: weighted positions of its three parts
      int nk[2];
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        int Lk = p.hi_lens[k] != nullptr ? p.hi_lens[k][b] : 0;
        Lk = Lk < 0 ? 0 : (Lk > p.hi_max[k] ? p.hi_max[k] : Lk);
        nk[k] = (Lk + BLOCK_TOKENS - 1) / BLOCK_TOKENS;
      }
      nblk = mixed_positions(nk[0], nblk, nk[1]);
    }
    nch = (nblk + p.tpc - 1) / p.tpc;
    nch = nch < 1 ? 1 : (nch > p.max_chunks ? p.max_chunks : nch);
    base = (size_t)b * p.max_chunks * R + r;
  } else {
    // sequence b's blocks are the last n_b positions of its part of the block space, which
    // holds G more (the charge of its start) when it is not empty
    const int span = p.meta[2 + b] - p.meta[1 + b];
    const int nblk = span > 0 ? span - p.meta[p.B + 2] : 0;
    if (nblk <= 0) return;  // empty sequence: written by the decode kernel
    const int per = p.meta[0], last = p.meta[2 + b] - 1;
    const int i0 = (last - nblk + 1) / per, i1 = last / per;
    nch = i1 - i0 + 1;
    base = ((size_t)b + i0) * R + r;
  }
  const int d_c = p.d_c;
  const size_t stride = step * d_c;               // between consecutive partials
  const bool vec4 = (d_c & 3) == 0;               // 16-byte column groups (else element by element)
  float lse_out = NEG_INF;
  for (int d = tid * 4; d < d_c; d += 512) {
    float m = NEG_INF, wsum = 0.f;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int c0 = 0; c0 < nch; c0 += CB) {
      const int n = min(CB, nch - c0);
      const size_t ub = base + (size_t)c0 * step;
      float lc[CB], iv[CB];
      f32x4 v[CB];
#pragma unroll
      for (int j = 0; j < CB; ++j) {
        const bool ok = j < n;
        lc[j] = ok ? p.part_lse[ub + (size_t)j * step] : NEG_INF;
        iv[j] = ok && p.part_inv != nullptr ? p.part_inv[ub + (size_t)j * step] : 1.f;
        v[j] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (ok) {
          const float* src = p.part_o + ub * d_c + d + j * stride;
          if (vec4) {
            v[j] = *(const f32x4*)src;
          } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) v[j][i] = d + i < d_c ? src[i] : 0.f;
          }
        }
      }
      float mb = NEG_INF;
#pragma unroll
      for (int j = 0; j < CB; ++j) mb = fmaxf(mb, lc[j]);
      if (mb > m) {
        // every earlier weight is relative to m; m = -inf means nothing was added yet
        const float sc = m == NEG_INF ? 0.f : __builtin_amdgcn_exp2f((m - mb) * LOG2E);
        acc *= sc;
        wsum *= sc;
        m = mb;
      }
#pragma unroll
      for (int j = 0; j < CB; ++j) {
        const float wc = lc[j] == NEG_INF ? 0.f : __builtin_amdgcn_exp2f((lc[j] - m) * LOG2E);
        wsum += wc;
        acc += (wc * iv[j]) * v[j];
      }
    }
    const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
    const f32x4 o = acc * inv;
    const size_t ob = ((size_t)b * R + r) * d_c + d;
    if (!vec4) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (d + i >= d_c) break;
        if (p.out_bf16)
          ((uint16_t*)p.out)[ob + i] = (uint16_t)f32_to_bf16_bits(o[i]);
        else
          ((float*)p.out)[ob + i] = o[i];
      }
    } else if (p.out_bf16) {
      *(uint2*)((bf16_t*)p.out + ob) = uint2{pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3])};
    } else {
      *(f32x4*)((float*)p.out + ob) = o;
    }
    lse_out = wsum > 0.f ? m + logf(wsum) : NEG_INF;
  }
  if (p.out_lse != nullptr && tid == 0) p.out_lse[(size_t)b * R + r] = lse_out;
}

// ---------------------------------------------------------------------------------------
// Range mode over a 512-wide latent (the row-owner decode's pieces): the same merge as
// combine_kernel, each lane owning 8 columns of a (b, row).  WPR = 1: one wavefront per
// (b, row), four per workgroup, for rows with a few pieces; WPR = 4: the four wavefronts of a
// workgroup share the pieces of one (b, row) (wavefront w takes pieces w, w + 4, ...) and
// merge their running (max, sum, o) through LDS, for rows with many pieces.  Everything that
// depends only on (b, row) (the block-space positions, the pieces' lse and 1/sum(P)) is
// wave-uniform and read through the scalar cache, and all loads of a batch of CB pieces are
// issued together.
// ---------------------------------------------------------------------------------------
template <int WPR, int CB>
__global__ __launch_bounds__(256) void combine_rows_kernel(CombineParams p) {
  constexpr float LOG2E = 1.4426950408889634f;
  const float NEG_INF = -__builtin_inff();
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  const int R = p.R, B = p.B;
  const int idx = WPR == 1 ? (int)blockIdx.x * 4 + w : (int)blockIdx.x;   // b * R + row
  if (idx >= B * R) return;
  const int b = idx / R, r = idx - b * R;
  const int32_t* meta = p.meta;
  // sequence b's blocks are the last n_b positions of its part of the block space, which
  // holds G more (the charge of its start) when it is not empty
  const int P0 = meta[1 + b], P1 = meta[2 + b];
  const int nblk = P1 > P0 ? P1 - P0 - meta[B + 2] : 0;
  if (nblk <= 0) return;  // empty sequence: written by the decode kernel
  const int per = meta[0], last = P1 - 1;
  const int i0 = (last - nblk + 1) / per, i1 = last / per;
  const int nch = i1 - i0 + 1;
  const size_t base = ((size_t)b + i0) * R + r;   // piece c of (b, row) at row base + c * R
  const int d = lane * 8;
  const float* po = p.part_o + base * 512 + d;
  const size_t stride = (size_t)R * 512;
  // this wavefront's pieces: c = w0 + WPR k, k < nk
  const int w0 = WPR == 1 ? 0 : w;
  const int nk = nch > w0 ? (nch - w0 + WPR - 1) / WPR : 0;
  float m = NEG_INF, wsum = 0.f;
  f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = acc0;
  for (int k0 = 0; k0 < nk; k0 += CB) {
    const int n = min(CB, nk - k0);
    float lc[CB], iv[CB];
    f32x4 v0[CB], v1[CB];
    // the pieces' lse and 1/sum(P) first: a negative factor marks an fp16 piece (a range's last
    // piece: 512 fp16 values in the first half of its row, scaled by -factor), whose lane chunk
    // is then loaded twice (the second load hits the cache) instead of two fp32 halves
#pragma unroll
    for (int j = 0; j < CB; ++j) {
      // past the last piece the loads repeat it (no branches around them) and are dropped
      const int c = w0 + WPR * (j < n ? k0 + j : nk - 1);
      const size_t u = base + (size_t)c * R;
      lc[j] = p.part_lse[u];
      iv[j] = p.part_inv[u];
    }
#pragma unroll
    for (int j = 0; j < CB; ++j) {
      const int c = w0 + WPR * (j < n ? k0 + j : nk - 1);
      const bool h = iv[j] < 0.f;
      const float* a = h ? p.part_o + (base + (size_t)c * R) * 512 + lane * 4 : po + (size_t)c * stride;
      v0[j] = *(const f32x4*)a;
      v1[j] = *(const f32x4*)(h ? a : a + 4);
    }
#pragma unroll
    for (int j = 0; j < CB; ++j) {
      if (iv[j] < 0.f) {
        const u32x4 q = __builtin_bit_cast(u32x4, v0[j]);
        v0[j] = f32x4{half_bits_to_f32(q[0] & 0xFFFFu), half_bits_to_f32(q[0] >> 16), half_bits_to_f32(q[1] & 0xFFFFu),
                      half_bits_to_f32(q[1] >> 16)};
        v1[j] = f32x4{half_bits_to_f32(q[2] & 0xFFFFu), half_bits_to_f32(q[2] >> 16), half_bits_to_f32(q[3] & 0xFFFFu),
                      half_bits_to_f32(q[3] >> 16)};
        iv[j] = -iv[j];
      }
      lc[j] = j < n ? lc[j] : NEG_INF;
      iv[j] = j < n ? iv[j] : 0.f;
    }
    float mb = NEG_INF;
#pragma unroll
    for (int j = 0; j < CB; ++j) mb = fmaxf(mb, lc[j]);
    if (mb > m) {
      // every earlier weight is relative to m; m = -inf means nothing was added yet
      const float sc = m == NEG_INF ? 0.f : __builtin_amdgcn_exp2f((m - mb) * LOG2E);
      acc0 *= sc;
      acc1 *= sc;
      wsum *= sc;
      m = mb;
    }
#pragma unroll
    for (int j = 0; j < CB; ++j) {
      const float wc = lc[j] == NEG_INF ? 0.f : __builtin_amdgcn_exp2f((lc[j] - m) * LOG2E);
      wsum += wc;
      const float f = wc * iv[j];   // 0 for the repeated loads past the last piece
      acc0 += f * v0[j];
      acc1 += f * v1[j];
    }
  }
  if constexpr (WPR > 1) {
    // the wavefronts' running states, merged by wavefront 0 (a wavefront without pieces
    // has m = -inf and weight 0)
    __shared__ f32x4 xo[WPR - 1][2][64];
    __shared__ float xm[WPR - 1], xs[WPR - 1];
    if (w > 0) {
      xo[w - 1][0][lane] = acc0;
      xo[w - 1][1][lane] = acc1;
      if (lane == 0) {
        xm[w - 1] = m;
        xs[w - 1] = wsum;
      }
    }
    __syncthreads();
    if (w > 0) return;
    float mm = m;
#pragma unroll
    for (int q = 0; q < WPR - 1; ++q) mm = fmaxf(mm, xm[q]);
    if (mm == NEG_INF) {
      wsum = 0.f;
    } else {
      const float e = m == NEG_INF ? 0.f : __builtin_amdgcn_exp2f((m - mm) * LOG2E);
      acc0 *= e;
      acc1 *= e;
      wsum *= e;
#pragma unroll
      for (int q = 0; q < WPR - 1; ++q) {
        const float eq = xm[q] == NEG_INF ? 0.f : __builtin_amdgcn_exp2f((xm[q] - mm) * LOG2E);
        wsum += eq * xs[q];
        acc0 += eq * xo[q][0][lane];
        acc1 += eq * xo[q][1][lane];
      }
    }
    m = mm;
  }
  const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
  const f32x4 o0 = acc0 * inv, o1 = acc1 * inv;
  const size_t ob = (size_t)idx * 512 + d;
  if (p.out_bf16) {
    *(u32x4*)((bf16_t*)p.out + ob) =
        u32x4{pack_bf16x2(o0[0], o0[1]), pack_bf16x2(o0[2], o0[3]), pack_bf16x2(o1[0], o1[1]), pack_bf16x2(o1[2], o1[3])};
  } else {
    *(f32x4*)((float*)p.out + ob) = o0;
    *(f32x4*)((float*)p.out + ob + 4) = o1;
  }
  if (p.out_lse != nullptr && lane == 0) p.out_lse[idx] = wsum > 0.f ? m + logf(wsum) : NEG_INF;
}

// ---------------------------------------------------------------------------------------
// Partition mode over a 512-wide latent (not a mixed history): the same merge as
// combine_kernel with one wavefront per (b, row), four per workgroup, each lane owning 8
// columns.  A partial's address does not depend on the sequence's partition count, so the
// first batch of partials (and their lse) is loaded together with seq_lens[b], and the
// partitions past the count (never written by this decode) are masked afterwards: the kernel
// costs one memory round trip, not the two of a count loaded first.
// ---------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void combine_part_kernel(CombineParams p) {
  constexpr int CB = 8;
  constexpr float LOG2E = 1.4426950408889634f;
  const float NEG_INF = -__builtin_inff();
  const int lane = threadIdx.x & 63;
  const int R = p.R, B = p.B, MC = p.max_chunks;
  const int idx = (int)blockIdx.x * 4 + __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);   // b * R + row
  if (idx >= B * R) return;
  const int b = idx / R, r = idx - b * R;
  const size_t base = (size_t)b * MC * R + r;   // partial c of (b, row) at row base + c * R
  const int d = lane * 8;
  const float* po = p.part_o + base * 512 + d;
  const size_t stride = (size_t)R * 512;
  float lc[CB];
  f32x4 v0[CB], v1[CB];
  // first batch: partitions 0 .. CB - 1 (repeating the last one when there are fewer)
#pragma unroll
  for (int j = 0; j < CB; ++j) {
    const int c = j < MC ? j : MC - 1;
    lc[j] = p.part_lse[base + (size_t)c * R];
    v0[j] = *(const f32x4*)(po + (size_t)c * stride);
    v1[j] = *(const f32x4*)(po + (size_t)c * stride + 4);
  }
  int L = p.seq_lens[b];
  L = L < 0 ? 0 : (L > p.max_seq_len ? p.max_seq_len : L);
  const int nblk = (L + BLOCK_TOKENS - 1) / BLOCK_TOKENS;
  int nch = (nblk + p.tpc - 1) / p.tpc;
  nch = nch < 1 ? 1 : (nch > MC ? MC : nch);
  float m = NEG_INF, wsum = 0.f;
  f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = acc0;
  // merge a loaded batch of partitions c0 .. c0 + CB - 1; those past nch (stale bytes) drop out
  auto merge = [&](int c0) {
#pragma unroll
    for (int j = 0; j < CB; ++j) {
      const bool ok = c0 + j < nch;
      lc[j] = ok ? lc[j] : NEG_INF;
      v0[j] = ok ? v0[j] : f32x4{0.f, 0.f, 0.f, 0.f};
      v1[j] = ok ? v1[j] : f32x4{0.f, 0.f, 0.f, 0.f};
    }
    float mb = NEG_INF;
#pragma unroll
    for (int j = 0; j < CB; ++j) mb = fmaxf(mb, lc[j]);
    if (mb > m) {
      // every earlier weight is relative to m; m = -inf means nothing was added yet
      const float sc = m == NEG_INF ? 0.f : __builtin_amdgcn_exp2f((m - mb) * LOG2E);
      acc0 *= sc;
      acc1 *= sc;
      wsum *= sc;
      m = mb;
    }
#pragma unroll
    for (int j = 0; j < CB; ++j) {
      const float wc = lc[j] == NEG_INF ? 0.f : __builtin_amdgcn_exp2f((lc[j] - m) * LOG2E);
      wsum += wc;
      acc0 += wc * v0[j];
      acc1 += wc * v1[j];
    }
  };
  merge(0);
  for (int c0 = CB; c0 < nch; c0 += CB) {
#pragma unroll
    for (int j = 0; j < CB; ++j) {
      const int c = c0 + j < nch ? c0 + j : nch - 1;
      lc[j] = p.part_lse[base + (size_t)c * R];
      v0[j] = *(const f32x4*)(po + (size_t)c * stride);
      v1[j] = *(const f32x4*)(po + (size_t)c * stride + 4);
    }
    merge(c0);
  }
  const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
  const f32x4 o0 = acc0 * inv, o1 = acc1 * inv;
  const size_t ob = (size_t)idx * 512 + d;
  if (p.out_bf16) {
    *(u32x4*)((bf16_t*)p.out + ob) =
        u32x4{pack_bf16x2(o0[0], o0[1]), pack_bf16x2(o0[2], o0[3]), pack_bf16x2(o1[0], o1[1]), pack_bf16x2(o1[2], o1[3])};
  } else {
    *(f32x4*)((float*)p.out + ob) = o0;
    *(f32x4*)((float*)p.out + ob + 4) = o1;
  }
  if (p.out_lse != nullptr && lane == 0) p.out_lse[idx] = wsum > 0.f ? m + logf(wsum) : NEG_INF;
}

// ---------------------------------------------------------------------------------------
// Merge over several decodes (the mixed-precision history): attention over disjoint token
// sets merges exactly by log-sum-exp, so the split partials of every part, partition or range
// mode, are read in place and merged in one pass: one workgroup of 128 threads per (b, row),
// each thread owning 4 columns, partials taken in batches of CB per part with a running
// maximum across parts.  A (b, row) with no token in any part gets o = 0 and lse = -inf.
// ---------------------------------------------------------------------------------------
template <int CB>
__global__ __launch_bounds__(128) void combine_parts_kernel(CombinePartsParams p) {
  constexpr float LOG2E = 1.4426950408889634f;
  const float NEG_INF = -__builtin_inff();
  const int tid = threadIdx.x;
  const int R = p.R, d_c = p.d_c;
  const int b = blockIdx.x / R, r = blockIdx.x % R;
  const bool vec4 = (d_c & 3) == 0;
  float lse_out = NEG_INF;
  for (int d = tid * 4; d < d_c; d += 512) {
    float m = NEG_INF, wsum = 0.f;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int pi = 0; pi < p.n_parts; ++pi) {
      const CombinePart& q = p.part[pi];
      int nch;
      size_t base;
      if (q.meta == nullptr) {
        int L = q.seq_lens[b];
        L = L < 0 ? 0 : (L > q.max_seq_len ? q.max_seq_len : L);
        const int nblk = (L + BLOCK_TOKENS - 1) / BLOCK_TOKENS;
        nch = (nblk + q.tpc - 1) / q.tpc;
        nch = nch < 1 ? 1 : (nch > q.max_chunks ? q.max_chunks : nch);
        base = (size_t)b * q.max_chunks * R + r;
      } else {
        const int span = q.meta[2 + b] - q.meta[1 + b];
        const int nblk = span > 0 ? span - q.meta[p.B + 2] : 0;   // blocks (see combine_kernel)
        if (nblk <= 0) continue;   // no piece
        const int per = q.meta[0], last = q.meta[2 + b] - 1;
        const int i0 = (last - nblk + 1) / per, i1 = last / per;
        nch = i1 - i0 + 1;
        base = ((size_t)b + i0) * R + r;
      }
      const size_t stride = (size_t)R * d_c;
      for (int c0 = 0; c0 < nch; c0 += CB) {
        const int n = min(CB, nch - c0);
        const size_t ub = base + (size_t)c0 * R;
        float lc[CB], iv[CB];
        f32x4 v[CB];
#pragma unroll
        for (int j = 0; j < CB; ++j) {
          const bool ok = j < n;
          lc[j] = ok ? q.lse[ub + (size_t)j * R] : NEG_INF;
          iv[j] = ok && q.inv != nullptr ? q.inv[ub + (size_t)j * R] : 1.f;
          v[j] = f32x4{0.f, 0.f, 0.f, 0.f};
          if (ok) {
            const float* src = q.o + ub * d_c + d + j * stride;
            if (iv[j] < 0.f) {
              // a range's last piece of a row-owner decode: fp16 values scaled by -iv
              const uint2 hh = *(const uint2*)((const uint16_t*)(q.o + (ub + (size_t)j * R) * d_c) + d);
              v[j] = f32x4{half_bits_to_f32(hh.x & 0xFFFFu), half_bits_to_f32(hh.x >> 16), half_bits_to_f32(hh.y & 0xFFFFu),
                           half_bits_to_f32(hh.y >> 16)};
              iv[j] = -iv[j];
            } else if (vec4) {
              v[j] = *(const f32x4*)src;
            } else {
#pragma unroll
              for (int i = 0; i < 4; ++i) v[j][i] = d + i < d_c ? src[i] : 0.f;
            }
          }
        }
        float mb = NEG_INF;
#pragma unroll
        for (int j = 0; j < CB; ++j) mb = fmaxf(mb, lc[j]);
        if (mb > m) {
          // earlier weights are relative to m; m = -inf means nothing was added yet
          const float sc = m == NEG_INF ? 0.f : __builtin_amdgcn_exp2f((m - mb) * LOG2E);
          acc *= sc;
          wsum *= sc;
          m = mb;
        }
#pragma unroll
        for (int j = 0; j < CB; ++j) {
          const float wc = lc[j] == NEG_INF ? 0.f : __builtin_amdgcn_exp2f((lc[j] - m) * LOG2E);
          wsum += wc;
          acc += (wc * iv[j]) * v[j];
        }
      }
    }
    const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
    const f32x4 o = acc * inv;
    const size_t ob = ((size_t)b * R + r) * d_c + d;
    if (!vec4) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (d + i >= d_c) break;
        if (p.out_bf16)
          ((uint16_t*)p.out)[ob + i] = (uint16_t)f32_to_bf16_bits(o[i]);
        else
          ((float*)p.out)[ob + i] = o[i];
      }
    } else if (p.out_bf16) {
      *(uint2*)((bf16_t*)p.out + ob) = uint2{pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3])};
    } else {
      *(f32x4*)((float*)p.out + ob) = o;
    }
    lse_out = wsum > 0.f ? m + logf(wsum) : NEG_INF;
  }
  if (p.out_lse != nullptr && tid == 0) p.out_lse[(size_t)b * R + r] = lse_out;
}

hipError_t launch_decode_f32(const DecodeParams& p, hipStream_t st) {
  hipLaunchKernelGGL(decode_f32_kernel, dim3(p.total_units), dim3(128), 0, st, p);
  return hipGetLastError();
}

hipError_t launch_combine(const CombineParams& p, int batch, hipStream_t st) {
  if (p.meta != nullptr && !p.chunk_major && p.d_c == 512 && p.part_inv != nullptr) {
    if (p.many_parts) {
      hipLaunchKernelGGL((combine_rows_kernel<4, 8>), dim3((unsigned)((int64_t)batch * p.R)), dim3(256), 0, st, p);
    } else {
      const int64_t quads = ((int64_t)batch * p.R + 3) / 4;
      hipLaunchKernelGGL((combine_rows_kernel<1, 4>), dim3((unsigned)quads), dim3(256), 0, st, p);
    }
    return hipGetLastError();
  }
  if (p.meta == nullptr && !p.chunk_major && !p.mixed && p.d_c == 512 && p.part_inv == nullptr &&
      p.max_chunks >= 1) {
    const int64_t quads = ((int64_t)batch * p.R + 3) / 4;
    hipLaunchKernelGGL(combine_part_kernel, dim3((unsigned)quads), dim3(256), 0, st, p);
    return hipGetLastError();
  }
  if (p.many_parts)
    hipLaunchKernelGGL(combine_kernel<32>, dim3(batch * p.R), dim3(128), 0, st, p);
  else
    hipLaunchKernelGGL(combine_kernel<8>, dim3(batch * p.R), dim3(128), 0, st, p);
  return hipGetLastError();
}

hipError_t launch_combine_parts(const CombinePartsParams& p, hipStream_t st) {
  if (p.many_parts)
    hipLaunchKernelGGL(combine_parts_kernel<32>, dim3(p.B * p.R), dim3(128), 0, st, p);
  else
    hipLaunchKernelGGL(combine_parts_kernel<8>, dim3(p.B * p.R), dim3(128), 0, st, p);
  return hipGetLastError();
}

}  // namespace mla
