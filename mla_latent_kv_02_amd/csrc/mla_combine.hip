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
    if (tok < tok_end) {
      const int id = btab[tok / BLOCK_TOKENS];
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
      const int id = btab[tk / BLOCK_TOKENS];
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
    const int nblk = (L + BLOCK_TOKENS - 1) / BLOCK_TOKENS;
    nch = (nblk + p.tpc - 1) / p.tpc;
    nch = nch < 1 ? 1 : (nch > p.max_chunks ? p.max_chunks : nch);
    base = (size_t)b * p.max_chunks * R + r;
  } else {
    // sequence b's blocks are the last n_b positions of its part of the block space
    int L = p.seq_lens[b];
    L = L < 0 ? 0 : (L > p.max_seq_len ? p.max_seq_len : L);
    const int nblk = (L + BLOCK_TOKENS - 1) / BLOCK_TOKENS;
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

hipError_t launch_decode_f32(const DecodeParams& p, hipStream_t st) {
  hipLaunchKernelGGL(decode_f32_kernel, dim3(p.total_units), dim3(128), 0, st, p);
  return hipGetLastError();
}

hipError_t launch_combine(const CombineParams& p, int batch, hipStream_t st) {
  if (p.many_parts)
    hipLaunchKernelGGL(combine_kernel<32>, dim3(batch * p.R), dim3(128), 0, st, p);
  else
    hipLaunchKernelGGL(combine_kernel<8>, dim3(batch * p.R), dim3(128), 0, st, p);
  return hipGetLastError();
}

}  // namespace mla
