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
// Combine: lse = log sum_c exp(lse_c), o = sum_c exp(lse_c - lse) o_c over the partitions of
// one (b, row), o_c = part_o_c (partition mode) or part_o_c * part_inv_c (range mode).  One workgroup of 128 threads per (b, row); weights go through LDS in
// batches of 128 partitions and each thread sums 4 columns with independent loads.
// ---------------------------------------------------------------------------------------
__global__ __launch_bounds__(128) void combine_kernel(CombineParams p) {
  __shared__ float wsh[128];   // weight of a partial's lse
  __shared__ float vsh[128];   // the same times its normalisation factor
  __shared__ float red[2];
  const int tid = threadIdx.x;
  const int R = p.R;
  const int b = blockIdx.x / R, r = blockIdx.x % R;
  const float NEG_INF = -__builtin_inff();
  int nch;
  size_t u0;
  if (p.meta == nullptr) {
    int L = p.seq_lens[b];
    L = L < 0 ? 0 : (L > p.max_seq_len ? p.max_seq_len : L);
    const int nblk = (L + BLOCK_TOKENS - 1) / BLOCK_TOKENS;
    nch = (nblk + p.tpc - 1) / p.tpc;
    nch = nch < 1 ? 1 : (nch > p.max_chunks ? p.max_chunks : nch);
    u0 = (size_t)b * p.max_chunks;
  } else {
    const int per = p.meta[0], first = p.meta[1 + b], nblk = p.meta[2 + b] - first;
    if (nblk <= 0) return;  // empty sequence: written by the decode kernel
    const int i0 = first / per, i1 = (first + nblk - 1) / per;
    nch = i1 - i0 + 1;
    u0 = (size_t)b + i0;
  }
  // max of the partition LSEs
  float m = NEG_INF;
  for (int c = tid; c < nch; c += 128) m = fmaxf(m, p.part_lse[(u0 + c) * R + r]);
  for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
  if ((tid & 63) == 0) red[tid >> 6] = m;
  __syncthreads();
  m = fmaxf(red[0], red[1]);
  const int d_c = p.d_c;
  f32x4 acc[4];
  for (int k = 0; k < 4; ++k) acc[k] = f32x4{0.f, 0.f, 0.f, 0.f};
  float wsum = 0.f;
  for (int c0 = 0; c0 < nch; c0 += 128) {
    const int n = min(128, nch - c0);
    __syncthreads();
    if (tid < n) {
      const float lc = p.part_lse[(u0 + c0 + tid) * R + r];
      const float wc = m == NEG_INF ? 0.f : expf(lc - m);
      wsh[tid] = wc;
      vsh[tid] = p.part_inv == nullptr ? wc : wc * p.part_inv[(u0 + c0 + tid) * R + r];
    }
    __syncthreads();
    for (int j = 0; j < n; ++j) wsum += wsh[j];
    for (int k = 0; k < 4; ++k) {
      const int d = (tid + k * 128) * 4;
      if (d >= d_c) break;
      const float* base = p.part_o + ((u0 + c0) * R + r) * (size_t)d_c + d;
      const size_t stride = (size_t)R * d_c;
      int j = 0;
      for (; j + 4 <= n; j += 4) {
        const f32x4 v0 = *(const f32x4*)(base + (j + 0) * stride);
        const f32x4 v1 = *(const f32x4*)(base + (j + 1) * stride);
        const f32x4 v2 = *(const f32x4*)(base + (j + 2) * stride);
        const f32x4 v3 = *(const f32x4*)(base + (j + 3) * stride);
        acc[k] += vsh[j] * v0 + vsh[j + 1] * v1 + vsh[j + 2] * v2 + vsh[j + 3] * v3;
      }
      for (; j < n; ++j) acc[k] += vsh[j] * *(const f32x4*)(base + j * stride);
    }
  }
  const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
  for (int k = 0; k < 4; ++k) {
    const int d = (tid + k * 128) * 4;
    if (d >= d_c) break;
    const f32x4 v = acc[k] * inv;
    const size_t ob = ((size_t)b * R + r) * d_c + d;
    if (p.out_bf16)
      *(uint2*)((bf16_t*)p.out + ob) = uint2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
    else
      *(f32x4*)((float*)p.out + ob) = v;
  }
  if (p.out_lse != nullptr && tid == 0) p.out_lse[(size_t)b * R + r] = wsum > 0.f ? m + logf(wsum) : NEG_INF;
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
