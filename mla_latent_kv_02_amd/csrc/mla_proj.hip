// Per-head projections around the latent attention:
//   query absorption    q_lat[n,h,:] = q_nope[n,h,:] . W_UK[h]   (GQLA abstract: absorbed MQA form)
//   value up-projection out[n,h,:]  = o_lat[n,h,:] . W_UV[h]    (RAQ-MLA abstract: latent up-projected)
// Both are Y[n][h][:] = X[n][h][:] . W[h] with W [H][K][M] row-major.  At decode batch
// sizes (N = batch * s_q rows) this is a latency-bound read of W, so the work is cut
// fine: one workgroup per (head, 16 output columns), the K reduction split over the 4
// wavefronts and merged through LDS.  bf16 weights use v_mfma_f32_16x16x32_bf16 with
// W^T operands read by ds_read_b64_tr_b16; fp32 X is split into hi + lo bf16 terms so
// the product keeps ~16 mantissa bits of X.  Other dtype combinations run a plain fp32 loop.
#include <hip/hip_runtime.h>

#include "mla_device.hpp"
#include "mla_internal.hpp"

namespace mla {

typedef __attribute__((address_space(3))) i16x4 lds_i16x4_p;

constexpr int PJ_NT = 256;
constexpr int PJ_MT = 8;  // 16-row tiles per pass (128 rows)

__device__ __forceinline__ void split_hi_lo(const f32x4& a, const f32x4& b, u32x4& vh, u32x4& vl) {
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const float x0 = a[2 * j], x1 = a[2 * j + 1], y0 = b[2 * j], y1 = b[2 * j + 1];
    const uint32_t hx = pack_bf16x2(x0, x1), hy = pack_bf16x2(y0, y1);
    vh[j] = hx;
    vh[2 + j] = hy;
    vl[j] = pack_bf16x2(x0 - bf16_bits_to_f32(hx & 0xFFFFu), x1 - bf16_bits_to_f32(hx >> 16));
    vl[2 + j] = pack_bf16x2(y0 - bf16_bits_to_f32(hy & 0xFFFFu), y1 - bf16_bits_to_f32(hy >> 16));
  }
}

// grid (M/16, H); K % 128 == 0, K <= 1024
template <bool XF32, bool YF32>
__global__ __launch_bounds__(PJ_NT) void proj_mfma_kernel(ProjParams p) {
  __shared__ __attribute__((aligned(16))) bf16_t Ws[1024 * 16];      // [K][16]
  __shared__ __attribute__((aligned(16))) f32x4 part[3][PJ_MT][64];  // partial sums of waves 1..3
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, lr = lane & 15, lg = lane >> 4;
  const int h = blockIdx.y;
  const int c0 = blockIdx.x * 16;
  const int K = p.K, M = p.M, N = p.N;
  const bf16_t* W = (const bf16_t*)p.W + (size_t)h * K * M + c0;
  for (int q = tid; q < K * 2; q += PJ_NT) {
    const int k = q >> 1, piece = q & 1;
    *(u32x4*)&Ws[k * 16 + piece * 8] = *(const u32x4*)(W + (size_t)k * M + piece * 8);
  }
  const int KW = K / 4;  // k range of this wavefront
  const int kb = w * KW;
  __syncthreads();
  for (int nb = 0; nb < N; nb += 16 * PJ_MT) {
    const int mts = min(PJ_MT, (N - nb + 15) / 16);
    f32x4 acc[PJ_MT];
#pragma unroll
    for (int mt = 0; mt < PJ_MT; ++mt) acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int kk = kb; kk < kb + KW; kk += 32) {
      const bf16_t* wb = &Ws[(kk + lg * 8 + (lr >> 2)) * 16 + (lr & 3) * 4];
      const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_p*)wb);
      const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_p*)(wb + 4 * 16));
      const bf16x8 bv = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
      for (int mt = 0; mt < PJ_MT; ++mt) {
        if (mt >= mts) break;
        const int n = nb + mt * 16 + lr;
        const size_t xo = (size_t)n * p.sxn + (size_t)h * p.sxh + kk + lg * 8;
        if (!XF32) {
          const u32x4 v = n < N ? *(const u32x4*)((const bf16_t*)p.X + xo) : u32x4{0, 0, 0, 0};
          acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, v), bv, acc[mt], 0, 0, 0);
        } else {
          f32x4 a = {0.f, 0.f, 0.f, 0.f}, b = {0.f, 0.f, 0.f, 0.f};
          if (n < N) {
            a = *(const f32x4*)((const float*)p.X + xo);
            b = *(const f32x4*)((const float*)p.X + xo + 4);
          }
          u32x4 vh, vl;
          split_hi_lo(a, b, vh, vl);
          acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, vh), bv, acc[mt], 0, 0, 0);
          acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, vl), bv, acc[mt], 0, 0, 0);
        }
      }
    }
    // merge the four k ranges: waves 1..3 hand their sums to wave 0
    if (w > 0) {
#pragma unroll
      for (int mt = 0; mt < PJ_MT; ++mt)
        if (mt < mts) part[w - 1][mt][lane] = acc[mt];
    }
    __syncthreads();
    if (w == 0) {
#pragma unroll
      for (int mt = 0; mt < PJ_MT; ++mt) {
        if (mt >= mts) break;
        const f32x4 v = acc[mt] + part[0][mt][lane] + part[1][mt][lane] + part[2][mt][lane];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int n = nb + mt * 16 + lg * 4 + i;
          if (n >= N) continue;
          const size_t yo = ((size_t)n * p.H + h) * M + c0 + lr;
          if (YF32)
            ((float*)p.Y)[yo] = v[i];
          else
            ((uint16_t*)p.Y)[yo] = (uint16_t)f32_to_bf16_bits(v[i]);
        }
      }
    }
    __syncthreads();
  }
}

__device__ __forceinline__ float load_any(const void* base, size_t i, int f32) {
  return f32 ? ((const float*)base)[i] : bf16_bits_to_f32(((const uint16_t*)base)[i]);
}

// Plain fp32 fallback: one thread per output element.
__global__ __launch_bounds__(256) void proj_f32_kernel(ProjParams p) {
  const size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x;
  const size_t total = (size_t)p.N * p.H * p.M;
  if (idx >= total) return;
  const int m = (int)(idx % p.M);
  const int h = (int)((idx / p.M) % p.H);
  const int n = (int)(idx / ((size_t)p.M * p.H));
  const size_t xo = (size_t)n * p.sxn + (size_t)h * p.sxh;
  const size_t wo = (size_t)h * p.K * p.M + m;
  float acc = 0.f;
  for (int k = 0; k < p.K; ++k)
    acc = __builtin_fmaf(load_any(p.X, xo + k, p.x_f32), load_any(p.W, wo + (size_t)k * p.M, p.w_f32), acc);
  if (p.y_f32)
    ((float*)p.Y)[idx] = acc;
  else
    ((uint16_t*)p.Y)[idx] = (uint16_t)f32_to_bf16_bits(acc);
}

hipError_t launch_proj(const ProjParams& p, hipStream_t st) {
  const bool mfma = p.aligned16 && !p.w_f32 && p.K % 128 == 0 && p.K <= 1024 && p.M % 16 == 0 &&
                    (p.sxn % 8 == 0) && (p.sxh % 8 == 0);
  if (mfma) {
    const dim3 grid(p.M / 16, p.H);
    if (p.x_f32) {
      if (p.y_f32)
        hipLaunchKernelGGL((proj_mfma_kernel<true, true>), grid, dim3(PJ_NT), 0, st, p);
      else
        hipLaunchKernelGGL((proj_mfma_kernel<true, false>), grid, dim3(PJ_NT), 0, st, p);
    } else {
      if (p.y_f32)
        hipLaunchKernelGGL((proj_mfma_kernel<false, true>), grid, dim3(PJ_NT), 0, st, p);
      else
        hipLaunchKernelGGL((proj_mfma_kernel<false, false>), grid, dim3(PJ_NT), 0, st, p);
    }
  } else {
    const size_t total = (size_t)p.N * p.H * p.M;
    hipLaunchKernelGGL(proj_f32_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, st, p);
  }
  return hipGetLastError();
}

}  // namespace mla
