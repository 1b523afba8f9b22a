// Per-head projections around the latent attention:
//   query absorption    q_lat[n,h,:] = q_nope[n,h,:] . W_UK[h]   (GQLA abstract: absorbed MQA form)
//   value up-projection out[n,h,:]  = o_lat[n,h,:] . W_UV[h]    (RAQ-MLA abstract: latent up-projected)
// Both are Y[n][h][:] = X[n][h][:] . W[h] with W [H][K][M] row-major.  At decode batch
// sizes (N = batch * s_q rows) this is a latency-bound read of W, so the work is cut
// fine: one workgroup per (head, 16 output columns), the K reduction spread over up to 8
// wavefronts (k-step j on wavefront j % NW) and merged through LDS.  bf16 weights use v_mfma_f32_16x16x32_bf16 with
// W^T operands read by ds_read_b64_tr_b16; fp32 X is split into hi + lo bf16 terms so
// the product keeps ~16 mantissa bits of X.  Other dtype combinations run a plain fp32 loop.
#include <hip/hip_runtime.h>

#include "mla_device.hpp"
#include "mla_internal.hpp"

namespace mla {

typedef __attribute__((address_space(3))) i16x4 lds_i16x4_p;

constexpr int PJ_NW = 8;    // at most 8 wavefronts; k-step j of 32 belongs to wavefront j % NW
constexpr int PJ_KS = 4;    // at most 4 k-steps per wavefront (K <= 1024)

template <bool XF32>
constexpr int pj_mt() { return XF32 ? 4 : 8; }  // 16-row tiles per pass

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

// grid (M/16, H), NW = min(8, K/32) wavefronts; K % 32 == 0, K <= 1024.  Dynamic LDS:
// W tile [K][16] bf16, then (NW - 1) x PJ_MT x 64 partial sums.  Every X load of a wavefront
// (its k-steps, all row tiles of the pass) is issued before the W tile is waited for.
template <bool XF32, bool YF32>
__global__ __launch_bounds__(PJ_NW * 64) void proj_mfma_kernel(ProjParams p) {
  constexpr int PJ_MT = pj_mt<XF32>();
  extern __shared__ __attribute__((aligned(16))) uint8_t pj_lds[];
  const int NW = blockDim.x >> 6;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, lr = lane & 15, lg = lane >> 4;
  const int h = blockIdx.y;
  const int c0 = blockIdx.x * 16;
  const int K = p.K, M = p.M, N = p.N;
  bf16_t* Ws = (bf16_t*)pj_lds;                                   // [K][16]
  f32x4* part = (f32x4*)(pj_lds + (size_t)K * 32);                 // [NW-1][PJ_MT][64]
  const int nks = (K / 32 - w + NW - 1) / NW;  // k-steps w, w + NW, ...
  const bf16_t* W = (const bf16_t*)p.W + (size_t)h * K * M + c0;
  for (int nb = 0; nb < N; nb += 16 * PJ_MT) {
    const int mts = min(PJ_MT, (N - nb + 15) / 16);
    // X operands of this wavefront, loaded up front
    constexpr int XV = XF32 ? 2 : 1;
    u32x4 xr[PJ_KS][PJ_MT][XV];
#pragma unroll
    for (int ks = 0; ks < PJ_KS; ++ks) {
#pragma unroll
      for (int mt = 0; mt < PJ_MT; ++mt) {
        const int n = nb + mt * 16 + lr;
        const bool ok = ks < nks && mt < mts && n < N;
        const size_t xo = (size_t)(ok ? n : 0) * p.sxn + (size_t)h * p.sxh + (w + NW * ks) * 32 + lg * 8;
#pragma unroll
        for (int v = 0; v < XV; ++v) {
          if (XF32)
            xr[ks][mt][v] = ok ? *(const u32x4*)((const float*)p.X + xo + 4 * v) : u32x4{0, 0, 0, 0};
          else
            xr[ks][mt][v] = ok ? *(const u32x4*)((const bf16_t*)p.X + xo) : u32x4{0, 0, 0, 0};
        }
      }
    }
    if (nb == 0) {
      for (int q = tid; q < K * 2; q += NW * 64) {
        const int k = q >> 1, piece = q & 1;
        *(u32x4*)&Ws[k * 16 + piece * 8] = *(const u32x4*)(W + (size_t)k * M + piece * 8);
      }
      __syncthreads();
    }
    f32x4 acc[PJ_MT];
#pragma unroll
    for (int mt = 0; mt < PJ_MT; ++mt) acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < PJ_KS; ++ks) {
      if (ks >= nks) break;
      const bf16_t* wb = &Ws[((w + NW * ks) * 32 + lg * 8 + (lr >> 2)) * 16 + (lr & 3) * 4];
      const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_p*)wb);
      const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_p*)(wb + 4 * 16));
      const bf16x8 bv = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
      for (int mt = 0; mt < PJ_MT; ++mt) {
        if (mt >= mts) break;
        if (!XF32) {
          acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, xr[ks][mt][0]), bv, acc[mt], 0, 0, 0);
        } else {
          u32x4 vh, vl;
          split_hi_lo(__builtin_bit_cast(f32x4, xr[ks][mt][0]), __builtin_bit_cast(f32x4, xr[ks][mt][XV - 1]), vh, vl);
          acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, vh), bv, acc[mt], 0, 0, 0);
          acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, vl), bv, acc[mt], 0, 0, 0);
        }
      }
    }
    // merge the k ranges: waves 1..NW-1 hand their sums to wave 0
    if (w > 0) {
#pragma unroll
      for (int mt = 0; mt < PJ_MT; ++mt)
        if (mt < mts) part[((w - 1) * PJ_MT + mt) * 64 + lane] = acc[mt];
    }
    __syncthreads();
    if (w == 0) {
#pragma unroll
      for (int mt = 0; mt < PJ_MT; ++mt) {
        if (mt >= mts) break;
        f32x4 v = acc[mt];
        for (int j = 0; j < NW - 1; ++j) v += part[(j * PJ_MT + mt) * 64 + lane];
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

template <bool XF32, bool YF32>
static hipError_t launch_proj_mfma(const ProjParams& p, hipStream_t st) {
  const int nw = p.K / 32 < PJ_NW ? p.K / 32 : PJ_NW;
  const size_t lds = (size_t)p.K * 32 + (size_t)(nw - 1) * pj_mt<XF32>() * 64 * sizeof(f32x4);
  static bool attr_set = false;  // raise the dynamic-LDS limit once (max use 32 KB + 57 KB)
  if (!attr_set) {
    const hipError_t e = hipFuncSetAttribute((const void*)proj_mfma_kernel<XF32, YF32>,
                                             hipFuncAttributeMaxDynamicSharedMemorySize, 96 * 1024);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  hipLaunchKernelGGL((proj_mfma_kernel<XF32, YF32>), dim3(p.M / 16, p.H), dim3(nw * 64), lds, st, p);
  return hipGetLastError();
}

hipError_t launch_proj(const ProjParams& p, hipStream_t st) {
  const bool mfma = p.aligned16 && !p.w_f32 && p.K % 32 == 0 && p.K <= 1024 && p.M % 16 == 0 &&
                    (p.sxn % 8 == 0) && (p.sxh % 8 == 0);
  if (mfma) {
    if (p.x_f32) return p.y_f32 ? launch_proj_mfma<true, true>(p, st) : launch_proj_mfma<true, false>(p, st);
    return p.y_f32 ? launch_proj_mfma<false, true>(p, st) : launch_proj_mfma<false, false>(p, st);
  }
  const size_t total = (size_t)p.N * p.H * p.M;
  hipLaunchKernelGGL(proj_f32_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, st, p);
  return hipGetLastError();
}

}  // namespace mla
