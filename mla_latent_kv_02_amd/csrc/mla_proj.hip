// Per-head projections around the latent attention:
//   query absorption    q_lat[n,h,:] = q_nope[n,h,:] . W_UK[h]   (GQLA abstract: absorbed MQA form)
//   value up-projection out[n,h,:]  = o_lat[n,h,:] . W_UV[h]    (RAQ-MLA abstract: latent up-projected)
// Both are Y[n][h][:] = X[n][h][:] . W[h] with W [H][K][M] row-major.  At decode batch sizes
// (N = batch * s_q rows) this is a read of W with little reuse, so the kernel is built to
// read W once and X a few times, with one dependent memory round trip per workgroup:
//   * workgroup = (MB output columns, head h, 16 * waves rows); wave w owns rows 16 w .. +15
//     and all MB columns, over the whole K (no cross-wave reduction);
//   * the W tile [K][MB] is staged in LDS (rows padded by 8 elements so that transposed
//     reads of 4 rows fall on distinct banks) and read with ds_read_b64_tr_b16 as the A
//     operand of Y^T = W^T . X^T on v_mfma_f32_16x16x32_bf16;
//   * X rows are read from global memory one k-step ahead (B operand); fp32 X is split into
//     hi + lo bf16 terms so the product keeps ~16 mantissa bits of X.
// Other dtype combinations run a plain fp32 loop.
#include <hip/hip_runtime.h>

#include "mla_device.hpp"
#include "mla_internal.hpp"

namespace mla {

typedef __attribute__((address_space(3))) i16x4 lds_i16x4_p;

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

// grid (M / MB, H, ceil(N / (16 * RW))), block 256, RW = row tiles (16 rows each) per
// workgroup, K % 32 == 0, K <= 512.  All four waves stage the W tile.
//   KSPLIT = 1: wave w < RW owns row tile w over every k-step;
//   KSPLIT = 4: wave w owns k-steps w, w + 4, ... for every row tile, and the four partial
//               sums are added through LDS (the W tile's space, free by then).
// Every X fragment a wave needs is requested before the W tile is waited for.
// Dynamic LDS: max(W tile [K][MB + 8] bf16, KSPLIT = 4: 3 x RW x MB/16 x 1 KB partials).
template <bool XF32, bool YF32, int MB, int KSPLIT>
__global__ __launch_bounds__(256) void proj_mfma_kernel(ProjParams p, int RW) {
  constexpr int MT = MB / 16;            // column tiles
  constexpr int LD = MB + 8;             // padded LDS row (elements)
  constexpr int RT = KSPLIT == 1 ? 1 : 4;          // row tiles per wave (at most)
  constexpr int KSW = 16 / KSPLIT;                  // k-steps per wave (at most; K <= 512)
  constexpr int XV = XF32 ? 2 : 1;
  extern __shared__ __attribute__((aligned(16))) uint8_t pj_lds[];
  bf16_t* Ws = (bf16_t*)pj_lds;
  const int tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63, lr = lane & 15, lg = lane >> 4;
  const int h = blockIdx.y;
  const int m0 = blockIdx.x * MB;
  const int K = p.K, M = p.M, N = p.N;
  const int nks = K / 32;
  const int n0 = blockIdx.z * 16 * RW;
  // this wave's row tiles and k-steps
  const int rt0 = KSPLIT == 1 ? w : 0;
  const int nrt = KSPLIT == 1 ? (w < RW ? 1 : 0) : RW;
  auto kstep = [&](int j) { return KSPLIT == 1 ? j : w + 4 * j; };

  // X fragments: row n = n0 + 16 (rt0 + r) + lr, k = 32 ks + 8 lg .. + 7
  u32x4 xr[RT][KSW][XV];
#pragma unroll
  for (int r = 0; r < RT; ++r) {
    const int n = n0 + 16 * (rt0 + r) + lr;
    const bool rok = r < nrt && n < N;
    const size_t xo = (size_t)(rok ? n : 0) * p.sxn + (size_t)h * p.sxh + lg * 8;
#pragma unroll
    for (int j = 0; j < KSW; ++j) {
      const int ks = kstep(j);
      const bool ok = rok && ks < nks;
#pragma unroll
      for (int v = 0; v < XV; ++v) {
        if (XF32)
          xr[r][j][v] = ok ? *(const u32x4*)((const float*)p.X + xo + ks * 32 + 4 * v) : u32x4{0, 0, 0, 0};
        else
          xr[r][j][v] = ok ? *(const u32x4*)((const bf16_t*)p.X + xo + ks * 32) : u32x4{0, 0, 0, 0};
      }
    }
  }

  // W tile: K rows of MB elements, 16-byte pieces, CH per thread in flight at once
  const bf16_t* W = (const bf16_t*)p.W + (size_t)h * K * M + m0;
  constexpr int PR = MB / 8;
  constexpr int CH = 8;
  const int npieces = K * PR;
  for (int q0 = 0; q0 < npieces; q0 += CH * 256) {
    u32x4 v[CH];
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const int q = q0 + c * 256 + tid;
      const int k = q / PR, pc = q - k * PR;
      v[c] = q < npieces ? *(const u32x4*)(W + (size_t)k * M + pc * 8) : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const int q = q0 + c * 256 + tid;
      const int k = q / PR, pc = q - k * PR;
      if (q < npieces) *(u32x4*)&Ws[k * LD + pc * 8] = v[c];
    }
  }
  __syncthreads();

  // Y^T[m][n] += W^T[m][k] . X^T[k][n]: A = W^T from LDS (transposed reads), B = X^T
  f32x4 acc[RT][MT];
#pragma unroll
  for (int r = 0; r < RT; ++r)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[r][mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < KSW; ++j) {
    const int ks = kstep(j);
    if (ks >= nks) break;
    bf16x8 bh[RT], bl[RT];
#pragma unroll
    for (int r = 0; r < RT; ++r) {
      if (XF32) {
        u32x4 vh, vl;
        split_hi_lo(__builtin_bit_cast(f32x4, xr[r][j][0]), __builtin_bit_cast(f32x4, xr[r][j][XV - 1]), vh, vl);
        bh[r] = __builtin_bit_cast(bf16x8, vh);
        bl[r] = __builtin_bit_cast(bf16x8, vl);
      } else {
        bh[r] = __builtin_bit_cast(bf16x8, xr[r][j][0]);
      }
    }
    const bf16_t* wb = &Ws[(ks * 32 + lg * 8 + (lr >> 2)) * LD + (lr & 3) * 4];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_p*)(wb + mt * 16));
      const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_p*)(wb + 4 * LD + mt * 16));
      const bf16x8 av = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
      for (int r = 0; r < RT; ++r) {
        if (r >= nrt) break;
        acc[r][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bh[r], acc[r][mt], 0, 0, 0);
        if (XF32) acc[r][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bl[r], acc[r][mt], 0, 0, 0);
      }
    }
  }

  if constexpr (KSPLIT == 4) {
    // waves 1..3 hand their partial sums to wave 0 through LDS
    __syncthreads();
    f32x4* part = (f32x4*)pj_lds;   // [3][RW][MT][64]
    if (w > 0) {
#pragma unroll
      for (int r = 0; r < RT; ++r) {
        if (r >= nrt) break;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) part[(((w - 1) * RW + r) * MT + mt) * 64 + lane] = acc[r][mt];
      }
    }
    __syncthreads();
    if (w > 0) return;
#pragma unroll
    for (int r = 0; r < RT; ++r) {
      if (r >= nrt) break;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int q = 0; q < 3; ++q) acc[r][mt] += part[((q * RW + r) * MT + mt) * 64 + lane];
    }
  }

  // Y^T tile: this lane holds row n, columns m0 + 16 mt + 4 lg .. + 3
#pragma unroll
  for (int r = 0; r < RT; ++r) {
    if (r >= nrt) break;
    const int n = n0 + 16 * (rt0 + r) + lr;
    if (n >= N) continue;
    const size_t yo = ((size_t)n * p.H + h) * M + m0 + 4 * lg;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      if (YF32)
        *(f32x4*)((float*)p.Y + yo + mt * 16) = acc[r][mt];
      else
        *(uint2*)((bf16_t*)p.Y + yo + mt * 16) =
            uint2{pack_bf16x2(acc[r][mt][0], acc[r][mt][1]), pack_bf16x2(acc[r][mt][2], acc[r][mt][3])};
    }
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

template <bool XF32, bool YF32, int MB, int KSPLIT>
static hipError_t launch_mb(const ProjParams& p, int rw, hipStream_t st) {
  const size_t w_lds = (size_t)p.K * (MB + 8) * 2;
  const size_t r_lds = KSPLIT == 4 ? (size_t)3 * rw * (MB / 16) * 1024 : 0;
  const size_t lds = w_lds > r_lds ? w_lds : r_lds;
  static bool attr_set = false;  // raise the dynamic-LDS limit once
  if (!attr_set) {
    const hipError_t e = hipFuncSetAttribute((const void*)proj_mfma_kernel<XF32, YF32, MB, KSPLIT>,
                                             hipFuncAttributeMaxDynamicSharedMemorySize, 96 * 1024);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  const dim3 grid(p.M / MB, p.H, (p.N + 16 * rw - 1) / (16 * rw));
  hipLaunchKernelGGL((proj_mfma_kernel<XF32, YF32, MB, KSPLIT>), grid, dim3(256), lds, st, p, rw);
  return hipGetLastError();
}

template <bool XF32, bool YF32, int KSPLIT>
static hipError_t launch_ks(const ProjParams& p, int rw, int mb, hipStream_t st) {
  switch (mb) {
    case 128: return launch_mb<XF32, YF32, 128, KSPLIT>(p, rw, st);
    case 64: return launch_mb<XF32, YF32, 64, KSPLIT>(p, rw, st);
    case 32: return launch_mb<XF32, YF32, 32, KSPLIT>(p, rw, st);
    default: return launch_mb<XF32, YF32, 16, KSPLIT>(p, rw, st);
  }
}

// Split K over the four waves when X rows are few or fp32 (all threads share the X reads);
// column block: the widest of 128/64/32/16 dividing M whose grid still gives >= 256 workgroups
// and whose LDS (W tile, or the K-split partials) fits 96 KB.
template <bool XF32, bool YF32>
static hipError_t launch_proj_mfma(const ProjParams& p, hipStream_t st) {
  const int rw = p.N >= 64 ? 4 : (p.N + 15) / 16;   // row tiles per workgroup
  const int64_t nb = (p.N + 16 * rw - 1) / (16 * rw);
  const bool ksplit = (XF32 || p.N <= 32) && p.K / 32 >= 4;
  auto lds_of = [&](int mb) {
    const size_t w = (size_t)p.K * (mb + 8) * 2, r = ksplit ? (size_t)3 * rw * (mb / 16) * 1024 : 0;
    return w > r ? w : r;
  };
  int mb = 128;
  while (mb > 16 && (p.M % mb != 0 || (int64_t)(p.M / mb) * p.H * nb < 256 || lds_of(mb) > 96 * 1024)) mb >>= 1;
  return ksplit ? launch_ks<XF32, YF32, 4>(p, rw, mb, st) : launch_ks<XF32, YF32, 1>(p, rw, mb, st);
}

hipError_t launch_proj(const ProjParams& p, hipStream_t st) {
  const bool mfma = p.aligned16 && !p.w_f32 && p.K % 32 == 0 && p.K <= 512 && p.M % 16 == 0 &&
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
