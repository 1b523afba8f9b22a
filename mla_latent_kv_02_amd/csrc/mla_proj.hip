// Per-head projections around the latent attention:
//   query absorption    q_lat[n,h,:] = q_nope[n,h,:] . W_UK[h]   (GQLA abstract: absorbed MQA form)
//   value up-projection out[n,h,:]  = o_lat[n,h,:] . W_UV[h]    (RAQ-MLA abstract: latent up-projected)
// Both are Y[n][h][:] = X[n][h][:] . W[h] with W [H][K][M] row-major.  At decode batch sizes
// (N = batch * s_q rows) this is a stream of W with little reuse, so each workgroup makes one
// memory round trip with everything it needs in flight at once:
//   * workgroup = (head h, MB output columns, 16 * NBT rows); consecutive workgroups of one XCD
//     take the column and row blocks of one head, so X[h] and W[h] are shared in its L2;
//   * the W tile [K][MB] goes HBM -> LDS with global_load_lds_dwordx4 (no registers); piece c
//     of tile row k sits at physical piece c ^ wsw(k), so that the transposed reads
//     (ds_read_b64_tr_b16, the A operand of Y^T = W^T . X^T on v_mfma_f32_16x16x32_bf16) of 32
//     lanes fall on distinct banks;
//   * X fragments (the B operand) are loaded into registers at the same time; fp32 X is split
//     into hi + lo bf16 terms so the product keeps ~16 mantissa bits of X;
//   * the 16 x 16 output tiles are dealt to the four waves; with fewer than four tiles the
//     waves split K instead and add their partial sums through LDS.
// Other dtype combinations run a plain fp32 loop.
#include <hip/hip_runtime.h>

#include "mla_device.hpp"
#include "mla_internal.hpp"

namespace mla {

typedef __attribute__((address_space(3))) i16x4 lds_i16x4_p;
typedef __attribute__((address_space(3))) void lds_void_p;

__device__ __forceinline__ uint32_t lds_addr_of(const void* p) { return (uint32_t)(uintptr_t)(const lds_void_p*)p; }

// 16 bytes per lane HBM -> LDS bytes [dst + 16 lane, + 16) (dst wave-uniform)
__device__ __forceinline__ void dma16_lds(const void* src, lds_void_p* dst) {
  __builtin_amdgcn_global_load_lds(src, dst, 16, 0, 0);
}

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

// Piece swizzle of W tile row k (k mod 16 decides).  A transposed read covers, per 32 lanes,
// rows {0..3, 8..11} (+4 for the second half of the fragment) of a k-step and two adjacent
// pieces; these masks put the eight 32-byte row segments on eight distinct bank windows.
// (MB = 16 rows hold two pieces only: its reads take two passes.)
template <int MB>
__device__ __forceinline__ int wsw(int k) {
  if constexpr (MB == 128) return ((k & 3) << 1) | (k & 8);
  else if constexpr (MB == 64) return (k & 2) | ((k >> 1) & 4);
  else if constexpr (MB == 32) return (k >> 2) & 2;
  else return 0;
}

// grid: 8 * units_per_xcd workgroups of 256 threads; unit u = (h, column block, row block),
// row block fastest.  K % 32 == 0, K <= 32 * KSN, K * MB * 2 bytes of dynamic LDS.
template <bool XF32, int MB, int NBT, int KSN>
__global__ __launch_bounds__(256) void proj_mfma_kernel(ProjParams p, int n_mb, int n_nb, int units_per_xcd,
                                                        int total) {
  constexpr int MT = MB / 16, TILES = NBT * MT;
  constexpr int KSP = TILES >= 4 ? 1 : 4 / TILES;   // k partitions over the four waves
  constexpr int WPK = 4 / KSP;                       // waves per k partition
  constexpr int TPW = TILES / WPK;                   // output tiles per wave (all in one row tile)
  constexpr int PR = MB / 8;                         // 16-byte pieces per W tile row
  constexpr int KSW = KSN / KSP;                     // k-steps per wave, at most
  constexpr int XV = XF32 ? 2 : 1;
  constexpr int RED = (KSP - 1) * TILES * 64;
  extern __shared__ __attribute__((aligned(16))) uint8_t pj_lds[];
  __shared__ f32x4 red[RED > 0 ? RED : 1];

  const int u = (int)(blockIdx.x & 7) * units_per_xcd + (int)(blockIdx.x >> 3);
  if (u >= total) return;
  const int nb = u % n_nb, mb = (u / n_nb) % n_mb, h = u / (n_nb * n_mb);
  const int K = p.K, M = p.M, N = p.N, nks = K >> 5;
  const int m0 = mb * MB, n0 = nb * 16 * NBT;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, lr = lane & 15, lg = lane >> 4;

  // W tile -> LDS: DMA instruction j carries pieces [64 j, 64 j + 64) of the tile (row-major)
  {
    const bf16_t* Wh = (const bf16_t*)p.W + (size_t)h * K * M + m0;
    const int ninstr = (K * PR) >> 6;
    for (int j = w; j < ninstr; j += 4) {
      const int q = j * 64 + lane, k = q / PR, cp = q % PR;
      dma16_lds(Wh + (size_t)k * M + ((cp ^ wsw<MB>(k & 15)) << 3), (lds_void_p*)(pj_lds + j * 1024));
    }
  }

  // this wave's k partition, output tiles and row tile
  const int kp = w / WPK, wi = w % WPK;
  const int t0 = wi * TPW, rt = t0 / MT, mt0 = t0 % MT;
  const int n = n0 + 16 * rt + lr;
  const bool nok = n < N;
  // X fragments: row n, k = 32 ks + 8 lg .. + 7 for ks = kp, kp + KSP, ...
  u32x4 xr[KSW][XV];
  {
    const size_t xo = (size_t)(nok ? n : 0) * p.sxn + (size_t)h * p.sxh + lg * 8;
#pragma unroll
    for (int j = 0; j < KSW; ++j) {
      const int ks = kp + KSP * j;
      const bool ok = nok && ks < nks;
#pragma unroll
      for (int v = 0; v < XV; ++v) {
        if (XF32)
          xr[j][v] = ok ? *(const u32x4*)((const float*)p.X + xo + ks * 32 + 4 * v) : u32x4{0, 0, 0, 0};
        else
          xr[j][v] = ok ? *(const u32x4*)((const bf16_t*)p.X + xo + ks * 32) : u32x4{0, 0, 0, 0};
      }
    }
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // the W tile DMA (and the X fragments)
  __syncthreads();

  // transposed reads: rows k = 32 ks + 8 lg + (lr >> 2) (+4), logical piece 2 mt + (lr & 3) / 2,
  // bytes (lr & 1) * 8; the swizzle depends on k mod 16 only, so offsets are per lane
  uint32_t olo[TPW], ohi[TPW];
  {
    const uint32_t base = lds_addr_of(pj_lds);
    const int klo = 8 * lg + (lr >> 2), khi = klo + 4;
#pragma unroll
    for (int tt = 0; tt < TPW; ++tt) {
      const int c = 2 * (mt0 + tt) + ((lr & 3) >> 1);
      olo[tt] = base + klo * MB * 2 + ((c ^ wsw<MB>(klo & 15)) << 4) + (lr & 1) * 8;
      ohi[tt] = base + khi * MB * 2 + ((c ^ wsw<MB>(khi & 15)) << 4) + (lr & 1) * 8;
    }
  }
  f32x4 acc[TPW];
#pragma unroll
  for (int tt = 0; tt < TPW; ++tt) acc[tt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < KSW; ++j) {
    const int ks = kp + KSP * j;
    if (ks < nks) {
      bf16x8 bh, bl;
      if (XF32) {
        u32x4 vh, vl;
        split_hi_lo(__builtin_bit_cast(f32x4, xr[j][0]), __builtin_bit_cast(f32x4, xr[j][XV - 1]), vh, vl);
        bh = __builtin_bit_cast(bf16x8, vh);
        bl = __builtin_bit_cast(bf16x8, vl);
      } else {
        bh = __builtin_bit_cast(bf16x8, xr[j][0]);
      }
      const uint32_t kofs = (uint32_t)(ks * 32 * MB * 2);
#pragma unroll
      for (int tt = 0; tt < TPW; ++tt) {
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_p*)(uintptr_t)(olo[tt] + kofs));
        const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_p*)(uintptr_t)(ohi[tt] + kofs));
        const bf16x8 av = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        acc[tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bh, acc[tt], 0, 0, 0);
        if (XF32) acc[tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bl, acc[tt], 0, 0, 0);
      }
    }
  }

  if constexpr (KSP > 1) {
    // k partitions 1.. hand their partial sums to partition 0
    if (kp > 0) {
#pragma unroll
      for (int tt = 0; tt < TPW; ++tt) red[((kp - 1) * TILES + t0 + tt) * 64 + lane] = acc[tt];
    }
    __syncthreads();
    if (kp > 0) return;
#pragma unroll
    for (int q = 1; q < KSP; ++q)
#pragma unroll
      for (int tt = 0; tt < TPW; ++tt) acc[tt] += red[((q - 1) * TILES + t0 + tt) * 64 + lane];
  }

  // Y^T tile: this lane holds row n, columns m0 + 16 mt + 4 lg .. + 3
  if (!nok) return;
  const size_t yo = ((size_t)n * p.H + h) * M + m0 + 4 * lg;
#pragma unroll
  for (int tt = 0; tt < TPW; ++tt) {
    const int mt = mt0 + tt;
    if (p.y_f32)
      *(f32x4*)((float*)p.Y + yo + mt * 16) = acc[tt];
    else
      *(uint2*)((bf16_t*)p.Y + yo + mt * 16) =
          uint2{pack_bf16x2(acc[tt][0], acc[tt][1]), pack_bf16x2(acc[tt][2], acc[tt][3])};
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

template <bool XF32, int MB, int NBT, int KSN>
static hipError_t launch_shape(const ProjParams& p, int n_mb, int n_nb, hipStream_t st) {
  static bool attr_set = false;  // raise the dynamic-LDS limit once
  if (!attr_set) {
    const hipError_t e = hipFuncSetAttribute((const void*)proj_mfma_kernel<XF32, MB, NBT, KSN>,
                                             hipFuncAttributeMaxDynamicSharedMemorySize, 64 * 1024);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  const int total = p.H * n_mb * n_nb;
  const int per_xcd = (total + 7) / 8;
  const size_t lds = (size_t)p.K * MB * 2;
  hipLaunchKernelGGL((proj_mfma_kernel<XF32, MB, NBT, KSN>), dim3(8 * per_xcd), dim3(256), lds, st, p, n_mb, n_nb,
                     per_xcd, total);
  return hipGetLastError();
}

template <bool XF32, int NBT, int KSN>
static hipError_t launch_mb(const ProjParams& p, int mb, int n_nb, hipStream_t st) {
  const int n_mb = p.M / mb;
  switch (mb) {
    case 128: return launch_shape<XF32, 128, NBT, KSN>(p, n_mb, n_nb, st);
    case 64: return launch_shape<XF32, 64, NBT, KSN>(p, n_mb, n_nb, st);
    case 32: return launch_shape<XF32, 32, NBT, KSN>(p, n_mb, n_nb, st);
    default: return launch_shape<XF32, 16, NBT, KSN>(p, n_mb, n_nb, st);
  }
}

// Row blocks of 64 rows for N >= 64, else of 16; column block: the widest of 128/64/32/16
// dividing M whose grid still gives enough workgroups (two per CU; one per CU for fp32 X,
// which every column block re-reads) and whose W tile fits 64 KB of LDS, else the narrowest.
template <bool XF32>
static hipError_t launch_proj_mfma(const ProjParams& p, hipStream_t st) {
  const int nbt = p.N >= 64 ? 4 : 1;
  const int n_nb = (p.N + 16 * nbt - 1) / (16 * nbt);
  const int64_t want = XF32 ? 256 : 512;
  int mb = 128;
  while (mb > 16 && (p.M % mb != 0 || (int64_t)p.K * mb * 2 > 64 * 1024 || (int64_t)p.H * (p.M / mb) * n_nb < want))
    mb >>= 1;
  const bool short_k = p.K <= 128;
  if (nbt == 4)
    return short_k ? launch_mb<XF32, 4, 4>(p, mb, n_nb, st) : launch_mb<XF32, 4, 16>(p, mb, n_nb, st);
  return short_k ? launch_mb<XF32, 1, 4>(p, mb, n_nb, st) : launch_mb<XF32, 1, 16>(p, mb, n_nb, st);
}

hipError_t launch_proj(const ProjParams& p, hipStream_t st) {
  const bool mfma = p.aligned16 && !p.w_f32 && p.K % 32 == 0 && p.K <= 512 && p.M % 16 == 0 &&
                    (p.sxn % 8 == 0) && (p.sxh % 8 == 0) && (int64_t)p.H * p.M / 16 * ((p.N + 15) / 16) < (1LL << 30);
  if (mfma) return p.x_f32 ? launch_proj_mfma<true>(p, st) : launch_proj_mfma<false>(p, st);
  const size_t total = (size_t)p.N * p.H * p.M;
  hipLaunchKernelGGL(proj_f32_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, st, p);
  return hipGetLastError();
}

}  // namespace mla
