// Fixed orthogonal rotation of vectors: x <- x . H_d / sqrt(d), H_d the Sylvester-ordered
// Walsh-Hadamard matrix (H_d[i][j] = (-1)^popcount(i & j)), in place.
//
// The rotation is data-free and, being orthogonal, can be folded into the weights around the
// cached latent without changing any full-precision result (q_lat . c = (q_lat R).(c R),
// o_lat W_UV = (o_lat R)(R^T W_UV)); it spreads a few large channels over all of them before
// low-bit quantisation.  The pages' baselines include MLA adaptations of fixed rotations with
// the same quantiser (QuantMLA podcast page, comparison part), and QuantMLA's own transforms
// are fused into the model offline (QuantMLA English abstract).
//
// Vector (o, i) starts at x + o * outer_stride + i * inner_stride and its element k sits
// k * elem_stride further on: rows of W_UK [H][d_n][d_c] (elem_stride 1), columns of
// W_UV [H][d_c][d_v] (elem_stride d_v), latent rows of a token batch, or the pairs of the
// RoPE key (d = 2).  A workgroup holds 2048 elements (or one vector of up to 4096) in LDS as
// fp32 and runs the log2(d) butterfly stages there; bf16 vectors are rounded once at the end.
// Unit-stride vectors with 16-byte-aligned groups of 8 (the host checks) move as 16-byte
// accesses, 8 consecutive elements per lane, whose first three stages (pairs 1, 2 and 4
// apart) stay in registers.
#include <hip/hip_runtime.h>

#include "mla_device.hpp"
#include "mla_internal.hpp"

namespace mla {
namespace {

constexpr int kThreads = 256;
constexpr int kMaxElems = 4096;

__global__ __launch_bounds__(kThreads) void hadamard_kernel(RotateParams p) {
  __shared__ float buf[kMaxElems];
  const int tid = threadIdx.x;
  const int d = p.d, log2d = p.log2d;
  const int per = p.vecs_per_group;            // vectors in this workgroup's buffer
  const int64_t v0 = (int64_t)blockIdx.x * per;
  const int nel = per * d;
  auto addr = [&](int64_t v, int k) -> int64_t {
    const int64_t o = v / p.n_inner, i = v % p.n_inner;
    return o * p.outer_stride + i * p.inner_stride + (int64_t)k * p.elem_stride;
  };
  // pairs (j, j + h), h = 1, 2, 4, inside 8 registers
  auto bfly8 = [](float r[8]) {
#pragma unroll
    for (int h = 1; h < 8; h <<= 1)
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if ((j & h) == 0) {
          const float a = r[j], b = r[j + h];
          r[j] = a + b;
          r[j + h] = a - b;
        }
  };
  const int s0 = p.vec8 ? 3 : 0;   // stages already done in registers
  if (p.vec8) {
    for (int e0 = 8 * tid; e0 < nel; e0 += 8 * kThreads) {
      const int64_t v = v0 + e0 / d;
      float r[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
      if (v < p.n_vec) {
        const int64_t a = addr(v, e0 % d);
        if (p.f32) {
          const f32x4 lo = *(const f32x4*)((const float*)p.x + a), hi = *(const f32x4*)((const float*)p.x + a + 4);
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            r[j] = lo[j];
            r[4 + j] = hi[j];
          }
        } else {
          const u32x4 w = *(const u32x4*)((const uint16_t*)p.x + a);
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            r[2 * j] = __uint_as_float(w[j] << 16);
            r[2 * j + 1] = __uint_as_float(w[j] & 0xFFFF0000u);
          }
        }
      }
      bfly8(r);
#pragma unroll
      for (int j = 0; j < 8; ++j) buf[e0 + j] = r[j];
    }
  }
  for (int e = tid; e < nel && !p.vec8; e += kThreads) {
    const int64_t v = v0 + e / d;
    float x = 0.f;
    if (v < p.n_vec) {
      const int64_t a = addr(v, e % d);
      x = p.f32 ? ((const float*)p.x)[a] : __uint_as_float((uint32_t)((const uint16_t*)p.x)[a] << 16);
    }
    buf[e] = x;
  }
  __syncthreads();
  // stage h: pairs (j, j + h) with j & h == 0 inside each vector
  for (int s = s0; s < log2d; ++s) {
    const int h = 1 << s;
    for (int q = tid; q < nel / 2; q += kThreads) {
      const int j = ((q >> s) << (s + 1)) | (q & (h - 1));
      const float a = buf[j], b = buf[j + h];
      buf[j] = a + b;
      buf[j + h] = a - b;
    }
    __syncthreads();
  }
  const float scale = p.scale;
  if (p.vec8) {
    for (int e0 = 8 * tid; e0 < nel; e0 += 8 * kThreads) {
      const int64_t v = v0 + e0 / d;
      if (v >= p.n_vec) continue;
      const int64_t a = addr(v, e0 % d);
      float r[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) r[j] = buf[e0 + j] * scale;
      if (p.f32) {
        *(f32x4*)((float*)p.x + a) = f32x4{r[0], r[1], r[2], r[3]};
        *(f32x4*)((float*)p.x + a + 4) = f32x4{r[4], r[5], r[6], r[7]};
      } else {
        *(u32x4*)((uint16_t*)p.x + a) = u32x4{pack_bf16x2(r[0], r[1]), pack_bf16x2(r[2], r[3]),
                                              pack_bf16x2(r[4], r[5]), pack_bf16x2(r[6], r[7])};
      }
    }
    return;
  }
  for (int e = tid; e < nel; e += kThreads) {
    const int64_t v = v0 + e / d;
    if (v >= p.n_vec) continue;
    const int64_t a = addr(v, e % d);
    const float y = buf[e] * scale;
    if (p.f32) ((float*)p.x)[a] = y;
    else ((uint16_t*)p.x)[a] = (uint16_t)f32_to_bf16_bits(y);
  }
}

}  // namespace

hipError_t launch_rotate(const RotateParams& p, hipStream_t st) {
  if (p.n_vec <= 0) return hipSuccess;
  const int64_t groups = (p.n_vec + p.vecs_per_group - 1) / p.vecs_per_group;
  hipLaunchKernelGGL(hadamard_kernel, dim3((unsigned)groups), dim3(kThreads), 0, st, p);
  return hipGetLastError();
}

}  // namespace mla
