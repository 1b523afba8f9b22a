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
  for (int e = tid; e < nel; e += kThreads) {
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
  for (int s = 0; s < log2d; ++s) {
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
