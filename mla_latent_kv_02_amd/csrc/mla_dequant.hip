// mla_dequant_blocks: materialise cache blocks as bf16 with the decode kernel's own tile
// reader (TileReader in mla_device.hpp), so the values are bit-identical to the ones the
// attention loop consumes.  Used to test the in-kernel dequantisation exactly.
#include <hip/hip_runtime.h>

#include "mla_device.hpp"
#include "mla_internal.hpp"

namespace mla {

template <int FMT>
__global__ __launch_bounds__(256) void dequant_blocks_kernel(DequantParams p) {
  const int k = blockIdx.x;
  const int id = p.ids[k];
  const bool ok = id >= 0 && (int64_t)id < p.num_blocks;
  const uint8_t* blk = p.pool + (size_t)(ok ? id : 0) * (size_t)p.block_bytes;
  const int valid = ok ? BLOCK_TOKENS : 0;
  const QuantPlanes pl{(int)p.off_lc, (int)p.off_ls, (int)p.off_rc, (int)p.off_rs};
  TileReader<FMT, 256> rd;
  rd.load(blk, valid, threadIdx.x, pl, p.g_lat, p.g_rope);
  uint16_t* out = p.out + (size_t)k * BLOCK_TOKENS * 576;
  rd.emit([&](int tok, int col8, u32x4 v) { *(u32x4*)(out + tok * 576 + col8 * 8) = v; }, valid, threadIdx.x);
}

// fp32 caches of any width: round each value to bf16 (ties to even).
__global__ __launch_bounds__(256) void dequant_f32_kernel(DequantParams p) {
  const int k = blockIdx.x;
  const int id = p.ids[k];
  const bool ok = id >= 0 && (int64_t)id < p.num_blocks;
  const int dk = p.d_c + p.d_r;
  const float* blk = (const float*)(p.pool + (size_t)(ok ? id : 0) * (size_t)p.block_bytes);
  uint16_t* out = p.out + (size_t)k * BLOCK_TOKENS * dk;
  for (int i = threadIdx.x; i < BLOCK_TOKENS * dk; i += 256) out[i] = ok ? (uint16_t)f32_to_bf16_bits(blk[i]) : 0;
}

hipError_t launch_dequant(const DequantParams& p, int fmt, hipStream_t st) {
  switch (fmt) {
    case FMT_BF16: hipLaunchKernelGGL(dequant_blocks_kernel<FMT_BF16>, dim3(p.n), dim3(256), 0, st, p); break;
    case FMT_INT4: hipLaunchKernelGGL(dequant_blocks_kernel<FMT_INT4>, dim3(p.n), dim3(256), 0, st, p); break;
    case FMT_INT2: hipLaunchKernelGGL(dequant_blocks_kernel<FMT_INT2>, dim3(p.n), dim3(256), 0, st, p); break;
    case FMT_F32: hipLaunchKernelGGL(dequant_f32_kernel, dim3(p.n), dim3(256), 0, st, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace mla
