// mla_dequant_blocks: materialise cache blocks as bf16 (test/debug).  Quantised caches run the
// in-loop dequantisation of one of the decode kernel families (their own DMA producer and
// dequant routine, launched by launch_dequant_partition / launch_dequant_rows in the decode
// files), so the values are the ones that family's attention loop consumes.  Float caches
// need no unpacking: bf16 rows are what the decode copies into LDS; fp32 rows are rounded.
#include <hip/hip_runtime.h>

#include "libmla.h"
#include "mla_device.hpp"
#include "mla_internal.hpp"

namespace mla {

// Float caches of any width: bf16 rows copied, fp32 rows rounded to bf16 (ties to even);
// block ids outside the pool give zero rows.
template <bool F32>
__global__ __launch_bounds__(256) void dequant_float_kernel(DequantParams p) {
  const int k = blockIdx.x;
  const int id = p.ids[k];
  const bool ok = id >= 0 && (int64_t)id < p.num_blocks;
  const int dk = p.d_c + p.d_r;
  const uint8_t* blk = p.pool + (size_t)(ok ? id : 0) * (size_t)p.block_bytes;
  uint16_t* out = p.out + (size_t)k * BLOCK_TOKENS * dk;
  for (int i = threadIdx.x; i < BLOCK_TOKENS * dk; i += 256) {
    uint16_t v = 0;
    if (ok) v = F32 ? (uint16_t)f32_to_bf16_bits(((const float*)blk)[i]) : ((const uint16_t*)blk)[i];
    out[i] = v;
  }
}

hipError_t launch_dequant(const DequantParams& p, int fmt, hipStream_t st) {
  switch (fmt) {
    case FMT_F32: hipLaunchKernelGGL(dequant_float_kernel<true>, dim3(p.n), dim3(256), 0, st, p); break;
    case FMT_BF16: hipLaunchKernelGGL(dequant_float_kernel<false>, dim3(p.n), dim3(256), 0, st, p); break;
    case FMT_INT4:
    case FMT_INT2:
      return p.family == MLA_DEQUANT_ROWS ? launch_dequant_rows(p, fmt, st) : launch_dequant_partition(p, fmt, st);
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace mla
