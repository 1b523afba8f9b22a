// LDS stage layout and synchronisation helpers shared by the decode kernels (gfx950).
//
// A bf16 stage holds 32 tokens x 576 columns ([c (512) | k_rope (64)]) as 72 pieces of
// 8 bf16 per token; piece c of token t sits at physical piece c ^ sw(t).  Rows are 288
// dwords apart (32 mod 64 banks).  Timing probes on gfx950 show that a 16-byte LDS access is
// served 16 lanes per cycle, a lane set being (lane bit 5, parity of lane bits 2..4), and a
// ds_read_b64_tr_b16 32 consecutive lanes per cycle, over 64 four-byte banks; sw() makes the
// score operand reads, the transposed P.C operand reads and the dequantised piece stores of
// the decode kernels fill 64 distinct banks per cycle.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mla_device.hpp"

namespace mla {

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr int ST_TOK = 32;              // tokens per stage (half a paged block)
constexpr int ST_ELEMS = ST_TOK * 576;  // bf16 elements per stage
constexpr float RESCALE_SLACK = 8.f;    // log2 headroom of P before the running maximum moves

__device__ __forceinline__ int sw(int t) { return (t & 2) | ((t >> 1) & 4) | ((t >> 4) & 1); }

// bf16 element offset of (token t, latent/rope column d) in a stage
__device__ __forceinline__ int st_off(int t, int d) { return t * 576 + (((d >> 3) ^ sw(t)) << 3) + (d & 7); }

// Code stage of a quantised cache: the four code planes of a half block copied as they lie in
// the block, token-major: latent codes [32][LB], latent scales [32][groups] (4 bytes each), RoPE
// codes [32][32], RoPE scales [32][rgroups].
//
// Dequantisation tasks of a code stage.  Latent task k (0..511) is 32-element chunk kk of token
// t, RoPE task r (0..255) is the 8-element piece ri of token t.  Each aligned block of 64 tasks
// (one wavefront instruction) reads its codes and writes its bf16 pieces on 64 distinct banks
// per cycle under the lane sets above: a latent block covers the tokens {T, T^2, T^17, T^19}
// with all 16 chunks each (lanes 4m .. 4m + 3 read 64 consecutive code bytes), a RoPE block 8
// consecutive tokens with all 8 pieces each.
__device__ __forceinline__ void lat_task(int k, int& t, int& kk) {
  const int l = k & 63, blk = k >> 6, tau = (l >> 2) & 3;
  t = ((blk & 1) | ((blk & 6) << 1)) ^ ((tau & 1) << 1) ^ ((tau >> 1) * 17);
  kk = (l & 3) | ((((l >> 4) & 3) ^ (((l >> 2) & 1) * 3)) << 2);
}
__device__ __forceinline__ void rope_task(int r, int& t, int& ri) {
  const int l = r & 63;
  t = (r >> 6) * 8 + (l & 3) + ((l >> 5) << 2);
  ri = (l >> 2) & 7;
}

// s_waitcnt immediate: wait until at most n vector-memory operations are outstanding
__host__ __device__ constexpr int vmcnt_imm(int n) { return (n & 0xF) | ((n >> 4) << 14) | (7 << 4) | (0xF << 8); }

// All LDS traffic of this wave is complete, then workgroup barrier.  The memory
// clobber keeps the compiler from moving memory operations across it, without
// the release fence that would also wait for the in-flight LDS DMA of later stages.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

}  // namespace mla
