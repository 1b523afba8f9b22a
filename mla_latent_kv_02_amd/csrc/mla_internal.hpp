// Internal interface between the libmla host layer (libmla.cpp) and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mla {

// Arguments of the decode kernels, resolved by the host layer.
struct DecodeParams {
  const void* q_lat;        // [B][R][d_c]
  const void* q_rope;       // [B][R][d_r]
  int q_f32;                // q dtype is fp32 (else bf16)
  const uint8_t* pool;
  int64_t num_blocks;
  int64_t block_bytes;
  int64_t off_lc, off_ls, off_rc, off_rs;  // quantised plane offsets
  int g_lat, g_rope;        // quantisation group sizes
  const int32_t* block_table;
  int bt_stride;
  const int32_t* seq_lens;
  int max_seq_len;
  int B, s_q, H, R, RG, d_c, d_r;  // R = s_q * H rows per sequence, RG row groups
  int max_chunks, tpc;      // partitions per sequence (upper bound) and 64-token tiles per partition
  int total_units, units_per_xcd;
  float scale_log2;         // sm_scale * log2(e)
  void* out;                // partials [B*max_chunks][R][d_c] fp32, or o_lat when max_chunks == 1
  int out_bf16;
  float* out_lse;           // [B*max_chunks][R] or lse (may be null when writing o_lat directly)
};

// Arguments of the row-owner decode kernel (128 query rows per workgroup).  The batch's
// cache blocks, sequence after sequence, each non-empty sequence preceded by `phantom`
// positions that stand for the cost of starting a piece, are cut into n_ranges equal ranges;
// workgroup (range i, row group r) attends its rows over the blocks of range i.  Every piece (the
// blocks of one sequence inside one range) leaves a partial in slot b + i: o unnormalised,
// 1 / sum(P) and lse; the combine normalises and merges.  Empty sequences are written to
// out/out_lse directly.
struct RowsParams {
  const void* q_lat;        // [B][R][512]
  const void* q_rope;       // [B][R][64]
  int q_f32;
  const uint8_t* pool;
  int64_t num_blocks;
  int64_t block_bytes;
  int64_t off_lc, off_ls, off_rc, off_rs;
  int g_lat_log2, g_rope_log2;  // quantisation group sizes (powers of two: they divide 512 and 64)
  const int32_t* block_table;
  int bt_stride;
  const int32_t* seq_lens;
  int max_seq_len;
  int B, s_q, H, R, RG;
  int n_ranges, units_per_xcd, total_units;
  int phantom;              // block-space positions charged for each non-empty sequence's start
  float scale_log2;
  void* out;                // o_lat [B][R][512]
  int out_bf16;
  float* out_lse;           // [B][R], may be null
  float* part_o;            // [B + n_ranges - 1][R][512]
  float* part_lse;          // [B + n_ranges - 1][R]
  float* part_inv;          // [B + n_ranges - 1][R]
  int32_t* meta;            // [0]: positions per range; [1 + b]: first position of sequence b, b <= B
                            // (its blocks are the last n_b positions before that of b + 1)
};

// Combine of split partials.  Chunk-major mode: the parts of a decode over several caches.
// Partition mode (meta == null): max_chunks partitions of tpc
// blocks per sequence, slot b * max_chunks + c, o normalised.  Range mode: pieces of the
// ranges in meta, slots b + i, o unnormalised with its factor in part_inv; every non-empty
// sequence is combined (one piece included).
struct CombineParams {
  const float* part_o;
  const float* part_lse;
  const float* part_inv;    // range mode only
  const int32_t* seq_lens;
  int max_seq_len;
  int R, d_c, max_chunks, tpc;
  const int32_t* meta;
  void* out;
  int out_bf16;
  float* out_lse;
  int many_parts;           // rows usually hold more than 16 partials: wider load batches
  int chunk_major;          // max_chunks normalised partials per (b, row) at rows (c * B + b) * R + r
  int B;                    // batch (chunk-major mode)
};

struct ProjParams {
  const void* X;            // element (n, h, k) at X[n*sxn + h*sxh + k]
  int64_t sxn, sxh;
  int x_f32;
  const void* W;            // [H][K][M]
  int w_f32;
  void* Y;                  // [N][H][M]
  int y_f32;
  int N, H, K, M;
  int aligned16;            // X, W and Y base addresses are 16-byte aligned
};

struct DequantParams {
  const uint8_t* pool;
  int64_t num_blocks, block_bytes;
  int64_t off_lc, off_ls, off_rc, off_rs;
  int g_lat, g_rope;
  int d_c, d_r;
  const int32_t* ids;
  int n;
  uint16_t* out;            // [n][64][d_c + d_r] bf16 bits
};

// Cache writer: token i (of n) goes to slot slots[i] = block * 64 + position; slots outside
// [0, num_blocks * 64) are skipped.  c / k rows of d_c / d_r values, c_stride / k_stride
// elements apart, fp32 (in_f32) or bf16.
struct AppendParams {
  const void* c;
  const void* k;
  int in_f32;
  int64_t c_stride, k_stride;
  const int32_t* slots;
  int64_t n;
  uint8_t* pool;
  int64_t num_blocks, block_bytes;
  int64_t off_lc, off_ls, off_rc, off_rs;
  int d_c, d_r, g_lat, g_rope;
  int fmt_lat, fmt_rope;    // MLA_FMT_*
};

// In-place rotation x <- x . H_d / sqrt(d) of n_vec = n_outer * n_inner vectors: vector
// v = o * n_inner + i starts at x + o * outer_stride + i * inner_stride, element k at
// + k * elem_stride (elements of the dtype).  vecs_per_group * d <= 4096.
struct RotateParams {
  void* x;
  int f32;
  int d, log2d;
  int64_t elem_stride;
  int64_t n_inner, inner_stride, outer_stride;
  int64_t n_vec;
  int vecs_per_group;
  float scale;
  int vec8;                 // unit stride, 16-byte-aligned groups of 8: vector path
};

hipError_t launch_decode_mfma(const DecodeParams& p, int fmt, int rt, hipStream_t st);
hipError_t launch_decode_f32(const DecodeParams& p, hipStream_t st);
hipError_t launch_combine(const CombineParams& p, int batch, hipStream_t st);
hipError_t launch_decode_rows(const RowsParams& p, int fmt, hipStream_t st);
hipError_t launch_proj(const ProjParams& p, hipStream_t st);
hipError_t launch_dequant(const DequantParams& p, int fmt, hipStream_t st);
hipError_t launch_append(const AppendParams& p, hipStream_t st);
hipError_t launch_rotate(const RotateParams& p, hipStream_t st);

}  // namespace mla
