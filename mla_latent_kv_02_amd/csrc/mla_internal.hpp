// Internal interface between the libmla host layer (libmla.cpp) and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mla {

// Mixed histories in the partition kernels: partitions are cut over weighted block positions,
// a bf16 block counting kMixedBf16Weight (its rows come by DMA one step ahead of use, where a
// low-bit block's codes come four steps ahead), so the partition that holds the recent window
// takes fewer blocks.  Sequence b has nS sink, nM middle and nR recent blocks.
constexpr int kMixedBf16Weight = 2;
// The pipelined kernel keeps each block's address in 56 bits of a per-block table.
constexpr uint64_t kPipeAddrLimit = 1ULL << 56;
__host__ __device__ inline int mixed_positions(int nS, int nM, int nR) { return kMixedBf16Weight * (nS + nR) + nM; }
// the number of joint blocks whose first weighted position lies below x
__host__ __device__ inline int mixed_blocks_before(int x, int nS, int nM, int nR) {
  const int W = kMixedBf16Weight;
  const int xs = x, xm = x - W * nS, xr = x - W * nS - nM;
  const int s = xs <= 0 ? 0 : ((xs + W - 1) / W < nS ? (xs + W - 1) / W : nS);
  const int m = xm <= 0 ? 0 : (xm < nM ? xm : nM);
  const int r = xr <= 0 ? 0 : ((xr + W - 1) / W < nR ? (xr + W - 1) / W : nR);
  return s + m + r;
}

// A bf16 part of a mixed history (a sink of the earliest tokens or a recent window), decoded
// together with a low-bit middle as one sequence of blocks per batch entry.
struct MixedPart {
  const uint8_t* pool;
  int64_t num_blocks, block_bytes;
  const int32_t* block_table;
  int bt_stride;
  const int32_t* seq_lens;  // null: the part is absent (no token in any sequence)
  int max_seq_len;
};

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
  // mixed histories (decode_pipe_kernel's MIXED variant): sequence b's blocks are those of hi[0]
  // (bf16 sink), then those of the cache above (low-bit middle), then those of hi[1] (bf16
  // recent window ending with the s_q new tokens); partition c holds the joint blocks whose
  // weighted positions start in [c tpc, (c + 1) tpc)
  MixedPart hi[2];
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
                            // (its blocks are the last n_b positions before that of b + 1);
                            // [B + 2]: positions charged for a non-empty sequence's start
  // Mixed histories (decode_rows_kernel's MIXED variant): sequence b's blocks are those of
  // hi[0] (a bf16 sink), then those of the cache above (the low-bit middle), then those of
  // hi[1] (a bf16 recent window that ends with the s_q new tokens).
  MixedPart hi[2];
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
  // partition mode over mixed histories (mixed != 0): the bf16 parts' token counts (null: an
  // absent part); partitions count weighted positions (mixed_positions)
  int mixed;
  const int32_t* hi_lens[2];
  int hi_max[2];
};

// Where one decode left its split partials (a merge over several decodes reads them in place).
// Partition mode (meta == nullptr): normalised o and lse, partial c of (b, row) at row
// (b * max_chunks + c) * R + row, nch(b) = clamp(ceil(blocks(b) / tpc), 1, max_chunks).  Range
// mode: unnormalised o with inv = 1 / sum(P), pieces at rows (b + i) * R + row for b's ranges i
// (meta as the row-owner decode wrote it); a sequence without blocks has no piece.
struct CombinePart {
  const float* o;
  const float* lse;
  const float* inv;
  const int32_t* meta;
  const int32_t* seq_lens;
  int max_seq_len, max_chunks, tpc;
  int many;                 // rows usually hold more than 16 partials of this part
};

constexpr int kMaxCombineParts = 3;

struct CombinePartsParams {
  CombinePart part[kMaxCombineParts];
  int n_parts;
  int many_parts;           // some part usually holds more than 16 partials per row: wider batches
  int B, R, d_c;
  void* out;
  int out_bf16;
  float* out_lse;
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
  int family;               // quantised caches: MLA_DEQUANT_PARTITION or MLA_DEQUANT_ROWS
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

// GQLA per-group path.  Expanded pool block: G planes [64][k_nope 128 | v 128] bf16, then one
// RoPE plane [64][64] bf16.  Decode rows per unit: the group's s_q * H / G query rows.
struct GqaParams {
  const void* q_nope;       // [B][s_q][H][128] bf16
  const void* q_rope;       // [B][s_q][H][64] bf16
  const uint8_t* pool;
  int64_t num_blocks, block_bytes;
  const int32_t* block_table;
  int bt_stride;
  const int32_t* seq_lens;
  int max_seq_len;
  int B, s_q, H, G;
  int max_chunks, tpc;      // partitions per sequence (upper bound) and 64-token blocks per partition
  int total_units, units_per_xcd;
  float scale_log2;
  float* out;               // partials [B * max_chunks][s_q H][128], or out when max_chunks == 1
  float* out_lse;           // [B * max_chunks][s_q H] (may be null when writing out directly)
};

struct GqaExpandParams {
  const void* c;            // [n] rows of d_c bf16, c_stride elements apart
  const void* k;            // [n] rows of 64 bf16, k_stride elements apart
  int64_t c_stride, k_stride;
  const void* w_uk;         // [G][128][d_c] bf16
  const void* w_uv;         // [G][d_c][128] bf16
  int G, d_c;
  const int32_t* slots;
  int64_t n;
  uint8_t* pool;
  int64_t num_blocks, block_bytes;
};

hipError_t launch_gqa_expand(const GqaExpandParams& p, hipStream_t st);
hipError_t launch_gqa_decode(const GqaParams& p, int rt, hipStream_t st);

// Bytes of the per-device scratch array of mla_decode_paged_noalloc, and the device address
// of the current device's copy (looked up once per device).
constexpr size_t kNoAllocScratchBytes = (size_t)128 << 20;
hipError_t noalloc_scratch(void** ptr);

hipError_t launch_decode_mfma(const DecodeParams& p, int fmt, int rt, hipStream_t st);
hipError_t launch_decode_f32(const DecodeParams& p, hipStream_t st);
hipError_t launch_combine(const CombineParams& p, int batch, hipStream_t st);
// one log-sum-exp merge over the split partials of up to three decodes (the mixed history)
hipError_t launch_combine_parts(const CombinePartsParams& p, hipStream_t st);
hipError_t launch_decode_rows(const RowsParams& p, int fmt, hipStream_t st);
// the same kernel over mixed histories (p.hi; fmt: the middle's INT4 or INT2)
hipError_t launch_decode_rows_mixed(const RowsParams& p, int fmt, hipStream_t st);
// The pipelined partition kernel (at most 16 query rows, a quantised middle) over mixed
// histories (p.hi); pipe_mixed_fits says whether that kernel takes the middle's layout.
bool pipe_mixed_fits(int fmt, int g_lat, int g_rope);
hipError_t launch_decode_pipe_mixed(const DecodeParams& p, int fmt, hipStream_t st);
hipError_t launch_proj(const ProjParams& p, hipStream_t st);
hipError_t launch_dequant(const DequantParams& p, int fmt, hipStream_t st);
hipError_t launch_dequant_partition(const DequantParams& p, int fmt, hipStream_t st);
hipError_t launch_dequant_rows(const DequantParams& p, int fmt, hipStream_t st);
hipError_t launch_append(const AppendParams& p, hipStream_t st);
hipError_t launch_rotate(const RotateParams& p, hipStream_t st);

}  // namespace mla
