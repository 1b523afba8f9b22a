/*
 * libmla — Multi-Head Latent Attention decode over a paged latent KV cache,
 * for AMD Instinct MI355X (gfx950).
 *
 * What the library computes.  MLA keeps one compressed latent vector c_KV per
 * cached token plus a narrow, separately rotated RoPE key; at decode time the
 * latent is up-projected into per-head keys and values (RAQ-MLA abstract,
 * searcharxiv "Linchuan Xie" author page).  Because the key up-projection can
 * be folded into the query, every head can score the same shared latent: the
 * absorbed MQA decoding path (GQLA abstract, thelatestinai.com paper-cards
 * page).  One decode step is therefore three calls:
 *
 *   mla_absorb_q      q_lat[n,h,:] = q_nope[n,h,:] . W_UK[h]             (fold W_UK into q)
 *   mla_decode_paged  s_t = sm_scale (q_lat . c_t + q_rope . k_rope_t),
 *                     o_lat = softmax(s) . c  over the paged cache       (shared-latent attention)
 *   mla_out_proj      out[n,h,:] = o_lat[n,h,:] . W_UV[h]                (up-project to values)
 *
 * The cache may hold bf16/fp32 values or low-bit codes (INT4 latent + INT4
 * RoPE key, or INT2 latent + INT4 RoPE key) which are unpacked and
 * dequantised inside the attention loop, without a full-precision copy of the
 * history (QuantMLA English abstract, arxivdaily QuantMLA page; cache-layout
 * part of the QuantMLA podcast page).  Decoding with two query tokens per
 * sequence (s_q = 2, causal within the pair) is supported, the multi-token
 * prediction case named in the GQLA abstract.
 *
 * Conventions
 *   - Row-major, densely packed tensors unless a stride argument says otherwise.
 *   - W_UK is [H][d_n][d_c] (k_nope = W_UK[h] c); W_UV is [H][d_c][d_v].
 *   - seq_lens[b] counts every cached token of sequence b INCLUDING its s_q new
 *     query tokens; query i (0-based) attends cached tokens 0 .. L_b - s_q + i.
 *   - lse is the natural logarithm of the softmax denominator of the scaled scores.
 *
 * Ownership and streams
 *   The caller owns all memory (device pointers unless stated).  libmla never
 *   calls an allocator, frees or keeps pointers after a call returns.  Every compute call
 *   is asynchronous on the caller's stream (a hipStream_t passed as void*, NULL =
 *   the null stream); buffers must stay valid until that stream has completed.
 *   The only process-wide state is a cached per-device CU count, and the per-device scratch
 *   array (and its looked-up address) of mla_decode_paged_noalloc.
 *
 * Errors
 *   Every entry point returns an mla_status (int32_t).  Arguments are validated
 *   on the host before anything is launched, so a call that fails validation
 *   has launched nothing and touched no device.  No C++ exception crosses the ABI.
 */
#ifndef LIBMLA_H
#define LIBMLA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MLA_ABI_VERSION 2

/* Status codes. */
#define MLA_OK 0
#define MLA_ERR_INVALID_ARG 1  /* null pointer, non-positive size, bad enum, misaligned pointer, seq too short */
#define MLA_ERR_UNSUPPORTED 2  /* valid combination for which no kernel exists (e.g. bf16 cache with d_c != 512) */
#define MLA_ERR_WORKSPACE 3    /* workspace missing or smaller than mla_decode_workspace_size() */
#define MLA_ERR_HIP 4          /* a HIP runtime call or kernel launch failed */

/* Element types of q / weights / outputs. */
#define MLA_F32 0
#define MLA_BF16 1

/* Cache element formats. */
#define MLA_FMT_F32 0
#define MLA_FMT_BF16 1
#define MLA_FMT_INT4 2  /* 2 codes per byte; element 2j in the low nibble of byte j */
#define MLA_FMT_INT2 3  /* 4 codes per byte; element 4j+k in bits 2k..2k+1 of byte j */

/*
 * Paged-cache descriptor.  A block holds block_size (= 64) consecutive tokens
 * of one sequence.
 *   Float formats (latent_fmt == rope_fmt, F32 or BF16): one plane of rows
 *     [c (d_c values) | k_rope (d_r values)] per token, block = 64 rows.
 *   Quantised formats: four planes per block, each starting 16-byte aligned:
 *     latent codes [64][d_c*bits/8] | latent (scale, zero) fp16 pairs [64][d_c/latent_group][2] |
 *     rope codes   [64][d_r*bits/8] | rope   (scale, zero) fp16 pairs [64][d_r/rope_group][2].
 *   A quantised element dequantises to RNE_bf16((code - zero) * scale), with an
 *   integer-valued fp16 zero-point and an fp16 scale per (token, group).
 */
typedef struct mla_cache_desc {
  int32_t d_c;          /* latent width */
  int32_t d_r;          /* RoPE key width */
  int32_t block_size;   /* tokens per block; must be 64 */
  int32_t latent_fmt;   /* MLA_FMT_* */
  int32_t rope_fmt;     /* MLA_FMT_*; BF16/F32 must match latent_fmt; INT4 with a quantised latent */
  int32_t latent_group; /* channels per scale/zero group of the latent (quantised only) */
  int32_t rope_group;   /* channels per scale/zero group of the RoPE key (quantised only) */
} mla_cache_desc;

/* Bytes of one block for this descriptor, or -1 if the descriptor is invalid. */
int64_t mla_cache_block_bytes(const mla_cache_desc* desc);

/* Byte offsets of the four planes (latent codes, latent scale/zero, rope codes, rope
 * scale/zero) inside a block; float formats report {0, -1, -1, -1}. */
int32_t mla_cache_plane_offsets(const mla_cache_desc* desc, int64_t offsets[4]);

/*
 * mla_absorb_q: fold W_UK into the query (the absorbed MQA form, GQLA abstract).
 *   q_lat[n][h][:] = sum_i q_nope[n, h, i] * W_UK[h][i][:]          (fp32 accumulation)
 *   q_nope element (n, h, i) is at q_nope[n*q_stride_n + h*q_stride_h + i] (elements).
 *   w_uk [H][d_n][d_c] of w_dtype; q_lat [N][H][d_c] of out_dtype (dense).
 *   dtypes: q, w, out in {MLA_F32, MLA_BF16}.  bf16 weights use the MFMA kernel when
 *   d_n % 32 == 0 and d_c % 64 == 0; every other combination runs a plain fp32 kernel.
 */
int32_t mla_absorb_q(const void* q_nope, int64_t q_stride_n, int64_t q_stride_h, int32_t q_dtype,
                     const void* w_uk, int32_t w_dtype, void* q_lat, int32_t out_dtype, int32_t N,
                     int32_t H, int32_t d_n, int32_t d_c, void* stream);

/* Arguments of mla_decode_paged.  Every pointer is a device pointer except the struct itself. */
typedef struct mla_decode_args {
  const void* q_lat;          /* [batch][s_q][H][d_c], q_dtype; 16-byte aligned */
  const void* q_rope;         /* [batch][s_q][H][d_r], q_dtype, already rotated */
  int32_t q_dtype;            /* MLA_BF16 (bf16/quantised caches) or MLA_F32 (fp32 cache) */
  const void* cache_pool;     /* num_blocks blocks of mla_cache_block_bytes(&cache) bytes, 16-byte aligned */
  int64_t num_blocks;
  mla_cache_desc cache;
  const int32_t* block_table; /* [batch][block_table_stride]; entries of the first ceil(L_b/64) slots are used */
  int32_t block_table_stride; /* >= ceil(max_seq_len / 64) */
  const int32_t* seq_lens;    /* [batch], each in [s_q, max_seq_len] */
  int32_t max_seq_len;        /* host-side upper bound of seq_lens, used to plan the split */
  int64_t total_seq_len;      /* optional host-side sum of seq_lens (0 = unknown); balances the plan for ragged batches */
  int32_t batch;
  int32_t s_q;                /* 1 or 2 */
  int32_t num_heads;
  float sm_scale;             /* score scale, e.g. 1/sqrt(d_n + d_r) */
  int32_t num_splits;         /* fewer than 96 rows (s_q * H): context partitions per longest
                                 sequence; 96 or more rows: num_splits * batch block ranges.
                                 0 = automatic */
  void* o_lat;                /* [batch][s_q][H][d_c] of o_dtype */
  int32_t o_dtype;            /* MLA_F32 or MLA_BF16 */
  float* lse;                 /* [batch][s_q][H] natural-log LSE, or NULL */
  void* workspace;            /* scratch for split partials, >= mla_decode_workspace_size() bytes */
  size_t workspace_bytes;
} mla_decode_args;

/* Workspace needed by mla_decode_paged for these arguments: 0 for fewer than 96 query rows
 * per sequence when the plan uses no split; 96 rows or more always need one (every piece of
 * a sequence is written there unnormalised and merged by a second kernel).
 * Device memory, 256-byte aligned, owned by the caller; its contents need no initialisation
 * and are scratch between calls (calls that overlap on one workspace race). */
int32_t mla_decode_workspace_size(const mla_decode_args* args, size_t* bytes);

/* The same size for the plan made for num_cus compute units (0 = the current device).  With
 * num_cus > 0, or an explicit num_splits, this is pure host logic and touches no device.  The
 * size is that of the split partials, O(batch + ranges) x s_q x H x d_c fp32 values, and does
 * not grow with the context while the batch's blocks fit one round of ranges (at most 256
 * blocks per range); it is never a copy of the cached history. */
int32_t mla_decode_workspace_size_for(const mla_decode_args* args, int32_t num_cus, size_t* bytes);

/* The work split mla_decode_paged will use.  Fewer than 96 query rows per sequence
 * (s_q * num_heads): *num_splits partitions of the longest sequence of *tiles_per_split
 * 64-token blocks each.  96 rows or more: the batch's blocks, sequence after sequence, each
 * non-empty sequence counted with 3 extra positions for the cost of starting it (none when
 * every sequence already starts on a range boundary), cut into
 * *num_splits equal ranges (one workgroup per range and 128-row group) of at most
 * *tiles_per_split positions.  num_cus = compute units to plan for (0 = query the current
 * device).  Pure host logic. */
int32_t mla_decode_plan(const mla_decode_args* args, int32_t num_cus, int32_t* num_splits,
                        int32_t* tiles_per_split);

/*
 * mla_decode_paged: attention of the absorbed queries over the shared latent.
 *   For sequence b, query i < s_q, head h, over cached tokens t <= L_b - s_q + i:
 *     s_t  = sm_scale * (q_lat[b,i,h] . c_t + q_rope[b,i,h] . k_rope_t)
 *     o_lat[b,i,h] = sum_t softmax(s)_t c_t,   lse[b,i,h] = log sum_t exp(s_t)
 *   c_t and k_rope_t are read through block_table from the pool, dequantised in the
 *   kernel for INT4/INT2 caches.  Cache slots past L_b in a sequence's last block are
 *   never used.  Long contexts are split into partitions whose partial (o, lse) are
 *   merged by a log-sum-exp combine; the result is deterministic for fixed arguments.
 *   Block-table entries outside [0, num_blocks) are not dereferenced: their tokens take
 *   no part in the softmax.  seq_lens above max_seq_len are clamped to it; a sequence of
 *   length 0 gets o_lat = 0 and lse = -inf.
 *   Kernels: bf16 MFMA for BF16/INT4/INT2 caches with d_c = 512, d_r = 64; a plain
 *   fp32 kernel for F32 caches (d_c <= 1024, d_r <= 256).
 */
int32_t mla_decode_paged(const mla_decode_args* args, void* stream);

/*
 * mla_decode_paged_noalloc: mla_decode_paged that allocates nothing and takes no workspace, for
 *   callers that cannot allocate device memory (code under HIP graph capture, tight serving
 *   loops, harnesses that forbid allocation).  args->workspace and args->workspace_bytes are
 *   ignored: the split partials go to a scratch array of 128 MiB that the library holds on each
 *   device it runs on until the process ends (its address is looked up on the first call on a
 *   device).  A call whose partials need more than that (mla_decode_workspace_size() above
 *   128 MiB, e.g. 256 query rows per sequence over a V3-sized batch) returns MLA_ERR_WORKSPACE
 *   and launches nothing.  Every call on a device shares that device's array and leaves its
 *   contents behind: calls that overlap on one device (two streams, two threads) race.  Same
 *   results, bit for bit, as mla_decode_paged with the same arguments.
 */
int32_t mla_decode_paged_noalloc(const mla_decode_args* args, void* stream);

/*
 * mla_decode_mixed: one decode over a history kept at two precisions, the deployed policy of
 *   the QuantMLA cache layout (earliest tokens and a recent window kept in BF16, the tokens
 *   between them low-bit: QuantMLA podcast page, cache-layout part).  Sequence b's history is
 *   sink_b ++ middle_b ++ recent_b; each part is a paged cache of its own, described by an
 *   mla_decode_args whose cache, pool, block table, seq_lens (that part's token counts) and
 *   max_seq_len are used; q_lat, q_rope, q_dtype, batch, s_q, num_heads, sm_scale and the
 *   cache widths must be the same in every part (else MLA_ERR_INVALID_ARG), and num_splits
 *   applies per part; o_lat, o_dtype, lse and workspace of the parts are ignored.  Any part
 *   may be NULL (absent); at least one must be given, and with s_q = 2 the recent part must be
 *   (it holds the two new tokens, else MLA_ERR_INVALID_ARG).  The recent part ends with the s_q new
 *   tokens and carries the causal mask (query i sees its tokens 0 .. L - s_q + i); every query
 *   sees all sink and middle tokens (the sink and the recent window may also share one
 *   cache, passed as the recent part with no sink part: the attention does not depend on
 *   token order apart from that mask).  With a low-bit middle and bf16 sink and recent parts
 *   (the deployed policy), one decode streams each sequence's blocks of all three caches in
 *   one loop (bf16 blocks copied into the stage where low-bit blocks are dequantised) and
 *   merges its split partials; other combinations decode each part into fp32 partials and
 *   merge the parts by log-sum-exp.  Either way the result is the attention over the
 *   concatenated history, up to rounding: o_lat [batch][s_q][H][d_c] of o_dtype, lse
 *   [batch][s_q][H] or NULL.  A part
 *   with no token for a sequence contributes nothing; a sequence with no token at all gets
 *   o_lat = 0 and lse = -inf.  workspace: >= mla_decode_mixed_workspace_size() bytes,
 *   256-byte aligned, scratch.
 */
int32_t mla_decode_mixed(const mla_decode_args* sink, const mla_decode_args* middle, const mla_decode_args* recent,
                         void* o_lat, int32_t o_dtype, float* lse, void* workspace, size_t workspace_bytes,
                         void* stream);
int32_t mla_decode_mixed_workspace_size(const mla_decode_args* sink, const mla_decode_args* middle,
                                        const mla_decode_args* recent, size_t* bytes);

/*
 * mla_out_proj: up-project the latent attention output (W_UV, RAQ-MLA abstract).
 *   out[n][h][:] = sum_j o_lat[n, h, j] * W_UV[h][j][:]      (fp32 accumulation)
 *   o_lat element (n, h, j) at o_lat[n*o_stride_n + h*o_stride_h + j]; w_uv [H][d_c][d_v];
 *   out [N][H][d_v] dense.  fp32 o_lat with bf16 weights is split into two bf16 terms
 *   (hi + lo) for the MFMA so the product keeps fp32-level accuracy.
 */
int32_t mla_out_proj(const void* o_lat, int64_t o_stride_n, int64_t o_stride_h, int32_t o_dtype,
                     const void* w_uv, int32_t w_dtype, void* out, int32_t out_dtype, int32_t N,
                     int32_t H, int32_t d_c, int32_t d_v, void* stream);

/*
 * mla_append_kv: write n new tokens (their latent c_KV and RoPE key) into their slots of a
 *   paged cache, the step before decode that fills the cache the decode reads.
 *   Token i: c_new[i * c_stride + 0 .. d_c) and k_rope_new[i * k_stride + 0 .. d_r), both of
 *   in_dtype (MLA_F32 or MLA_BF16; the RoPE key already rotated), go to slot slots[i] =
 *   block * 64 + position of cache_pool (num_blocks blocks laid out as desc says; slots is
 *   int32 on the device).  Slots outside [0, num_blocks * 64) are skipped (padding); two
 *   tokens with the same slot in one call race.  Nothing else in the pool is written.
 *   Float caches store the values (fp32) or their bf16 rounding (ties to even).  Quantised
 *   caches store codes of the plain round-to-nearest asymmetric quantiser, per token and per
 *   group of channels (the latent at INT4 or INT2 with an INT4 RoPE key: QuantMLA English
 *   abstract, arxivdaily QuantMLA page; round-to-nearest as the plain quantiser: QuantMLA
 *   podcast page, comparison part), computed in float64 from the exact inputs:
 *     s = fp16((max - min) / (2^b - 1)), 1 where that is 0 (ties to even);
 *     z = clamp(rint(-min / s), 0, 2^b - 1), stored as fp16 (+0 when zero);
 *     code = clamp(rint(x / s) + z, 0, 2^b - 1),  rint ties to even,
 *   so that the decode reads back RNE_bf16((code - z) * s).  Inputs must be finite.
 *   Quantised formats need d_c, d_r and both group sizes to be multiples of 8 with
 *   group / 8 a power of two <= 64 (else MLA_ERR_UNSUPPORTED).  n = 0 is a no-op.
 */
int32_t mla_append_kv(const void* c_new, int64_t c_stride, const void* k_rope_new, int64_t k_stride,
                      int32_t in_dtype, const int32_t* slots, int64_t n, void* cache_pool, int64_t num_blocks,
                      const mla_cache_desc* desc, void* stream);

/*
 * mla_hadamard_rotate: in place, x <- x . H_d / sqrt(d) for a set of vectors, H_d the
 *   Sylvester-ordered Walsh-Hadamard matrix (H_d[i][j] = (-1)^popcount(i & j)); the result
 *   is orthogonal and its own inverse.  A fixed, data-free rotation folded into the weights
 *   around the cached latent leaves every full-precision result unchanged and spreads large
 *   channels over all of them before low-bit quantisation (the pages' baselines adapt fixed
 *   rotations to MLA with the same quantiser: QuantMLA podcast page, comparison part; the
 *   transforms are fused into the model offline: QuantMLA English abstract).  With R = H_d /
 *   sqrt(d_c): latent rows c -> c R (before mla_append_kv), W_UK[h] rows -> W_UK[h] R, and
 *   W_UV[h] columns -> R W_UV[h]; d = 2 on the RoPE key's pairs of both q_rope and k_rope is
 *   the pairwise form.
 *   Vector (o, i), o < n_outer, i < n_inner, starts at element o * outer_stride +
 *   i * inner_stride of x and its element k sits k * elem_stride further on (all counted in
 *   elements of dtype, MLA_F32 or MLA_BF16).  d is a power of two in [2, 4096].  Arithmetic
 *   is fp32; bf16 vectors are rounded once (ties to even).  Vectors must not overlap.
 *   n_outer = 0 is a no-op.
 */
int32_t mla_hadamard_rotate(void* x, int32_t dtype, int32_t d, int64_t elem_stride, int64_t n_outer,
                            int64_t outer_stride, int64_t n_inner, int64_t inner_stride, void* stream);

/* Decode kernel families whose in-loop dequantisation mla_dequant_blocks runs. */
#define MLA_DEQUANT_PARTITION 0  /* the partition and pipelined kernels (fewer than 96 query rows) */
#define MLA_DEQUANT_ROWS 1       /* the row-owner kernel (96 query rows or more) */

/*
 * mla_dequant_blocks (test/debug): materialise blocks of a paged cache as bf16, as a decode
 *   kernel sees them.  out_bf16[k][t][0:d_c] = latent of token t of block block_ids[k],
 *   [d_c:d_c+d_r] = RoPE key, for k < n_blocks, t < 64.  Quantised caches (the in-attention
 *   unpacking of the QuantMLA English abstract, arxivdaily QuantMLA page) run the chosen
 *   family's own code: its DMA of the code planes into an LDS code stage and its dequantisation
 *   routine into its swizzled bf16 stage, then the stage is copied out in logical order; each
 *   element is RNE_bf16((code - zero) * scale).  Every layout the decode accepts for that
 *   family is supported.  BF16 caches are copied (the decode streams their rows as they are);
 *   F32 caches are rounded to bf16 (ties to even).  Ids outside [0, num_blocks) give zero
 *   rows.  family: MLA_DEQUANT_PARTITION or MLA_DEQUANT_ROWS (ignored for float caches).
 */
int32_t mla_dequant_blocks(const void* cache_pool, int64_t num_blocks, const mla_cache_desc* desc,
                           const int32_t* block_ids, int32_t n_blocks, int32_t family, void* out_bf16,
                           void* stream);

/*
 * GQLA per-group path (GQLA abstract, thelatestinai.com paper-cards page).  GQLA ties the H heads
 * of each of num_groups groups (H / num_groups consecutive heads) to one key and one value
 * up-projection, W_UK^g [d_n][d_c] and W_UV^g [d_c][d_v], so the same weights decode two
 * algebraically equivalent ways: the absorbed MQA path above (with W_UK[h] = W_UK^g, W_UV[h] =
 * W_UV^g for g = h / (H / num_groups)), or grouped-query attention over a per-group expanded
 * cache, chosen per hardware.  On the GQA path the output is already in value space: no
 * absorption and no up-projection.
 *
 * Expanded cache, paged in blocks of 64 tokens: num_groups planes [64][k_nope (d_n) | v (d_v)]
 * bf16, then one RoPE-key plane [64][d_r] bf16 shared by the groups.  Kernels exist for
 * d_n = d_v = 128, d_r = 64 (the DeepSeek shapes); other widths give MLA_ERR_UNSUPPORTED.
 */

/* Bytes of one expanded block, or -1 if a size is not positive. */
int64_t mla_gqa_block_bytes(int32_t num_groups, int32_t d_n, int32_t d_v, int32_t d_r);

/*
 * mla_gqa_expand: write n new tokens into the expanded cache.  For token i (latent
 *   c_new[i * c_stride + 0 .. d_c), RoPE key k_rope_new[i * k_stride + 0 .. d_r), both bf16, the
 *   latent as the MLA cache holds it) and every group g, slot slots[i] = block * 64 + position
 *   receives k_nope_g = RNE_bf16(W_UK^g c) and v_g = RNE_bf16(c W_UV^g) (fp32 accumulation) in
 *   plane g, and the RoPE key in the shared plane.  w_uk_g [num_groups][d_n][d_c] and
 *   w_uv_g [num_groups][d_c][d_v] bf16.  c_new, k_rope_new, the weights and the pool 16-byte
 *   aligned, strides multiples of 8 elements, d_c a multiple of 32.  Slots outside
 *   [0, num_blocks * 64) are skipped; n = 0 is a no-op.
 */
int32_t mla_gqa_expand(const void* c_new, int64_t c_stride, const void* k_rope_new, int64_t k_stride,
                       const void* w_uk_g, const void* w_uv_g, int32_t num_groups, int32_t d_c, int32_t d_n,
                       int32_t d_v, int32_t d_r, const int32_t* slots, int64_t n, void* cache_pool,
                       int64_t num_blocks, void* stream);

/* Arguments of mla_gqa_decode_paged (device pointers except the struct itself). */
typedef struct mla_gqa_args {
  const void* q_nope;         /* [batch][s_q][H][d_n] bf16, 16-byte aligned */
  const void* q_rope;         /* [batch][s_q][H][d_r] bf16, already rotated */
  const void* cache_pool;     /* num_blocks expanded blocks, 16-byte aligned */
  int64_t num_blocks;
  int32_t num_groups, d_n, d_v, d_r;
  const int32_t* block_table; /* [batch][block_table_stride] */
  int32_t block_table_stride; /* >= ceil(max_seq_len / 64) */
  const int32_t* seq_lens;    /* [batch], each in [s_q, max_seq_len]; counts the s_q new tokens */
  int32_t max_seq_len;
  int64_t total_seq_len;      /* optional host-side sum of seq_lens (0 = unknown) */
  int32_t batch, s_q, num_heads;
  float sm_scale;
  int32_t num_splits;         /* context partitions per longest sequence, 0 = automatic */
  float* out;                 /* [batch][s_q][H][d_v] fp32 */
  float* lse;                 /* [batch][s_q][H] natural-log LSE, or NULL */
  void* workspace;            /* >= mla_gqa_workspace_size() bytes, 256-byte aligned, scratch */
  size_t workspace_bytes;
} mla_gqa_args;

/* Workspace for the split partials of mla_gqa_decode_paged (0 when the plan needs no split). */
int32_t mla_gqa_workspace_size(const mla_gqa_args* args, size_t* bytes);

/*
 * mla_gqa_decode_paged: grouped-query attention over the expanded cache.  Head h is in group
 *   g = h / (H / num_groups); its query i of sequence b attends tokens t <= L_b - s_q + i with
 *   s_t = sm_scale (q_nope . k_nope_g[t] + q_rope . k_rope[t]):  out = softmax(s) . v_g,
 *   lse = log sum_t exp(s_t).  s_q in {1, 2} (causal within the pair); num_groups divides H and
 *   s_q * H / num_groups <= 64.  Block-table entries outside the pool take no part; a sequence
 *   of length 0 gets out = 0 and lse = -inf.  Deterministic for fixed arguments.
 */
int32_t mla_gqa_decode_paged(const mla_gqa_args* args, void* stream);

/* Human-readable name of a status code (static string). */
const char* mla_status_string(int32_t status);

/* MLA_ABI_VERSION of the loaded library. */
int32_t mla_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* LIBMLA_H */
