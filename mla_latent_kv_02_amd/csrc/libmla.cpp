// libmla host layer: argument validation, cache layout, split planning and launches.
// Validation never touches the device, so a rejected call has no side effects.
#include "libmla.h"

#include <hip/hip_runtime.h>

#include <atomic>
#include <algorithm>
#include <cmath>
#include <cstdint>

#include "mla_internal.hpp"

namespace {

constexpr int kBlock = 64;
constexpr int kMaxDevices = 64;
constexpr int kMaxTilesPerSplit = 256;
std::atomic<int> g_cu_count[kMaxDevices];  // 0 = not queried yet

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }
int64_t align_up(int64_t v, int64_t a) { return (v + a - 1) / a * a; }
int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

bool valid_dtype(int32_t d) { return d == MLA_F32 || d == MLA_BF16; }
bool is_float_fmt(int32_t f) { return f == MLA_FMT_F32 || f == MLA_FMT_BF16; }
bool is_quant_fmt(int32_t f) { return f == MLA_FMT_INT4 || f == MLA_FMT_INT2; }
int fmt_bits(int32_t f) { return f == MLA_FMT_INT4 ? 4 : f == MLA_FMT_INT2 ? 2 : f == MLA_FMT_BF16 ? 16 : 32; }

struct Layout {
  int64_t block_bytes = -1;
  int64_t off[4] = {0, -1, -1, -1};
};

// Byte layout of one block (see mla_cache_desc).  Returns false for an invalid descriptor.
bool cache_layout(const mla_cache_desc* d, Layout* out) {
  if (d == nullptr || d->block_size != kBlock || d->d_c <= 0 || d->d_r <= 0) return false;
  if (is_float_fmt(d->latent_fmt)) {
    if (d->rope_fmt != d->latent_fmt) return false;
    out->block_bytes = (int64_t)kBlock * (d->d_c + d->d_r) * (fmt_bits(d->latent_fmt) / 8);
    out->off[0] = 0;
    out->off[1] = out->off[2] = out->off[3] = -1;
    return true;
  }
  if (!is_quant_fmt(d->latent_fmt) || !is_quant_fmt(d->rope_fmt)) return false;
  if (d->latent_group <= 0 || d->rope_group <= 0 || d->d_c % d->latent_group || d->d_r % d->rope_group) return false;
  const int lb = fmt_bits(d->latent_fmt), rb = fmt_bits(d->rope_fmt);
  if ((d->d_c * lb) % 8 || (d->d_r * rb) % 8) return false;
  const int64_t sizes[4] = {(int64_t)kBlock * d->d_c * lb / 8, (int64_t)kBlock * (d->d_c / d->latent_group) * 4,
                            (int64_t)kBlock * d->d_r * rb / 8, (int64_t)kBlock * (d->d_r / d->rope_group) * 4};
  int64_t pos = 0;
  for (int i = 0; i < 4; ++i) {
    out->off[i] = pos;
    pos += align_up(sizes[i], 16);
  }
  out->block_bytes = pos;
  return true;
}

// Is there a decode kernel for this (valid) descriptor and query dtype?
bool decode_supported(const mla_cache_desc* d, int32_t q_dtype) {
  if (d->latent_fmt == MLA_FMT_F32) return q_dtype == MLA_F32 && d->d_c <= 1024 && d->d_r <= 256;
  if (d->d_c != 512 || d->d_r != 64) return false;
  if (d->latent_fmt == MLA_FMT_BF16) return true;
  if (d->rope_fmt != MLA_FMT_INT4 || (d->rope_group != 32 && d->rope_group != 64)) return false;
  if (d->latent_fmt == MLA_FMT_INT4) return d->latent_group % 32 == 0;
  return d->latent_group % 32 == 0;  // INT2
}

int32_t validate_decode(const mla_decode_args* a, Layout* lay) {
  if (a == nullptr) return MLA_ERR_INVALID_ARG;
  if (!a->q_lat || !a->q_rope || !a->cache_pool || !a->block_table || !a->seq_lens || !a->o_lat)
    return MLA_ERR_INVALID_ARG;
  if (a->batch <= 0 || a->num_heads <= 0 || (a->s_q != 1 && a->s_q != 2)) return MLA_ERR_INVALID_ARG;
  if (a->max_seq_len < a->s_q || a->num_blocks <= 0) return MLA_ERR_INVALID_ARG;
  if (!valid_dtype(a->q_dtype) || !valid_dtype(a->o_dtype)) return MLA_ERR_INVALID_ARG;
  if (!std::isfinite(a->sm_scale) || a->num_splits < 0) return MLA_ERR_INVALID_ARG;
  if (!cache_layout(&a->cache, lay)) return MLA_ERR_INVALID_ARG;
  if (a->block_table_stride < ceil_div(a->max_seq_len, kBlock)) return MLA_ERR_INVALID_ARG;
  if (!aligned(a->q_lat, 16) || !aligned(a->q_rope, 16) || !aligned(a->cache_pool, 16) || !aligned(a->o_lat, 16))
    return MLA_ERR_INVALID_ARG;
  if (!aligned(a->block_table, 4) || !aligned(a->seq_lens, 4) || (a->lse && !aligned(a->lse, 4)))
    return MLA_ERR_INVALID_ARG;
  if (!decode_supported(&a->cache, a->q_dtype)) return MLA_ERR_UNSUPPORTED;
  const int64_t rows = (int64_t)a->s_q * a->num_heads;
  if (rows > (1 << 20) || (int64_t)a->batch * rows > (1LL << 30)) return MLA_ERR_UNSUPPORTED;
  return MLA_OK;
}

struct Plan {
  bool rows;       // row-owner kernel over balanced block ranges
  int rt;          // row tiles per workgroup (partition MFMA kernel), 0 = fp32 kernel
  int rg;          // row groups per sequence
  int splits;      // partitions of the longest sequence, or block ranges (rows)
  int tpc;         // 64-token tiles per partition, or an upper bound of blocks per range (rows)
};

constexpr int kRowsMinRows = 96;        // query rows per sequence from which the row-owner kernel runs
constexpr int kRowsPerGroup = 128;      // its rows per workgroup
constexpr int kRowsMaxBatch = 8192;     // sequences it tabulates in LDS
constexpr int kRowsMaxRangeBlocks = 256;
// Block-space positions charged for the start of each sequence when the row-owner kernel cuts
// the batch into ranges: a workgroup whose range starts a sequence in its middle stores a
// 256 KB piece and loads the next sequence's 144 KB of queries there, about the time of two
// to three blocks; 3 gave the shortest decode among 1..6 on the 128-head bf16 workloads.
// The kernel drops the charge when every sequence already starts on a range boundary.
constexpr int kRowsPhantom = 3;

Plan make_plan(const mla_decode_args* a, int cus) {
  Plan p{};
  const int R = a->s_q * a->num_heads;
  if (a->cache.latent_fmt != MLA_FMT_F32 && R >= kRowsMinRows && a->batch <= kRowsMaxBatch) {
    // the batch's blocks, sequence after sequence, cut into equal ranges: one workgroup per
    // (range, row group), a single round over the CUs unless the ranges would get too long
    p.rows = true;
    p.rg = (int)ceil_div(R, kRowsPerGroup);
    const int64_t bound = (int64_t)a->batch * ceil_div(a->max_seq_len, kBlock);  // blocks, at most
    const int64_t vbound = bound + (int64_t)a->batch * kRowsPhantom;              // positions, at most
    int64_t n = a->num_splits > 0 ? (int64_t)a->num_splits * a->batch : std::max<int64_t>(1, cus / p.rg);
    n = std::max<int64_t>(n, ceil_div(vbound, kRowsMaxRangeBlocks));
    n = std::min<int64_t>(n, bound);
    p.splits = (int)n;
    p.tpc = (int)ceil_div(vbound, n);
    return p;
  }
  int64_t target;  // workgroups to aim for
  if (a->cache.latent_fmt == MLA_FMT_F32) {
    p.rt = 0;
    p.rg = R;
    target = (int64_t)cus * 8;
  } else {
    p.rt = R <= 16 ? 1 : (R <= 32 ? 2 : 4);
    p.rg = (int)ceil_div(R, 16 * p.rt);
    target = (int64_t)cus;  // one 512-thread workgroup per CU: a single round of equal partitions
  }
  const int nblk = (int)ceil_div(a->max_seq_len, kBlock);
  int tpc;
  if (a->num_splits > 0) {
    tpc = (int)ceil_div(nblk, a->num_splits < nblk ? a->num_splits : nblk);
  } else if (a->total_seq_len > 0) {
    // balance by total work: the batch's blocks x row groups spread over the target
    tpc = (int)ceil_div(ceil_div(a->total_seq_len, kBlock) * p.rg, target);
  } else {
    tpc = (int)ceil_div((int64_t)nblk * a->batch * p.rg, target);
  }
  tpc = tpc < 1 ? 1 : (tpc > nblk ? nblk : tpc);
  if (p.rt > 0 && tpc > kMaxTilesPerSplit) tpc = kMaxTilesPerSplit;  // the MFMA kernel stages block ids in LDS
  p.tpc = tpc;
  p.splits = (int)ceil_div(nblk, tpc);
  return p;
}

int32_t device_cus(int* cus) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return MLA_ERR_HIP;
  if (dev >= 0 && dev < kMaxDevices) {
    int v = g_cu_count[dev].load(std::memory_order_relaxed);
    if (v > 0) {
      *cus = v;
      return MLA_OK;
    }
  }
  int v = 0;
  if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0)
    return MLA_ERR_HIP;
  if (dev >= 0 && dev < kMaxDevices) g_cu_count[dev].store(v, std::memory_order_relaxed);
  *cus = v;
  return MLA_OK;
}

// Workspace layout.  Row-owner kernel: meta [B + 3] int32, then partial o, lse and 1/sum(P)
// of the slots b + i (B + ranges - 1 of them).  Partition kernels: partial o, then lse.
size_t rows_meta_bytes(const mla_decode_args* a) { return (size_t)align_up(((int64_t)a->batch + 3) * 4, 256); }

size_t partial_bytes(const mla_decode_args* a, const Plan& p, size_t* lse_off) {
  if (p.rows) {
    const int64_t slots = (int64_t)a->batch + p.splits - 1;
    const int64_t rows = slots * a->s_q * a->num_heads;
    const int64_t o_bytes = align_up(rows * a->cache.d_c * 4, 256);
    *lse_off = rows_meta_bytes(a) + (size_t)o_bytes;
    return *lse_off + 2 * (size_t)align_up(rows * 4, 256);
  }
  if (p.splits <= 1) {
    *lse_off = 0;
    return 0;
  }
  const int64_t units = (int64_t)a->batch * p.splits * a->s_q * a->num_heads;
  const int64_t o_bytes = align_up(units * a->cache.d_c * 4, 256);
  *lse_off = (size_t)o_bytes;
  return (size_t)(o_bytes + align_up(units * 4, 256));
}

int32_t hip_status(hipError_t e) { return e == hipSuccess ? MLA_OK : MLA_ERR_HIP; }

int32_t validate_proj(const void* x, int32_t xdt, const void* w, int32_t wdt, void* y, int32_t ydt, int32_t N,
                      int32_t H, int32_t K, int32_t M, int64_t sn, int64_t sh) {
  if (!x || !w || !y) return MLA_ERR_INVALID_ARG;
  if (N <= 0 || H <= 0 || K <= 0 || M <= 0 || sn < 0 || sh < 0) return MLA_ERR_INVALID_ARG;
  if (!valid_dtype(xdt) || !valid_dtype(wdt) || !valid_dtype(ydt)) return MLA_ERR_INVALID_ARG;
  if (!aligned(x, xdt == MLA_F32 ? 4 : 2) || !aligned(w, wdt == MLA_F32 ? 4 : 2) || !aligned(y, ydt == MLA_F32 ? 4 : 2))
    return MLA_ERR_INVALID_ARG;
  if ((int64_t)N * H * M > (1LL << 40)) return MLA_ERR_UNSUPPORTED;
  return MLA_OK;
}

int32_t run_proj(const void* x, int64_t sn, int64_t sh, int32_t xdt, const void* w, int32_t wdt, void* y,
                 int32_t ydt, int32_t N, int32_t H, int32_t K, int32_t M, void* stream) {
  int32_t s = validate_proj(x, xdt, w, wdt, y, ydt, N, H, K, M, sn, sh);
  if (s != MLA_OK) return s;
  mla::ProjParams p{};
  p.X = x;
  p.sxn = sn;
  p.sxh = sh;
  p.x_f32 = xdt == MLA_F32;
  p.W = w;
  p.w_f32 = wdt == MLA_F32;
  p.Y = y;
  p.y_f32 = ydt == MLA_F32;
  p.N = N;
  p.H = H;
  p.K = K;
  p.M = M;
  p.aligned16 = aligned(x, 16) && aligned(w, 16) && aligned(y, 16);
  return hip_status(mla::launch_proj(p, (hipStream_t)stream));
}

// ---------------------------------------------------------------------------------------
// GQLA per-group path: validation, plan (partitions of the longest sequence, one workgroup per
// (sequence, partition, group), two workgroups per CU) and the partial layout.
struct GqaPlan {
  int rt, splits, tpc;
};

int32_t validate_gqa(const mla_gqa_args* a) {
  if (a == nullptr) return MLA_ERR_INVALID_ARG;
  if (!a->q_nope || !a->q_rope || !a->cache_pool || !a->block_table || !a->seq_lens || !a->out)
    return MLA_ERR_INVALID_ARG;
  if (a->batch <= 0 || a->num_heads <= 0 || a->num_groups <= 0 || (a->s_q != 1 && a->s_q != 2))
    return MLA_ERR_INVALID_ARG;
  if (a->max_seq_len < a->s_q || a->num_blocks <= 0 || a->num_splits < 0 || !std::isfinite(a->sm_scale))
    return MLA_ERR_INVALID_ARG;
  if (a->d_n <= 0 || a->d_v <= 0 || a->d_r <= 0 || a->num_heads % a->num_groups) return MLA_ERR_INVALID_ARG;
  if (a->block_table_stride < ceil_div(a->max_seq_len, kBlock)) return MLA_ERR_INVALID_ARG;
  if (!aligned(a->q_nope, 16) || !aligned(a->q_rope, 16) || !aligned(a->cache_pool, 16) || !aligned(a->out, 4))
    return MLA_ERR_INVALID_ARG;
  if (!aligned(a->block_table, 4) || !aligned(a->seq_lens, 4) || (a->lse && !aligned(a->lse, 4)))
    return MLA_ERR_INVALID_ARG;
  if (a->d_n != 128 || a->d_v != 128 || a->d_r != 64) return MLA_ERR_UNSUPPORTED;
  if ((int64_t)a->s_q * a->num_heads / a->num_groups > 64) return MLA_ERR_UNSUPPORTED;
  if ((int64_t)a->batch * a->s_q * a->num_heads > (1LL << 30)) return MLA_ERR_UNSUPPORTED;
  return MLA_OK;
}

GqaPlan gqa_plan(const mla_gqa_args* a, int cus) {
  GqaPlan p{};
  const int rg = a->s_q * a->num_heads / a->num_groups;
  p.rt = rg <= 16 ? 1 : (rg <= 32 ? 2 : 4);
  const int nblk = (int)ceil_div(a->max_seq_len, kBlock);
  const int64_t target = 2 * (int64_t)cus;   // two workgroups per CU: a single round of partitions
  int tpc;
  if (a->num_splits > 0) {
    tpc = (int)ceil_div(nblk, a->num_splits < nblk ? a->num_splits : nblk);
  } else {
    const int64_t blocks = a->total_seq_len > 0 ? ceil_div(a->total_seq_len, kBlock) : (int64_t)nblk * a->batch;
    tpc = (int)ceil_div(blocks * a->num_groups, target);
  }
  tpc = std::max(1, std::min(tpc, std::min(nblk, kMaxTilesPerSplit)));
  p.tpc = tpc;
  p.splits = (int)ceil_div(nblk, tpc);
  return p;
}

size_t gqa_partial_bytes(const mla_gqa_args* a, const GqaPlan& p) {
  if (p.splits <= 1) return 0;
  const int64_t rows = (int64_t)a->batch * p.splits * a->s_q * a->num_heads;
  return (size_t)(align_up(rows * a->d_v * 4, 256) + align_up(rows * 4, 256));
}

}  // namespace

// ---------------------------------------------------------------------------------------
// Mixed-precision history: parts[0] = sink (earliest tokens), parts[1] = middle (low-bit),
// parts[2] = recent window (ends with the s_q new tokens); any may be null.  Workspace:
// partial o [3][B][R][d_c] fp32, partial lse [3][B][R], then the parts' own decode workspace
// (used by one part after the other on the stream).
namespace {

struct MixedLayout {
  size_t o_bytes = 0, lse_off = 0, total = 0;
  size_t dec_off[3] = {0, 0, 0};   // each part's own decode workspace (its partials stay until the merge)
  bool joint = false;              // one row-owner decode over the joint history (workspace: its own)
};

// A mixed history that the row-owner kernel decodes as one sequence of blocks per batch
// entry: a low-bit middle of that kernel's family, with bf16 sink and recent parts (either may
// be absent).  J: the middle's arguments with the joint history's length bound; false: the
// parts are decoded one by one and merged.
bool mixed_joint(const mla_decode_args* const parts[3], int cus, mla_decode_args* J, Plan* plan) {
  const mla_decode_args* mid = parts[1];
  if (mid == nullptr || !is_quant_fmt(mid->cache.latent_fmt)) return false;
  Layout ml;
  if (!cache_layout(&mid->cache, &ml)) return false;
  int64_t nblk = ceil_div(mid->max_seq_len, kBlock);
  for (int i = 0; i < 3; i += 2) {
    const mla_decode_args* a = parts[i];
    if (a == nullptr) continue;
    Layout l;
    // a bf16 block's slot in the code ring receives a stand-in copy of its first
    // block_bytes(middle) bytes, so the bf16 block must be at least that long
    if (a->cache.latent_fmt != MLA_FMT_BF16 || !cache_layout(&a->cache, &l) || l.block_bytes < ml.block_bytes)
      return false;
    nblk += ceil_div(a->max_seq_len, kBlock);
  }
  if (nblk * kBlock > (1LL << 30)) return false;
  *J = *mid;
  J->max_seq_len = (int)(nblk * kBlock);
  if (mid->total_seq_len > 0) {
    int64_t t = mid->total_seq_len;
    for (int i = 0; i < 3; i += 2)
      if (parts[i] != nullptr)
        t += parts[i]->total_seq_len > 0 ? parts[i]->total_seq_len : (int64_t)mid->batch * parts[i]->max_seq_len;
    J->total_seq_len = t;
  }
  *plan = make_plan(J, cus);
  if (plan->rows) return true;   // the row-owner kernel
  // the pipelined partition kernel (at most 16 query rows): partitions over weighted positions
  if (plan->rt != 1 || !mla::pipe_mixed_fits(mid->cache.latent_fmt, mid->cache.latent_group, mid->cache.rope_group))
    return false;
  int64_t hi_blk = 0;
  for (int i = 0; i < 3; i += 2)
    if (parts[i] != nullptr) hi_blk += ceil_div(parts[i]->max_seq_len, kBlock);
  const int64_t wblk = mla::kMixedBf16Weight * hi_blk + ceil_div(mid->max_seq_len, kBlock);
  if (wblk * kBlock > (1LL << 30)) return false;
  J->max_seq_len = (int)(wblk * kBlock);
  J->total_seq_len = 0;   // plan by the weighted bound
  *plan = make_plan(J, cus);
  if (plan->rows || plan->rt != 1) return false;
  // the kernel keeps each block's address in 56 bits
  for (int i = 0; i < 3; ++i) {
    const mla_decode_args* a = parts[i];
    if (a == nullptr) continue;
    Layout l;
    cache_layout(&a->cache, &l);
    if ((uint64_t)(uintptr_t)a->cache_pool + (uint64_t)a->num_blocks * (uint64_t)l.block_bytes >= mla::kPipeAddrLimit)
      return false;
  }
  return true;
}

// The args a part is decoded with: its own cache and block table, the shared queries; sink
// and middle precede every query, so with s_q = 2 the two queries are decoded as 2H heads.
mla_decode_args part_args(const mla_decode_args* a, bool causal) {
  mla_decode_args p = *a;
  if (!causal && p.s_q == 2) {
    p.s_q = 1;
    p.num_heads *= 2;
  }
  p.o_dtype = MLA_F32;
  return p;
}

int32_t mixed_layout(const mla_decode_args* const parts[3], MixedLayout* m) {
  const mla_decode_args* ref = nullptr;
  for (int i = 0; i < 3; ++i)
    if (parts[i] != nullptr) {
      ref = parts[i];
      break;
    }
  if (ref == nullptr) return MLA_ERR_INVALID_ARG;
  // with two query tokens the new tokens sit in the recent part, the only one with the causal mask
  if (ref->s_q == 2 && parts[2] == nullptr) return MLA_ERR_INVALID_ARG;
  for (int i = 0; i < 3; ++i) {
    const mla_decode_args* a = parts[i];
    if (a == nullptr) continue;
    if (a->batch != ref->batch || a->s_q != ref->s_q || a->num_heads != ref->num_heads || a->q_lat != ref->q_lat ||
        a->q_rope != ref->q_rope || a->q_dtype != ref->q_dtype || a->sm_scale != ref->sm_scale ||
        a->cache.d_c != ref->cache.d_c || a->cache.d_r != ref->cache.d_r)
      return MLA_ERR_INVALID_ARG;
  }
  const int64_t rows = (int64_t)ref->batch * ref->s_q * ref->num_heads;
  m->o_bytes = (size_t)align_up(3 * rows * ref->cache.d_c * 4, 256);
  m->lse_off = m->o_bytes;
  size_t off = m->lse_off + (size_t)align_up(3 * rows * 4, 256);
  int cus = 0;
  int32_t s = device_cus(&cus);
  if (s != MLA_OK) return s;
  for (int i = 0; i < 3; ++i) {
    if (parts[i] == nullptr) continue;
    mla_decode_args p = part_args(parts[i], i == 2);
    p.o_lat = (void*)(uintptr_t)256;   // placeholders for validation only
    p.lse = nullptr;
    Layout lay;
    s = validate_decode(&p, &lay);
    if (s != MLA_OK) return s;
    size_t lse_off = 0;
    m->dec_off[i] = off;
    off += (size_t)align_up((int64_t)partial_bytes(&p, make_plan(&p, cus), &lse_off), 256);
  }
  m->total = off;
  mla_decode_args J;
  Plan jp;
  m->joint = mixed_joint(parts, cus, &J, &jp);
  if (m->joint) {
    size_t lse_off = 0;
    m->total = (size_t)align_up((int64_t)partial_bytes(&J, jp, &lse_off), 256);
  }
  return MLA_OK;
}

}  // namespace

extern "C" {

int32_t mla_abi_version(void) { return MLA_ABI_VERSION; }

const char* mla_status_string(int32_t s) {
  switch (s) {
    case MLA_OK: return "MLA_OK";
    case MLA_ERR_INVALID_ARG: return "MLA_ERR_INVALID_ARG: invalid argument";
    case MLA_ERR_UNSUPPORTED: return "MLA_ERR_UNSUPPORTED: no kernel for this combination";
    case MLA_ERR_WORKSPACE: return "MLA_ERR_WORKSPACE: workspace missing or too small";
    case MLA_ERR_HIP: return "MLA_ERR_HIP: HIP runtime error";
  }
  return "unknown mla status";
}

int64_t mla_cache_block_bytes(const mla_cache_desc* desc) {
  Layout l;
  return cache_layout(desc, &l) ? l.block_bytes : -1;
}

int32_t mla_cache_plane_offsets(const mla_cache_desc* desc, int64_t offsets[4]) {
  Layout l;
  if (offsets == nullptr || !cache_layout(desc, &l)) return MLA_ERR_INVALID_ARG;
  for (int i = 0; i < 4; ++i) offsets[i] = l.off[i];
  return MLA_OK;
}

int32_t mla_absorb_q(const void* q_nope, int64_t q_stride_n, int64_t q_stride_h, int32_t q_dtype, const void* w_uk,
                     int32_t w_dtype, void* q_lat, int32_t out_dtype, int32_t N, int32_t H, int32_t d_n, int32_t d_c,
                     void* stream) {
  return run_proj(q_nope, q_stride_n, q_stride_h, q_dtype, w_uk, w_dtype, q_lat, out_dtype, N, H, d_n, d_c, stream);
}

int32_t mla_out_proj(const void* o_lat, int64_t o_stride_n, int64_t o_stride_h, int32_t o_dtype, const void* w_uv,
                     int32_t w_dtype, void* out, int32_t out_dtype, int32_t N, int32_t H, int32_t d_c, int32_t d_v,
                     void* stream) {
  return run_proj(o_lat, o_stride_n, o_stride_h, o_dtype, w_uv, w_dtype, out, out_dtype, N, H, d_c, d_v, stream);
}

int32_t mla_decode_plan(const mla_decode_args* args, int32_t num_cus, int32_t* num_splits, int32_t* tiles_per_split) {
  Layout lay;
  int32_t s = validate_decode(args, &lay);
  if (s != MLA_OK) return s;
  if (num_splits == nullptr || tiles_per_split == nullptr || num_cus < 0) return MLA_ERR_INVALID_ARG;
  int cus = num_cus;
  if (cus == 0) {
    s = device_cus(&cus);
    if (s != MLA_OK) return s;
  }
  const Plan p = make_plan(args, cus);
  *num_splits = p.splits;
  *tiles_per_split = p.tpc;
  return MLA_OK;
}

int32_t mla_decode_workspace_size_for(const mla_decode_args* args, int32_t num_cus, size_t* bytes) {
  Layout lay;
  int32_t s = validate_decode(args, &lay);
  if (s != MLA_OK) return s;
  if (bytes == nullptr || num_cus < 0) return MLA_ERR_INVALID_ARG;
  int cus = num_cus;
  if (cus == 0 && args->num_splits == 0) {
    s = device_cus(&cus);
    if (s != MLA_OK) return s;
  }
  size_t lse_off = 0;
  *bytes = partial_bytes(args, make_plan(args, cus), &lse_off);
  return MLA_OK;
}

int32_t mla_decode_workspace_size(const mla_decode_args* args, size_t* bytes) {
  return mla_decode_workspace_size_for(args, 0, bytes);
}

}  // extern "C"

namespace {

// Row-owner kernel arguments of decode `a` under `plan`, its split partials in `ws` at the
// layout partial_bytes gives (lse_off).
int32_t rows_params(const mla_decode_args* a, const Layout& lay, const Plan& plan, void* ws, size_t lse_off,
                    mla::RowsParams* out) {
  mla::RowsParams r{};
  r.q_lat = a->q_lat;
  r.q_rope = a->q_rope;
  r.q_f32 = a->q_dtype == MLA_F32;
  r.pool = (const uint8_t*)a->cache_pool;
  r.num_blocks = a->num_blocks;
  r.block_bytes = lay.block_bytes;
  r.off_lc = lay.off[0];
  r.off_ls = lay.off[1];
  r.off_rc = lay.off[2];
  r.off_rs = lay.off[3];
  auto log2i = [](int v) { int l = 0; while ((1 << (l + 1)) <= v) ++l; return l; };
  r.g_lat_log2 = log2i(a->cache.latent_group > 0 ? a->cache.latent_group : 1);
  r.g_rope_log2 = log2i(a->cache.rope_group > 0 ? a->cache.rope_group : 1);
  r.block_table = a->block_table;
  r.bt_stride = a->block_table_stride;
  r.seq_lens = a->seq_lens;
  r.max_seq_len = a->max_seq_len;
  r.B = a->batch;
  r.s_q = a->s_q;
  r.H = a->num_heads;
  r.R = a->s_q * a->num_heads;
  r.RG = plan.rg;
  r.n_ranges = plan.splits;
  r.phantom = kRowsPhantom;
  const int64_t units = (int64_t)plan.splits * plan.rg;
  if (units > (1LL << 30)) return MLA_ERR_UNSUPPORTED;
  r.total_units = (int)units;
  r.units_per_xcd = (int)ceil_div(units, 8);
  r.scale_log2 = a->sm_scale * 1.4426950408889634f;
  r.out = a->o_lat;
  r.out_bf16 = a->o_dtype == MLA_BF16;
  r.out_lse = a->lse;
  r.meta = (int32_t*)ws;
  r.part_o = (float*)((char*)ws + rows_meta_bytes(a));
  r.part_lse = (float*)((char*)ws + lse_off);
  r.part_inv = (float*)((char*)ws + lse_off + align_up((int64_t)(a->batch + plan.splits - 1) * r.R * 4, 256));
  *out = r;
  return MLA_OK;
}

// The merge of a row-owner decode's pieces into o_lat and lse.
int32_t rows_combine(const mla_decode_args* a, const mla::RowsParams& r, const Plan& plan, hipStream_t st) {
  mla::CombineParams c{};
  c.part_o = r.part_o;
  c.part_lse = r.part_lse;
  c.part_inv = r.part_inv;
  c.seq_lens = a->seq_lens;
  c.max_seq_len = a->max_seq_len;
  c.R = r.R;
  c.d_c = a->cache.d_c;
  c.meta = r.meta;
  c.out = a->o_lat;
  c.out_bf16 = a->o_dtype == MLA_BF16;
  c.out_lse = a->lse;
  c.B = a->batch;
  // a sequence meets about n_ranges / batch + 1 ranges
  c.many_parts = plan.splits > 16 * a->batch;
  return hip_status(mla::launch_combine(c, a->batch, st));
}

// Partition-kernel arguments of decode `a` under `plan`: split partials in `ws` (layout of
// partial_bytes, lse at lse_off) when the plan splits, else o_lat and lse directly.
int32_t partition_params(const mla_decode_args* a, const Layout& lay, const Plan& plan, void* ws, size_t lse_off,
                         mla::DecodeParams* out) {
  mla::DecodeParams p{};
  p.q_lat = a->q_lat;
  p.q_rope = a->q_rope;
  p.q_f32 = a->q_dtype == MLA_F32;
  p.pool = (const uint8_t*)a->cache_pool;
  p.num_blocks = a->num_blocks;
  p.block_bytes = lay.block_bytes;
  p.off_lc = lay.off[0];
  p.off_ls = lay.off[1];
  p.off_rc = lay.off[2];
  p.off_rs = lay.off[3];
  p.g_lat = a->cache.latent_group > 0 ? a->cache.latent_group : 1;
  p.g_rope = a->cache.rope_group > 0 ? a->cache.rope_group : 1;
  p.block_table = a->block_table;
  p.bt_stride = a->block_table_stride;
  p.seq_lens = a->seq_lens;
  p.max_seq_len = a->max_seq_len;
  p.B = a->batch;
  p.s_q = a->s_q;
  p.H = a->num_heads;
  p.R = a->s_q * a->num_heads;
  p.RG = plan.rg;
  p.d_c = a->cache.d_c;
  p.d_r = a->cache.d_r;
  p.max_chunks = plan.splits;
  p.tpc = plan.tpc;
  p.scale_log2 = a->sm_scale * 1.4426950408889634f;
  const bool split = plan.splits > 1;
  p.out = split ? ws : a->o_lat;
  p.out_bf16 = split ? 0 : (a->o_dtype == MLA_BF16);
  p.out_lse = split ? (float*)((char*)ws + lse_off) : a->lse;
  const int64_t units = (int64_t)a->batch * plan.splits * plan.rg;
  if (units > (1LL << 30)) return MLA_ERR_UNSUPPORTED;
  p.total_units = (int)units;
  p.units_per_xcd = (int)ceil_div(units, 8);
  *out = p;
  return MLA_OK;
}

// The merge of a split partition decode into o_lat and lse (hi: the bf16 parts of a mixed
// history, whose blocks count with the sequence's, or null).
int32_t partition_combine(const mla_decode_args* a, const mla::DecodeParams& p, const Plan& plan,
                          const mla::MixedPart* hi, hipStream_t st) {
  mla::CombineParams c{};
  c.part_o = (const float*)p.out;
  c.part_lse = p.out_lse;
  c.seq_lens = a->seq_lens;
  c.max_seq_len = a->max_seq_len;
  c.R = p.R;
  c.d_c = p.d_c;
  c.max_chunks = plan.splits;
  c.tpc = plan.tpc;
  c.out = a->o_lat;
  c.out_bf16 = a->o_dtype == MLA_BF16;
  c.out_lse = a->lse;
  c.many_parts = plan.splits > 16;
  c.B = a->batch;
  c.mixed = hi != nullptr;
  for (int k = 0; k < 2 && hi != nullptr; ++k) {
    c.hi_lens[k] = hi[k].seq_lens;
    c.hi_max[k] = hi[k].max_seq_len;
  }
  return hip_status(mla::launch_combine(c, a->batch, st));
}

// The decode with its split partials in `ws`: the caller's workspace (mla_decode_paged) or
// the library's per-device scratch array (mla_decode_paged_noalloc, ws == nullptr on entry).
// With `defer`, only the decode kernel runs and *defer says where its partials are, for a
// merge over several decodes (a decode without split partials wrote o_lat and lse, which
// must then be fp32 and present: that pair is its single partial).
int32_t decode_paged(const mla_decode_args* a, bool noalloc, void* stream, mla::CombinePart* defer = nullptr) {
  Layout lay;
  int32_t s = validate_decode(a, &lay);
  if (s != MLA_OK) return s;
  // an explicit split count fixes the plan without the device's CU count
  int cus = 0;
  if (a->num_splits == 0) {
    s = device_cus(&cus);
    if (s != MLA_OK) return s;
  }
  const Plan plan = make_plan(a, cus);
  size_t lse_off = 0;
  const size_t need = partial_bytes(a, plan, &lse_off);
  void* ws = a->workspace;
  if (noalloc) {
    if (need > mla::kNoAllocScratchBytes) return MLA_ERR_WORKSPACE;
    ws = nullptr;
    if (need > 0 && mla::noalloc_scratch(&ws) != hipSuccess) return MLA_ERR_HIP;
  } else if (need > 0 && (ws == nullptr || a->workspace_bytes < need || !aligned(ws, 256))) {
    return MLA_ERR_WORKSPACE;
  }

  hipStream_t st = (hipStream_t)stream;
  if (plan.rows) {
    mla::RowsParams r{};
    s = rows_params(a, lay, plan, ws, lse_off, &r);
    if (s != MLA_OK) return s;
    hipError_t e = mla::launch_decode_rows(r, a->cache.latent_fmt, st);
    if (e != hipSuccess) return MLA_ERR_HIP;
    if (defer != nullptr) {
      *defer = mla::CombinePart{r.part_o, r.part_lse, r.part_inv, r.meta, a->seq_lens, a->max_seq_len, 0, 1,
                                plan.splits > 16 * a->batch};
      return MLA_OK;
    }
    return rows_combine(a, r, plan, st);
  }

  mla::DecodeParams p{};
  s = partition_params(a, lay, plan, ws, lse_off, &p);
  if (s != MLA_OK) return s;
  const bool split = plan.splits > 1;
  float* part_o = split ? (float*)p.out : nullptr;
  float* part_lse = split ? p.out_lse : nullptr;

  hipError_t e = plan.rt == 0 ? mla::launch_decode_f32(p, st) : mla::launch_decode_mfma(p, a->cache.latent_fmt, plan.rt, st);
  if (e != hipSuccess) return MLA_ERR_HIP;
  if (defer != nullptr) {
    if (split)
      *defer = mla::CombinePart{part_o, part_lse, nullptr, nullptr, a->seq_lens, a->max_seq_len, plan.splits, plan.tpc,
                                plan.splits > 16};
    else if (a->o_dtype != MLA_F32 || a->lse == nullptr)
      return MLA_ERR_INVALID_ARG;
    else
      *defer = mla::CombinePart{(const float*)a->o_lat, a->lse, nullptr, nullptr, a->seq_lens, a->max_seq_len, 1, plan.tpc,
                                0};
    return MLA_OK;
  }
  if (split) return partition_combine(a, p, plan, nullptr, st);
  return MLA_OK;
}

}  // namespace

extern "C" {

int32_t mla_decode_paged(const mla_decode_args* a, void* stream) { return decode_paged(a, false, stream); }

int32_t mla_decode_paged_noalloc(const mla_decode_args* a, void* stream) { return decode_paged(a, true, stream); }

int32_t mla_decode_mixed_workspace_size(const mla_decode_args* sink, const mla_decode_args* middle,
                                        const mla_decode_args* recent, size_t* bytes) {
  if (bytes == nullptr) return MLA_ERR_INVALID_ARG;
  const mla_decode_args* parts[3] = {sink, middle, recent};
  MixedLayout m;
  const int32_t s = mixed_layout(parts, &m);
  if (s != MLA_OK) return s;
  *bytes = m.total;
  return MLA_OK;
}

int32_t mla_decode_mixed(const mla_decode_args* sink, const mla_decode_args* middle, const mla_decode_args* recent,
                         void* o_lat, int32_t o_dtype, float* lse, void* workspace, size_t workspace_bytes,
                         void* stream) {
  const mla_decode_args* parts[3] = {sink, middle, recent};
  MixedLayout m;
  int32_t s = mixed_layout(parts, &m);
  if (s != MLA_OK) return s;
  if (o_lat == nullptr || !valid_dtype(o_dtype) || !aligned(o_lat, 16) || (lse && !aligned(lse, 4)))
    return MLA_ERR_INVALID_ARG;
  if (workspace == nullptr || workspace_bytes < m.total || !aligned(workspace, 256)) return MLA_ERR_WORKSPACE;
  hipStream_t st = (hipStream_t)stream;
  if (m.joint) {
    // one decode over sink ++ middle ++ recent per sequence, then its merge
    int cus = 0;
    s = device_cus(&cus);
    if (s != MLA_OK) return s;
    mla_decode_args J;
    Plan plan;
    mixed_joint(parts, cus, &J, &plan);
    J.o_lat = o_lat;
    J.o_dtype = o_dtype;
    J.lse = lse;
    Layout lay;
    cache_layout(&J.cache, &lay);
    size_t lse_off = 0;
    partial_bytes(&J, plan, &lse_off);
    mla::MixedPart hi[2] = {};
    for (int i = 0; i < 3; i += 2) {
      const mla_decode_args* a = parts[i];
      if (a == nullptr) continue;   // no lengths: an absent part
      Layout l;
      cache_layout(&a->cache, &l);
      mla::MixedPart& h = hi[i >> 1];
      h.pool = (const uint8_t*)a->cache_pool;
      h.num_blocks = a->num_blocks;
      h.block_bytes = l.block_bytes;
      h.block_table = a->block_table;
      h.bt_stride = a->block_table_stride;
      h.seq_lens = a->seq_lens;
      h.max_seq_len = a->max_seq_len;
    }
    if (plan.rows) {
      mla::RowsParams r{};
      s = rows_params(&J, lay, plan, workspace, lse_off, &r);
      if (s != MLA_OK) return s;
      r.max_seq_len = middle->max_seq_len;   // the middle's own bound (J has the joint one)
      r.hi[0] = hi[0];
      r.hi[1] = hi[1];
      if (mla::launch_decode_rows_mixed(r, J.cache.latent_fmt, st) != hipSuccess) return MLA_ERR_HIP;
      return rows_combine(&J, r, plan, st);
    }
    mla::DecodeParams p{};
    s = partition_params(&J, lay, plan, workspace, lse_off, &p);
    if (s != MLA_OK) return s;
    p.max_seq_len = middle->max_seq_len;
    p.hi[0] = hi[0];
    p.hi[1] = hi[1];
    if (mla::launch_decode_pipe_mixed(p, J.cache.latent_fmt, st) != hipSuccess) return MLA_ERR_HIP;
    if (plan.splits <= 1) return MLA_OK;
    J.max_seq_len = middle->max_seq_len;   // the combine counts the middle's blocks from its own lengths
    return partition_combine(&J, p, plan, hi, st);
  }
  const mla_decode_args* ref = sink ? sink : (middle ? middle : recent);
  const int B = ref->batch, R = ref->s_q * ref->num_heads, d_c = ref->cache.d_c;
  const size_t rows = (size_t)B * R;
  float* part_o = (float*)workspace;
  float* part_lse = (float*)((char*)workspace + m.lse_off);
  // each part's decode leaves its split partials in its own workspace region; one
  // log-sum-exp merge then reads all of them (a part with no token for a sequence contributes
  // nothing; a sequence with no token at all gets o = 0 and lse = -inf)
  mla::CombinePartsParams c{};
  int n = 0;
  for (int i = 0; i < 3; ++i) {
    if (parts[i] == nullptr) continue;
    mla_decode_args p = part_args(parts[i], i == 2);
    p.o_lat = part_o + (size_t)n * rows * d_c;
    p.lse = part_lse + (size_t)n * rows;
    p.workspace = (char*)workspace + m.dec_off[i];
    p.workspace_bytes = workspace_bytes - m.dec_off[i];
    s = decode_paged(&p, false, stream, &c.part[n]);
    if (s != MLA_OK) return s;
    ++n;
  }
  c.n_parts = n;
  for (int i = 0; i < n; ++i) c.many_parts |= c.part[i].many;
  c.B = B;
  c.R = R;
  c.d_c = d_c;
  c.out = o_lat;
  c.out_bf16 = o_dtype == MLA_BF16;
  c.out_lse = lse;
  return hip_status(mla::launch_combine_parts(c, st));
}

int32_t mla_append_kv(const void* c_new, int64_t c_stride, const void* k_rope_new, int64_t k_stride,
                      int32_t in_dtype, const int32_t* slots, int64_t n, void* cache_pool, int64_t num_blocks,
                      const mla_cache_desc* desc, void* stream) {
  Layout lay;
  if (n < 0 || num_blocks <= 0 || !valid_dtype(in_dtype)) return MLA_ERR_INVALID_ARG;
  if (!cache_layout(desc, &lay)) return MLA_ERR_INVALID_ARG;
  if (n == 0) return MLA_OK;
  if (!c_new || !k_rope_new || !slots || !cache_pool) return MLA_ERR_INVALID_ARG;
  if (c_stride < desc->d_c || k_stride < desc->d_r) return MLA_ERR_INVALID_ARG;
  const int esz = in_dtype == MLA_F32 ? 4 : 2;
  if (!aligned(c_new, esz) || !aligned(k_rope_new, esz) || !aligned(slots, 4) || !aligned(cache_pool, 16))
    return MLA_ERR_INVALID_ARG;
  if (n > (1LL << 31) - 1) return MLA_ERR_UNSUPPORTED;
  if (!is_float_fmt(desc->latent_fmt)) {
    // one lane per 8 channels; a group is a power-of-two number of lanes within a wavefront
    auto lanes_ok = [](int d, int g) {
      const int l = g / 8;
      return d % 8 == 0 && g % 8 == 0 && l <= 64 && (l & (l - 1)) == 0;
    };
    if (!lanes_ok(desc->d_c, desc->latent_group) || !lanes_ok(desc->d_r, desc->rope_group)) return MLA_ERR_UNSUPPORTED;
  }
  mla::AppendParams p{};
  p.c = c_new;
  p.k = k_rope_new;
  p.in_f32 = in_dtype == MLA_F32;
  p.c_stride = c_stride;
  p.k_stride = k_stride;
  p.slots = slots;
  p.n = n;
  p.pool = (uint8_t*)cache_pool;
  p.num_blocks = num_blocks;
  p.block_bytes = lay.block_bytes;
  p.off_lc = lay.off[0];
  p.off_ls = lay.off[1];
  p.off_rc = lay.off[2];
  p.off_rs = lay.off[3];
  p.d_c = desc->d_c;
  p.d_r = desc->d_r;
  p.g_lat = desc->latent_group > 0 ? desc->latent_group : 1;
  p.g_rope = desc->rope_group > 0 ? desc->rope_group : 1;
  p.fmt_lat = desc->latent_fmt;
  p.fmt_rope = desc->rope_fmt;
  return hip_status(mla::launch_append(p, (hipStream_t)stream));
}

int32_t mla_hadamard_rotate(void* x, int32_t dtype, int32_t d, int64_t elem_stride, int64_t n_outer,
                            int64_t outer_stride, int64_t n_inner, int64_t inner_stride, void* stream) {
  if (!valid_dtype(dtype) || d < 2 || d > 4096 || (d & (d - 1)) != 0) return MLA_ERR_INVALID_ARG;
  if (elem_stride < 1 || n_outer < 0 || n_inner < 1 || outer_stride < 0 || inner_stride < 0)
    return MLA_ERR_INVALID_ARG;
  if (n_outer == 0) return MLA_OK;
  if (x == nullptr || !aligned(x, dtype == MLA_F32 ? 4 : 2)) return MLA_ERR_INVALID_ARG;
  if (n_outer > (1LL << 40) / n_inner) return MLA_ERR_UNSUPPORTED;
  mla::RotateParams p{};
  p.x = x;
  p.f32 = dtype == MLA_F32;
  p.d = d;
  int l = 0;
  while ((1 << l) < d) ++l;
  p.log2d = l;
  p.elem_stride = elem_stride;
  p.n_inner = n_inner;
  p.inner_stride = inner_stride;
  p.outer_stride = outer_stride;
  p.n_vec = n_outer * n_inner;
  p.vecs_per_group = d >= 2048 ? 1 : 2048 / d;
  if (ceil_div(p.n_vec, p.vecs_per_group) > (1LL << 31) - 1) return MLA_ERR_UNSUPPORTED;
  p.scale = (float)(1.0 / std::sqrt((double)d));
  p.vec8 = elem_stride == 1 && d >= 8 && aligned(x, 16) && outer_stride % 8 == 0 && inner_stride % 8 == 0;
  return hip_status(mla::launch_rotate(p, (hipStream_t)stream));
}

int64_t mla_gqa_block_bytes(int32_t num_groups, int32_t d_n, int32_t d_v, int32_t d_r) {
  if (num_groups <= 0 || d_n <= 0 || d_v <= 0 || d_r <= 0) return -1;
  return (int64_t)kBlock * 2 * ((int64_t)num_groups * (d_n + d_v) + d_r);
}

int32_t mla_gqa_expand(const void* c_new, int64_t c_stride, const void* k_rope_new, int64_t k_stride,
                       const void* w_uk_g, const void* w_uv_g, int32_t num_groups, int32_t d_c, int32_t d_n,
                       int32_t d_v, int32_t d_r, const int32_t* slots, int64_t n, void* cache_pool,
                       int64_t num_blocks, void* stream) {
  if (n < 0 || num_blocks <= 0 || num_groups <= 0 || d_c <= 0) return MLA_ERR_INVALID_ARG;
  const int64_t bb = mla_gqa_block_bytes(num_groups, d_n, d_v, d_r);
  if (bb < 0) return MLA_ERR_INVALID_ARG;
  if (d_n != 128 || d_v != 128 || d_r != 64 || d_c % 32 != 0) return MLA_ERR_UNSUPPORTED;
  if (n == 0) return MLA_OK;
  if (!c_new || !k_rope_new || !w_uk_g || !w_uv_g || !slots || !cache_pool) return MLA_ERR_INVALID_ARG;
  if (c_stride < d_c || k_stride < d_r || c_stride % 8 || k_stride % 8) return MLA_ERR_INVALID_ARG;
  if (!aligned(c_new, 16) || !aligned(k_rope_new, 16) || !aligned(w_uk_g, 16) || !aligned(w_uv_g, 16) ||
      !aligned(slots, 4) || !aligned(cache_pool, 16))
    return MLA_ERR_INVALID_ARG;
  if (ceil_div(n, 16) * num_groups > (1LL << 31) - 1) return MLA_ERR_UNSUPPORTED;
  mla::GqaExpandParams p{};
  p.c = c_new;
  p.k = k_rope_new;
  p.c_stride = c_stride;
  p.k_stride = k_stride;
  p.w_uk = w_uk_g;
  p.w_uv = w_uv_g;
  p.G = num_groups;
  p.d_c = d_c;
  p.slots = slots;
  p.n = n;
  p.pool = (uint8_t*)cache_pool;
  p.num_blocks = num_blocks;
  p.block_bytes = bb;
  return hip_status(mla::launch_gqa_expand(p, (hipStream_t)stream));
}

int32_t mla_gqa_workspace_size(const mla_gqa_args* a, size_t* bytes) {
  const int32_t s = validate_gqa(a);
  if (s != MLA_OK) return s;
  if (bytes == nullptr) return MLA_ERR_INVALID_ARG;
  int cus = 0;
  if (a->num_splits == 0) {
    const int32_t e = device_cus(&cus);
    if (e != MLA_OK) return e;
  }
  *bytes = gqa_partial_bytes(a, gqa_plan(a, cus));
  return MLA_OK;
}

int32_t mla_gqa_decode_paged(const mla_gqa_args* a, void* stream) {
  int32_t s = validate_gqa(a);
  if (s != MLA_OK) return s;
  int cus = 0;
  if (a->num_splits == 0) {
    s = device_cus(&cus);
    if (s != MLA_OK) return s;
  }
  const GqaPlan plan = gqa_plan(a, cus);
  const size_t need = gqa_partial_bytes(a, plan);
  if (need > 0 && (a->workspace == nullptr || a->workspace_bytes < need || !aligned(a->workspace, 256)))
    return MLA_ERR_WORKSPACE;
  const int R = a->s_q * a->num_heads;
  const bool split = plan.splits > 1;
  mla::GqaParams p{};
  p.q_nope = a->q_nope;
  p.q_rope = a->q_rope;
  p.pool = (const uint8_t*)a->cache_pool;
  p.num_blocks = a->num_blocks;
  p.block_bytes = mla_gqa_block_bytes(a->num_groups, a->d_n, a->d_v, a->d_r);
  p.block_table = a->block_table;
  p.bt_stride = a->block_table_stride;
  p.seq_lens = a->seq_lens;
  p.max_seq_len = a->max_seq_len;
  p.B = a->batch;
  p.s_q = a->s_q;
  p.H = a->num_heads;
  p.G = a->num_groups;
  p.max_chunks = plan.splits;
  p.tpc = plan.tpc;
  const int64_t units = (int64_t)a->batch * plan.splits * a->num_groups;
  if (units > (1LL << 30)) return MLA_ERR_UNSUPPORTED;
  p.total_units = (int)units;
  p.units_per_xcd = (int)ceil_div(units, 8);
  p.scale_log2 = a->sm_scale * 1.4426950408889634f;
  float* part_o = split ? (float*)a->workspace : nullptr;
  float* part_lse = split ? (float*)((char*)a->workspace + align_up((int64_t)a->batch * plan.splits * R * a->d_v * 4, 256))
                          : nullptr;
  p.out = split ? part_o : a->out;
  p.out_lse = split ? part_lse : a->lse;
  hipStream_t st = (hipStream_t)stream;
  hipError_t e = mla::launch_gqa_decode(p, plan.rt, st);
  if (e != hipSuccess) return MLA_ERR_HIP;
  if (split) {
    mla::CombineParams c{};
    c.part_o = part_o;
    c.part_lse = part_lse;
    c.seq_lens = a->seq_lens;
    c.max_seq_len = a->max_seq_len;
    c.R = R;
    c.d_c = a->d_v;
    c.max_chunks = plan.splits;
    c.tpc = plan.tpc;
    c.out = a->out;
    c.out_bf16 = 0;
    c.out_lse = a->lse;
    c.many_parts = plan.splits > 16;
    e = mla::launch_combine(c, a->batch, st);
    if (e != hipSuccess) return MLA_ERR_HIP;
  }
  return MLA_OK;
}

int32_t mla_dequant_blocks(const void* cache_pool, int64_t num_blocks, const mla_cache_desc* desc,
                           const int32_t* block_ids, int32_t n_blocks, int32_t family, void* out_bf16,
                           void* stream) {
  Layout lay;
  if (!cache_pool || !block_ids || !out_bf16 || n_blocks <= 0 || num_blocks <= 0) return MLA_ERR_INVALID_ARG;
  if (family != MLA_DEQUANT_PARTITION && family != MLA_DEQUANT_ROWS) return MLA_ERR_INVALID_ARG;
  if (!cache_layout(desc, &lay)) return MLA_ERR_INVALID_ARG;
  if (!aligned(cache_pool, 16) || !aligned(out_bf16, 16) || !aligned(block_ids, 4)) return MLA_ERR_INVALID_ARG;
  if (desc->latent_fmt != MLA_FMT_F32 && !decode_supported(desc, MLA_BF16)) return MLA_ERR_UNSUPPORTED;
  mla::DequantParams p{};
  p.pool = (const uint8_t*)cache_pool;
  p.num_blocks = num_blocks;
  p.block_bytes = lay.block_bytes;
  p.off_lc = lay.off[0];
  p.off_ls = lay.off[1];
  p.off_rc = lay.off[2];
  p.off_rs = lay.off[3];
  p.g_lat = desc->latent_group > 0 ? desc->latent_group : 1;
  p.g_rope = desc->rope_group > 0 ? desc->rope_group : 1;
  p.d_c = desc->d_c;
  p.d_r = desc->d_r;
  p.ids = block_ids;
  p.n = n_blocks;
  p.out = (uint16_t*)out_bf16;
  p.family = family;
  if ((int64_t)n_blocks * 2 > (1LL << 31) - 1) return MLA_ERR_UNSUPPORTED;
  return hip_status(mla::launch_dequant(p, desc->latent_fmt, (hipStream_t)stream));
}

}  // extern "C"
