// Host-side validation and split-K planning for MLRA decode attention.
//
// Pure C++ (no HIP calls): argument checks, default strides, the choice of
// kernel shape and the split plan. The plan splits each sequence's 64-token
// tiles into chunks so that roughly a fixed number of workgroups fill the GPU
// (flash-decoding); each chunk yields a partial (output, log-sum-exp) per
// query row and branch that the combine kernel merges.
#include <algorithm>
#include <cmath>
#include <cstring>
#include <initializer_list>

#include "mlra_internal.h"

namespace mlra {

static bool pow2_in(int v, std::initializer_list<int> allowed) {
  for (int a : allowed)
    if (v == a) return true;
  return false;
}

mlra_status resolve_dims(const mlra_decode_dims* d, int32_t n_branch, Resolved* r) {
  if (!d || !r) return MLRA_ERR_NULL_PTR;
  if (d->dtype != MLRA_BF16 && d->dtype != MLRA_FP32) return MLRA_ERR_BAD_DIMS;
  if (d->reduce != MLRA_BRANCH_SUM && d->reduce != MLRA_BRANCH_CONCAT) return MLRA_ERR_BAD_DIMS;
  if (d->flags & ~MLRA_DECODE_FLAG_FUSED_MERGE) return MLRA_ERR_BAD_DIMS;
  if (d->num_seqs < 1 || d->num_heads < 1 || d->q_len < 1) return MLRA_ERR_BAD_DIMS;
  if (d->num_seqs > kMaxSeqs) return MLRA_ERR_UNSUPPORTED;  // grid y dimension
  if (d->q_len > 4) return MLRA_ERR_UNSUPPORTED;
  if (d->num_heads * d->q_len > 128) return MLRA_ERR_UNSUPPORTED;
  if (n_branch < 1) return MLRA_ERR_BAD_DIMS;
  if (!pow2_in(n_branch, {1, 2, 4})) return MLRA_ERR_UNSUPPORTED;
  if (d->d_latent < 1 || d->d_rope < 1) return MLRA_ERR_BAD_DIMS;
  if (!pow2_in(d->d_rope, {32, 64})) return MLRA_ERR_UNSUPPORTED;
  if (d->dtype == MLRA_BF16) {
    if (!pow2_in(d->d_latent, {64, 128, 256, 512})) return MLRA_ERR_UNSUPPORTED;
    if (d->d_latent == 512 && (n_branch != 1 || d->d_rope != 64)) return MLRA_ERR_UNSUPPORTED;
    if (d->d_latent == 256 && (n_branch > 2 || d->d_rope != 64)) return MLRA_ERR_UNSUPPORTED;
  } else {
    if (!pow2_in(d->d_latent, {64, 128, 256, 512})) return MLRA_ERR_UNSUPPORTED;
  }
  if (d->block_size != kBlock) return d->block_size < 1 ? MLRA_ERR_BAD_DIMS : MLRA_ERR_UNSUPPORTED;
  if (d->max_blocks_per_seq < 1 || d->num_blocks < 1) return MLRA_ERR_BAD_DIMS;
  if (d->max_seq_len < 0) return MLRA_ERR_BAD_DIMS;
  if ((int64_t)d->max_seq_len > (int64_t)d->max_blocks_per_seq * kBlock) return MLRA_ERR_BAD_DIMS;
  if (d->num_splits < 0 || d->sum_seq_lens < 0) return MLRA_ERR_BAD_DIMS;
  if (d->sum_seq_lens > (int64_t)d->num_seqs * d->max_seq_len) return MLRA_ERR_BAD_DIMS;

  Resolved o;
  o.S = d->num_seqs;
  o.Q = d->q_len;
  o.H = d->num_heads;
  o.rows = d->num_heads * d->q_len;
  o.NB = n_branch;
  o.DC = d->d_latent;
  o.DR = d->d_rope;
  o.max_blocks = d->max_blocks_per_seq;
  o.num_blocks = d->num_blocks;
  o.max_seq_len = d->max_seq_len;
  o.lcap = d->max_seq_len;
  o.causal = d->causal ? 1 : 0;
  o.dtype = d->dtype;
  o.reduce = d->reduce;
  o.flags = d->flags;
  o.lsbr = d->latent_stride_branch ? d->latent_stride_branch : o.DC;
  o.lst = d->latent_stride_token ? d->latent_stride_token : (int64_t)o.NB * o.DC;
  o.lsb = d->latent_stride_block ? d->latent_stride_block : (int64_t)kBlock * o.lst;
  o.rst = d->rope_stride_token ? d->rope_stride_token : o.DR;
  o.rsb = d->rope_stride_block ? d->rope_stride_block : (int64_t)kBlock * o.rst;
  if (o.lsbr < 0 || o.lst < 0 || o.lsb < 0 || o.rst < 0 || o.rsb < 0) return MLRA_ERR_BAD_DIMS;
  // Token-major ([blk][64][NB][DC]) and branch-major ([blk][NB][64][DC]) are
  // both accepted: strides must be positive and one block's rows must fit
  // inside the block stride, so distinct blocks never overlap.
  if ((o.NB > 1 && o.lsbr < 1) || o.lst < 1 || o.rst < 1) return MLRA_ERR_BAD_DIMS;
  if (o.lsb < (int64_t)(kBlock - 1) * o.lst + (int64_t)(o.NB - 1) * o.lsbr + o.DC)
    return MLRA_ERR_BAD_DIMS;
  if (o.rsb < (int64_t)(kBlock - 1) * o.rst + o.DR) return MLRA_ERR_BAD_DIMS;
  // Byte offsets inside one block are 32-bit on the device.
  if ((o.lsb - 0) * (o.dtype == MLRA_BF16 ? 2 : 4) >= (int64_t(1) << 31) ||
      o.rsb * (o.dtype == MLRA_BF16 ? 2 : 4) >= (int64_t(1) << 31))
    return MLRA_ERR_UNSUPPORTED;
  // 16-byte rule for every stride.
  const int64_t vec = (o.dtype == MLRA_BF16) ? 8 : 4;
  if (o.lsbr % vec || o.lst % vec || o.lsb % vec || o.rst % vec || o.rsb % vec)
    return MLRA_ERR_ALIGNMENT;
  *r = o;
  return MLRA_OK;
}

static int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

KernelShape choose_shape(const Resolved& r) {
  KernelShape k{};
  if (r.dtype == MLRA_FP32) {
    k.variant = kVariantValuFp32;
    k.NRT = 1;
    k.waves = 4;  // four (row, branch) pairs per workgroup
    k.groups_per_cu = 2;
    return k;
  }
  // Loader/compute kernel: four loader waves and four compute waves, each
  // compute wave one (branch, 32-row tile, 128-column latent slice) triple;
  // any tile count per split (up to kPcMaxTiles). A workgroup reads only its
  // own branches' latents: the groups of a split (branch groups, or row
  // groups for the 512-wide latent at 64 rows) are XCD-paired and share the
  // rest through L2.
  k.variant = kVariantPcBf16;
  k.NRT = pc_groups(r.NB, r.rows, r.DC);
  k.waves = 8;
  k.groups_per_cu = 1;  // one workgroup fills a CU
  return k;
}

// Tiles per split that minimise the estimated makespan of the split kernel:
// rounds * (tiles per split + a fixed per-workgroup cost), where a round is
// one workgroup on each of the target_groups slots. The fixed cost counts
// the prologue and merge (about two tiles of streaming) plus writing and
// re-reading the workgroup's fp32 partial results, in tile-sized units. Sequence lengths live on
// the device, so the number of non-empty workgroups is estimated from the
// host-side hints: exact when every sequence has max_seq_len (sum_seq_lens =
// S * max_seq_len, or no hint), otherwise the batch's tiles / tps plus half a
// workgroup of rounding per sequence. Ties go to the larger split (fewer
// partial results to combine).
static int64_t choose_tiles_per_split(const Resolved& r, const KernelShape& k,
                                      int64_t slots, int64_t max_tiles, int64_t sum_seq_lens) {
  const int64_t elem = r.dtype == MLRA_BF16 ? 2 : 4;
  // one workgroup's share: its branches' tiles and partial results
  const int nbw = k.variant == kVariantPcBf16 ? pc_nbw(r.NB, r.rows, r.DC) : r.NB;
  const int row_groups = k.NRT / (r.NB / nbw);
  const double tile_bytes = (double)kBlock * (nbw * r.DC + r.DR) * elem;
  const double partial_bytes = (double)nbw * (r.rows / row_groups) * (r.DC + 1) * 4;
  const double fixed = 2.0 + 2.0 * partial_bytes / tile_bytes;
  const bool uniform = sum_seq_lens <= 0 || sum_seq_lens >= (int64_t)r.S * r.lcap;
  const int64_t total = uniform ? (int64_t)r.S * max_tiles : cdiv(sum_seq_lens, kBlock);
  int64_t top = std::max<int64_t>(max_tiles, 1);
  if (k.variant == kVariantPcBf16) top = std::min<int64_t>(top, kPcMaxTiles);
  int64_t best = top;
  double best_cost = -1.0;
  for (int64_t tps = top; tps >= 1; --tps) {
    const int64_t groups = k.NRT * (uniform ? (int64_t)r.S * cdiv(max_tiles, tps)
                                            : cdiv(total, tps) + cdiv(r.S, 2));
    const double cost =
        (double)cdiv(std::max<int64_t>(groups, 1), slots) * ((double)tps + fixed);
    if (best_cost < 0 || cost < best_cost * 0.999) {
      best_cost = cost;
      best = tps;
    }
    if (groups > 64 * slots) break;  // finer splits only add rounds
  }
  return best;
}

mlra_status plan_call(const Resolved& r, const KernelShape& k, int32_t num_cus,
                      int32_t num_splits, int64_t sum_seq_lens, mlra_decode_plan* plan) {
  if (!plan) return MLRA_ERR_NULL_PTR;
  if (num_cus < 1) return MLRA_ERR_BAD_DIMS;
  mlra_decode_plan p;
  std::memset(&p, 0, sizeof(p));
  p.num_cus = num_cus;
  p.waves_per_group = k.waves;
  p.kernel_variant = k.variant;

  const int64_t max_tiles = cdiv(r.lcap, kBlock);
  int64_t tps;
  if (k.variant == kVariantValuFp32) {
    // One workgroup covers 4 (row, branch) pairs; groups along the pairs
    // multiply the split count.
    const int64_t pair_groups = cdiv((int64_t)r.rows * r.NB, k.waves);
    p.target_groups = (int32_t)std::max<int64_t>(1, (int64_t)num_cus * k.groups_per_cu / pair_groups);
  } else {
    p.target_groups = num_cus * k.groups_per_cu;
  }
  if (num_splits > 0) {
    tps = cdiv(std::max<int64_t>(max_tiles, 1), num_splits);
    // The loader/compute kernel stages a split's block ids in LDS: a request
    // for fewer splits than that allows is raised.
    if (k.variant == kVariantPcBf16) tps = std::min<int64_t>(tps, kPcMaxTiles);
  } else {
    tps = choose_tiles_per_split(r, k, p.target_groups, max_tiles, sum_seq_lens);
  }
  const int64_t spl = std::max<int64_t>(1, cdiv(max_tiles, tps));
  if (spl > 65535 || tps > (1 << 24) || (int64_t)r.S * spl * k.NRT > (1 << 28))
    return MLRA_ERR_UNSUPPORTED;
  p.tiles_per_split = (int32_t)tps;
  p.splits_per_seq = (int32_t)spl;
  p.row_groups = k.NRT;
  p.lds_bytes = k.variant == kVariantPcBf16
                    ? pc_lds(pc_nbw(r.NB, r.rows, r.DC), pc_rt(r.rows, r.DC), pc_wd(r.DC), r.DC, r.DR).total
                    : 0;
  // In-kernel merge (when asked for): every workgroup of a sequence on one XCD (sequence s on
  // the ids congruent to s mod kXcdSlots), all workgroups resident at once
  // (one per CU), and a length bound shared by the batch (the hint, when
  // given, says every sequence reaches it: a ragged batch would load the
  // XCDs unevenly).
  const int64_t per = spl * k.NRT;
  const bool uniform = sum_seq_lens <= 0 || sum_seq_lens >= (int64_t)r.S * r.lcap;
  p.fused_merge = k.variant == kVariantPcBf16 && (r.flags & MLRA_DECODE_FLAG_FUSED_MERGE) &&
                  uniform && r.S % kXcdSlots == 0 && r.S <= kSyncSeqs && per <= kSyncSlots &&
                  (int64_t)r.S * per <= num_cus && per * kXcdSlots <= num_cus;
  // Header, then partials: output [S][spl][NB][rows][DC] and lse
  // [S][spl][NB][rows], fp32.
  const int64_t slots = (int64_t)r.S * spl * r.NB * r.rows;
  const int64_t o_bytes = cdiv(slots * r.DC * 4, 256) * 256;
  const int64_t l_bytes = cdiv(slots * 4, 256) * 256;
  p.workspace_bytes = (size_t)(kWsHeaderBytes + o_bytes + l_bytes);
  *plan = p;
  return MLRA_OK;
}

}  // namespace mlra

extern "C" const char* mlra_status_string(mlra_status s) {
  switch (s) {
    case MLRA_OK: return "ok";
    case MLRA_ERR_NULL_PTR: return "a required pointer is NULL";
    case MLRA_ERR_BAD_DIMS: return "a size is out of range or inconsistent";
    case MLRA_ERR_UNSUPPORTED: return "valid, but no kernel is built for this shape";
    case MLRA_ERR_WORKSPACE: return "workspace is NULL or smaller than required";
    case MLRA_ERR_ALIGNMENT: return "a pointer or stride breaks the 16-byte rule";
    case MLRA_ERR_HIP: return "a HIP runtime call or kernel launch failed";
  }
  return "unknown status";
}

extern "C" int32_t mlra_version(void) { return 100; }  // 0.1.0
