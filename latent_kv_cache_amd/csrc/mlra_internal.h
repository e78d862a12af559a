// Internal declarations shared by the host planner (mlra_host.cpp) and the
// HIP kernels (mlra_kernels.hip). Nothing here is part of the public ABI.
#pragma once

#include <stdint.h>

#include "mlra.h"

namespace mlra {

constexpr int kBlock = 64;      // tokens per cache block (= one split-K tile)
constexpr int kSub = 32;        // tokens per MFMA sub-tile (M of the 32x32 MFMA)
constexpr int kLdsPad = 8;      // bf16 elements of padding per LDS latent row

enum Variant : int32_t {
  kVariantValuFp32 = 1,  // float32 inputs: one wave per (row, branch), vector ALU
  kVariantMfmaBf16 = 2,  // bfloat16 inputs: 32x32x16 bf16 MFMA, LDS transpose for P.C
};

// Dims after validation, with defaults resolved.
struct Resolved {
  int32_t S, Q, H, rows, NB, DC, DR;
  int32_t max_blocks, num_blocks, max_seq_len, lcap, causal, dtype, reduce;
  int64_t lsb, lst, lsbr;  // latent strides (elements): block, token, branch
  int64_t rsb, rst;        // rope strides (elements): block, token
};

// Shape of the split-kernel workgroup.
struct KernelShape {
  int32_t variant;
  int32_t NT;       // 32-row tiles of query rows (H*Q): 1 or 2
  int32_t WD;       // waves that split the latent width of one branch (DC = 512 -> 4)
  int32_t WT;       // waves that split the workgroup's tokens (merged in LDS)
  int32_t NPF;      // sub-tiles in flight per wave (register prefetch depth)
  int32_t waves;    // waves per workgroup
  int32_t groups_per_cu;  // resident workgroups per CU the planner aims for
};

// LDS bytes of one MFMA split workgroup: the per-wave latent sub-tile used for
// the LDS transpose, the score exchange when WD > 1, and (aliased over both,
// after the token loop) the cross-wave merge buffer when WT > 1.
inline int32_t mfma_lds_bytes(int NB, int DCW, int WD, int NT, int WT) {
  const int waves = NB * WD * WT;
  const int tile = waves * kSub * (DCW + kLdsPad) * 2;
  const int xchg = (WD > 1) ? 2 * NB * WT * WD * NT * 64 * 16 * 4 : 0;
  const int ndt = DCW / 32;
  const int merge = (WT > 1) ? (WT - 1) * NB * WD * 64 * (NT * ndt * 16 + 4) * 4 : 0;
  const int loop = tile + xchg;
  return loop > merge ? loop : merge;
}

mlra_status resolve_dims(const mlra_decode_dims* d, int32_t n_branch, Resolved* r);
KernelShape choose_shape(const Resolved& r);
mlra_status plan_call(const Resolved& r, const KernelShape& k, int32_t num_cus,
                      int32_t num_splits, int64_t sum_seq_lens, mlra_decode_plan* plan);

}  // namespace mlra
