// Internal declarations shared by the host planner (mlra_host.cpp) and the
// HIP kernels (mlra_kernels.hip). Nothing here is part of the public ABI.
#pragma once

#include <stdint.h>

#include "mlra.h"

namespace mlra {

constexpr int kBlock = 64;      // tokens per cache block (= one split-K tile)
constexpr int kMaxSeqs = 65535;  // grid y limit
constexpr int kSub = 32;        // tokens per MFMA sub-tile (M of the 32x32 MFMA)

// Workgroup shape of the bf16 MFMA split kernel, shared by planner and
// launcher. One workgroup fills one CU: 2 waves per SIMD when a wave holds 32
// query rows (4 SIMDs -> 8 waves), 1 per SIMD with 64 rows or the 512-wide
// latent. Its waves split the branches (NB), the latent width (WD) and the
// workgroup's tiles (WT).
constexpr int mfma_wd(int DC) { return DC == 512 ? 4 : 1; }
constexpr int mfma_waves_per_simd(int NT, int DC) { return (NT == 1 && DC != 512) ? 2 : 1; }
// 32-token sub-tiles each wave keeps in flight in registers (48 VGPRs each at
// DC = 128, DR = 64): a wave requests PD sub-tiles before it computes the
// first, and refills each buffer as soon as it is staged in LDS.
constexpr int mfma_pd(int /*NT*/, int /*DC*/) { return 2; }
// Query rows in each wave's registers (true: 48 VGPRs at DC = 128) or read
// from the staged copy in LDS before each MFMA (false). With two sub-tiles in
// flight only the 512-wide latent (one wave per SIMD) has room for them.
constexpr bool mfma_qreg(int NT, int DC) { return NT == 1 && DC == 512; }
constexpr int mfma_wt(int NB, int DC, int NT) {
  return 4 * mfma_waves_per_simd(NT, DC) / (NB * mfma_wd(DC)) > 0
             ? 4 * mfma_waves_per_simd(NT, DC) / (NB * mfma_wd(DC))
             : 1;
}
// Staged row pitches in 16-byte chunks: latent rows get 2 spare chunks, RoPE
// rows 1 (see the kernel for the bank analysis).
constexpr int mfma_lpitch(int DCW) { return DCW / 8 + 2; }
constexpr int mfma_rpitch(int DR) { return DR / 8 + 1; }

enum Variant : int32_t {
  kVariantValuFp32 = 1,    // float32 inputs: one wave per (row, branch), vector ALU
  kVariantMfmaBf16 = 2,    // bfloat16, latent 512: 32x32x16 bf16 MFMA, waves split the width
  kVariantStreamBf16 = 3,  // bfloat16, latent 64/128: four waves, deep per-wave prefetch
};

// Streaming kernel (latent 64 or 128): 4 or 8 waves per workgroup (one or
// two per SIMD); each keeps stream_pd(NT) sub-tiles in flight. Query rows sit
// in registers when stream_qreg(NT), else in LDS.

// LDS layout of one streaming workgroup (byte offsets):
//   stage  [waves][32 rows][lpitch + rpitch chunks]  latent then RoPE sub-tile
//   query  [NB][NT*32][lpitch] latent rows, then [NT*32][rpitch] RoPE rows
//   merge  [waves][NT*DC/32*4 + 1][64 lanes] float4, when waves / NB > 1;
//          after the stages and queries if it fits, else over them.
struct StreamLds {
  int32_t stage, stage_bytes, query, merge, total;
  bool merge_aliases;
};
constexpr StreamLds stream_lds(int NB, int DC, int DR, int NT, int waves) {
  const int lp = DC / 8 + 2, rp = DR / 8 + 1;
  const int stage_bytes = kSub * (lp + rp) * 16;
  const int query = waves * stage_bytes;
  const int loop_end = query + (NB * NT * kSub * lp + NT * kSub * rp) * 16;
  const int merge_bytes = (waves / NB > 1) ? waves * (NT * (DC / 32) * 4 + 1) * 64 * 16 : 0;
  const bool fits = loop_end + merge_bytes <= 160 * 1024;
  return StreamLds{0, stage_bytes, query, fits ? loop_end : 0,
                   fits ? loop_end + merge_bytes : (loop_end > merge_bytes ? loop_end : merge_bytes),
                   !fits};
}
// Eight waves (two per SIMD, to hide each other's latencies) when their
// stages, queries and merge records fit in the CU's 160 KB of LDS.
// Two row tiles need more registers than two waves per SIMD leave.
constexpr int stream_waves(int NB, int DC, int DR, int NT) {
  return NT == 1 && stream_lds(NB, DC, DR, NT, 8).total <= 160 * 1024 ? 8 : 4;
}
// Sub-tiles in flight while a wave computes one: one at two waves per SIMD
// (eight waves keep 96 KB per CU requested), two at one wave per SIMD.
constexpr int stream_pd(int /*NT*/, int waves) { return waves == 8 ? 1 : 2; }
// Query rows in registers (48 VGPRs at DC = 128) when one row tile does;
// otherwise read from LDS per MFMA.
constexpr bool stream_qreg(int NT, int /*waves*/) { return NT == 1; }

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
  int32_t NT;       // 32-row tiles of query rows one wave holds (bf16: 1)
  int32_t NRT;      // workgroups per split, one per 32 query rows (H*Q <= 64: 1 or 2)
  int32_t WD;       // waves that split the latent width of one branch (DC = 512 -> 4)
  int32_t WT;       // waves that split the workgroup's tokens (merged in LDS)
  int32_t NPF;      // sub-tiles in flight per wave (register prefetch depth)
  int32_t waves;    // waves per workgroup
  int32_t groups_per_cu;  // resident workgroups per CU the planner aims for
};

// LDS bytes of one MFMA split workgroup:
//   latent sub-tile stage   one per wave           [32][lpitch] chunks
//   RoPE sub-tile stage     one per (wt, branch)   [32][rpitch]
//   latent query rows       one per (branch, wd)   [NT*32][lpitch]  (unless in registers)
//   RoPE query rows         one                    [NT*32][rpitch]  (unless in registers)
//   score exchange (WD > 1) [NB*WT][WD][NT][64 lanes][16 floats]
// and, aliased over all of it after the token loop, the cross-wave merge
// records when WT > 1: [WT][NB*WD][NT*NDT*4 + 1][64 lanes] float4. In the
// slotted layout (below) every wave instead owns one slot holding its latent
// and RoPE stages and, after its loop, its merge record.
// Slotted layout: with one latent stage per wave, queries in registers and a
// token-split merge, each wave's stage and merge record share one slot.
constexpr bool mfma_slotted(int WD, int WT, bool qreg) { return WD == 1 && WT > 1 && qreg; }

inline int32_t mfma_lds_bytes(int NB, int DCW, int WD, int DR, int NT, int WT, bool qreg) {
  const int waves = NB * WD * WT;
  const int lp = mfma_lpitch(DCW), rp = mfma_rpitch(DR);
  // Register-resident queries are first staged at the start of LDS.
  const int qstage = qreg ? (NB * WD * lp + rp) * NT * 32 * 16 : 0;
  if (mfma_slotted(WD, WT, qreg)) {
    const int stage = 32 * (lp + rp) * 16;
    const int rec = (NT * (DCW / 32) * 4 + 1) * 64 * 16;
    const int slots = waves * (stage > rec ? stage : rec);
    return slots > qstage ? slots : qstage;
  }
  const int stage = waves * 32 * lp * 16 + NB * WT * 32 * rp * 16;
  const int qry = qreg ? 0 : (NB * WD * lp + rp) * NT * 32 * 16;
  const int xchg = (WD > 1) ? NB * WT * WD * NT * 64 * 16 * 4 : 0;
  const int ndt = DCW / 32;
  const int merge = (WT > 1) ? WT * NB * WD * 64 * (NT * ndt * 16 + 4) * 4 : 0;
  const int loop = stage + qry + xchg;
  const int most = loop > merge ? loop : merge;
  return most > qstage ? most : qstage;
}

mlra_status resolve_dims(const mlra_decode_dims* d, int32_t n_branch, Resolved* r);
KernelShape choose_shape(const Resolved& r);
mlra_status plan_call(const Resolved& r, const KernelShape& k, int32_t num_cus,
                      int32_t num_splits, int64_t sum_seq_lens, mlra_decode_plan* plan);

}  // namespace mlra
