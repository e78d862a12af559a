// Internal declarations shared by the host planner (mlra_host.cpp) and the
// HIP kernels (mlra_kernels.hip). Nothing here is part of the public ABI.
#pragma once

#include <stdint.h>

#include "mlra.h"

namespace mlra {

constexpr int kBlock = 64;      // tokens per cache block (= one split-K tile)
constexpr int kMaxSeqs = 65535;  // grid y limit
constexpr int kSub = 32;        // tokens per MFMA sub-tile (M of the 32x32 MFMA)

// Workgroup shape of the bf16 MFMA split kernel (latent widths 256 and 512),
// shared by planner and launcher. One workgroup fills one CU: 2 waves per SIMD
// when a wave holds 32 query rows of a latent of at most 128 (4 SIMDs -> 8
// waves), else 1 per SIMD (the width-split score exchange needs more than the
// 256 registers two waves per SIMD leave). Its waves split the branches (NB),
// the latent width (WD, 128 columns per wave) and the workgroup's tiles (WT).
constexpr int mfma_wd(int DC) { return DC == 512 ? 4 : (DC == 256 ? 2 : 1); }
constexpr int mfma_waves_per_simd(int NT, int DC) { return (NT == 1 && DC <= 128) ? 2 : 1; }
// 32-token sub-tiles each wave keeps in flight in registers (48 VGPRs each at
// DC = 128, DR = 64); a wave requests PD sub-tiles ahead of the one it computes.
// With two row tiles a CU runs only 4 waves, so each requests two ahead.
constexpr int mfma_pd(int NT, int DC) { return (NT == 2 && DC != 512) ? 2 : 1; }
// Query rows in each wave's registers (true) or staged once per workgroup in LDS.
constexpr bool mfma_qreg(int NT, int /*DC*/) { return NT == 1; }
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
  kVariantValuFp32 = 1,  // float32 inputs: one wave per (row, branch), vector ALU
  kVariantMfmaBf16 = 2,  // bfloat16, latent 256/512: 32x32x16 bf16 MFMA, waves split the width
  kVariantPcBf16 = 4,    // bfloat16, latent 64/128: loader waves fill an LDS ring for compute waves
};

// Loader/compute kernel: block ids of one split are staged in LDS, so a split
// holds at most kPcMaxTiles 64-token tiles (the planner splits longer runs).
constexpr int kPcMaxTiles = 1024;
// A workgroup holds RT 32-row tiles of query rows (1 up to 32 rows, 2 up to
// 64) and NBW of the NB branches: all of them with one row tile; with two,
// at most two, so that its four compute waves cover every (branch, row tile)
// pair; four branches then take two workgroups per split (branch groups).
constexpr int pc_rt(int rows) { return rows > 32 ? 2 : 1; }
constexpr int pc_nbw(int NB, int rows) { return rows > 32 && NB > 2 ? 2 : NB; }
// LDS layout (byte offsets): ring [nslot][slot_bytes] at 0 (a slot holds the
// NBW latents and the RoPE key of 32 tokens; the staged query rows, RT
// slots' worth, alias it), then the merge records of every token stream but
// the merging one of each (branch, row tile) pair (P * (4/P - 1) records of
// (DC/32 * 4 + 1) x 64 x 16 bytes, P = NBW * RT; none when P = 4), then the
// block ids, then the counters ready[nslot], consumed[nslot], qdone,
// recorded[P].
struct PcLds {
  int32_t slot_bytes, nslot, merge, table, flags, total;
};
constexpr PcLds pc_lds(int NBW, int RT, int DC, int DR) {
  const int slot = (NBW * kSub * (DC / 8 + 2) + kSub * (DR / 8 + 1)) * 16;
  const int fixed = kPcMaxTiles * 4 + 256;
  const int P = NBW * RT;
  const int rec = P * (4 / P - 1) * ((DC / 32) * 4 + 1) * 64 * 16;
  int nslot = (160 * 1024 - fixed - rec) / slot;
  if (nslot > 12) nslot = 12;
  const int ring = nslot * slot;
  const int qry = RT * slot;  // the query rows use RT slots' layout
  const int front = ring > qry ? ring : qry;
  return PcLds{slot, nslot, front, front + rec, front + rec + kPcMaxTiles * 4, front + rec + fixed};
}
// Sub-tiles each loader keeps in flight: about kPcLoaderKB KB of loads per
// loader, 48 KB per CU (measured best of 36..72 KB at B=16, T=8192). A CU
// accepts some 32-48 KB of outstanding loads before issue starts to stall;
// a loader stalled in issue cannot hand over slots whose data has arrived.
constexpr int kPcLoaderKB = 12;
constexpr int pc_pl(int NBW, int DC, int DR) {
  const int nload = NBW * (DC / 16) + DR / 16;  // 16-byte-per-lane loads per sub-tile
  const int per = (nload + 3) / 4;
  const int pl = (kPcLoaderKB + per - 1) / per;
  return pl < 2 ? 2 : (pl > 12 ? 12 : pl);
}



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
  int32_t NRT;      // workgroups per split: one per 32 query rows (width-split kernel),
                    // one per branch group (loader/compute kernel); 1 or 2
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
  if (mfma_slotted(WD, WT, qreg)) {
    const int stage = 32 * (lp + rp) * 16;
    const int rec = (NT * (DCW / 32) * 4 + 1) * 64 * 16;
    return waves * (stage > rec ? stage : rec);
  }
  const int stage = waves * 32 * lp * 16 + NB * WT * 32 * rp * 16;
  const int qry = qreg ? 0 : (NB * WD * lp + rp) * NT * 32 * 16;
  const int xchg = (WD > 1) ? NB * WT * WD * NT * 64 * 16 * 4 : 0;
  const int ndt = DCW / 32;
  const int merge = (WT > 1) ? WT * NB * WD * 64 * (NT * ndt * 16 + 4) * 4 : 0;
  const int loop = stage + qry + xchg;
  return loop > merge ? loop : merge;
}

mlra_status resolve_dims(const mlra_decode_dims* d, int32_t n_branch, Resolved* r);
KernelShape choose_shape(const Resolved& r);
mlra_status plan_call(const Resolved& r, const KernelShape& k, int32_t num_cus,
                      int32_t num_splits, int64_t sum_seq_lens, mlra_decode_plan* plan);

}  // namespace mlra
