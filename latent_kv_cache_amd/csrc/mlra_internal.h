// Internal declarations shared by the host planner (mlra_host.cpp) and the
// HIP kernels (mlra_kernels.hip). Nothing here is part of the public ABI.
#pragma once

#include <stdint.h>

#include "mlra.h"

namespace mlra {

constexpr int kBlock = 64;      // tokens per cache block (= one split-K tile)
// Decode workspace header: a status word, then one slot per sequence of the
// in-kernel merge: kSyncSlots publication counters and kSyncSlots verdict
// counters (64-bit each). Partial results follow the header.
constexpr int kWsStatusBytes = 256;
constexpr int kSyncSeqs = 64;           // sequences the in-kernel merge handles
constexpr int kSyncSlots = 32;          // workgroups per sequence it handles
constexpr int kSyncSlotBytes = 1024;    // 2 x 32 x 8 bytes, padded
constexpr int kWsHeaderBytes = kWsStatusBytes + kSyncSeqs * kSyncSlotBytes;
static_assert(kWsHeaderBytes == MLRA_DECODE_WS_HEADER_BYTES, "header size");
static_assert(2 * kSyncSlots * 8 <= kSyncSlotBytes, "sync slot");
// Workgroups whose ids are congruent modulo this many run on the same XCD
// (the dispatcher deals workgroups to the XCDs round robin; the MI355X has 8,
// and the 1- and 4-XCD partition modes divide it).
constexpr int kXcdSlots = 8;
// Default bound of the split kernel's LDS waits, in polls.
constexpr int kDefaultWaitPolls = 1 << 22;
constexpr int kMaxSeqs = 65535;  // grid y limit
constexpr int kSub = 32;        // tokens per MFMA sub-tile (M of the 32x32 MFMA)

// Staged row pitches in 16-byte chunks: latent rows get 2 spare chunks, RoPE
// rows 1 (see the split kernel for the bank analysis).
constexpr int stage_lpitch(int DC) { return DC / 8 + 2; }
constexpr int stage_rpitch(int DR) { return DR / 8 + 1; }

enum Variant : int32_t {
  kVariantValuFp32 = 1,  // float32 inputs: one wave per (row, branch), vector ALU
  // (2: an earlier bf16 kernel for latents 256/512, replaced by variant 4)
  kVariantPcBf16 = 4,    // bfloat16: loader waves fill an LDS ring for compute waves
};

// Loader/compute kernel: block ids of one split are staged in LDS, so a split
// holds at most kPcMaxTiles 64-token tiles (the planner splits longer runs).
constexpr int kPcMaxTiles = 1024;
// Shape of a workgroup. Each of the four compute waves takes one (branch,
// 32-row tile, latent slice) triple: WD waves split a latent wider than 128
// into 128-column slices (WD = DC/128); a workgroup holds RT 32-row tiles of
// query rows (the power of two covering the call's row tiles, as far as the
// slices leave waves) and NBW of the NB branches (as many as the remaining
// waves allow). The rest goes to more workgroups per split: branch groups
// (NB / NBW) times row groups (the row tiles RT does not cover), at most 4.
constexpr int pc_wd(int DC) { return DC > 128 ? DC / 128 : 1; }
constexpr int pc_row_tiles(int rows) { return (rows + 31) / 32; }
constexpr int pc_rt(int rows, int DC) {
  return (pc_row_tiles(rows) <= 1 ? 1 : (pc_row_tiles(rows) <= 2 ? 2 : 4)) < 4 / pc_wd(DC)
             ? (pc_row_tiles(rows) <= 1 ? 1 : (pc_row_tiles(rows) <= 2 ? 2 : 4))
             : 4 / pc_wd(DC);
}
constexpr int pc_nbw(int NB, int rows, int DC) {
  return NB < 4 / (pc_rt(rows, DC) * pc_wd(DC)) ? NB : 4 / (pc_rt(rows, DC) * pc_wd(DC));
}
constexpr int pc_row_groups(int rows, int DC) {
  return (pc_row_tiles(rows) + pc_rt(rows, DC) - 1) / pc_rt(rows, DC);
}
constexpr int pc_groups(int NB, int rows, int DC) {
  return (NB / pc_nbw(NB, rows, DC)) * pc_row_groups(rows, DC);
}
// LDS layout (byte offsets): ring [nslot][slot_bytes] at 0 (a slot holds the
// NBW latents and the RoPE key of 32 tokens; the staged query rows, RT
// slots' worth, alias its END, from qoff: loaders fill the first slots
// before the compute waves have read their queries, and wait for that only
// before the first write into slot qslot or later), then the merge records of every token stream but
// the merging one of each compute wave's triple (C * (4/C - 1) records of
// (DC/WD/32 * 4 + 1) x 64 x 16 bytes, C = NBW * RT * WD; none when C = 4),
// then, with WD > 1, the partial-score exchange [2][4 waves][16 floats x 64
// lanes], then the block ids, then the counters ready[nslot],
// consumed[nslot], qdone, recorded[4], exchanged[4].
struct PcLds {
  int32_t slot_bytes, nslot, merge, xchg, table, flags, total, qoff, qslot;
};
constexpr PcLds pc_lds(int NBW, int RT, int WD, int DC, int DR) {
  const int slot = (NBW * kSub * (DC / 8 + 2) + kSub * (DR / 8 + 1)) * 16;
  const int fixed = kPcMaxTiles * 4 + 256;
  const int C = NBW * RT * WD;
  const int rec = C * (4 / C - 1) * ((DC / WD / 32) * 4 + 1) * 64 * 16;
  const int xchg = WD > 1 ? 2 * 4 * 64 * 64 : 0;
  int nslot = (160 * 1024 - fixed - rec - xchg) / slot;
  if (nslot > 12) nslot = 12;
  const int ring = nslot * slot;
  const int qry = RT * slot;  // the query rows use RT slots' layout
  const int front = ring > qry ? ring : qry;
  return PcLds{slot,
               nslot,
               front,
               front + rec,
               front + rec + xchg,
               front + rec + xchg + kPcMaxTiles * 4,
               front + rec + xchg + fixed,
               front - qry,
               (front - qry) / slot};
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
  int32_t max_blocks, num_blocks, max_seq_len, lcap, causal, dtype, reduce, flags;
  int64_t lsb, lst, lsbr;  // latent strides (elements): block, token, branch
  int64_t rsb, rst;        // rope strides (elements): block, token
};

// Shape of the split-kernel workgroup.
struct KernelShape {
  int32_t variant;
  int32_t NRT;      // workgroups per split (branch groups x row groups; 1 to 4)
  int32_t waves;    // waves per workgroup
  int32_t groups_per_cu;  // resident workgroups per CU the planner aims for
};

mlra_status resolve_dims(const mlra_decode_dims* d, int32_t n_branch, Resolved* r);
KernelShape choose_shape(const Resolved& r);
mlra_status plan_call(const Resolved& r, const KernelShape& k, int32_t num_cus,
                      int32_t num_splits, int64_t sum_seq_lens, mlra_decode_plan* plan);

}  // namespace mlra
