// HIP kernels and C-ABI entry points for MLRA decode attention on gfx950.
//
// Method (wispaper.ai blog "MLRA: Breaking the Sharding Bottleneck in Latent
// Attention", "The Core Insight: Sum of Branches, Not Sum of Keys"): every
// latent branch b runs its own softmax attention over the cached latents and
// the branch outputs are summed afterwards, then multiplied by a fixed factor
// ("Mathematical Calibration: Scaling the Latents"). Keys are scored in
// absorbed form against the cached latent c_b[t] plus one decoupled RoPE key
// k_r[t] shared by all branches.
//
// Decode is bound by moving the cache from HBM (arXiv 2603.02188 abstract), so
// the split kernel streams each cache byte once per workgroup that needs it:
//   * one workgroup per (sequence, split, group); a split is a run of 64-token
//     tiles (one cache block each); four loader waves stream its 32-token
//     sub-tiles into a ring of LDS slots and four compute waves take them,
//     each one (branch, 32-row tile, 128-column latent slice) triple;
//   * S^T = C . Q^T on v_mfma_f32_32x32x16_bf16 with the slot rows as the A
//     operand (lane (m, g) reads 8 consecutive features of token m) and the
//     query rows in registers as B; the score tile lands with the query row
//     along the lanes, so the online softmax is lane-local plus one
//     v_permlane32_swap for the row max, and the probabilities are already in
//     B-operand order for O^T += C^T . P^T, whose A operand (tokens along K)
//     comes from transposing LDS reads of the same slot;
//   * each (split, branch, row) writes a partial (output / l, lse); the combine
//     kernel merges the splits with the log-sum-exp rule, sums the branches
//     (or lays them side by side) and applies the output factor.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <cmath>

#include "mlra_device.h"
#include "mlra_internal.h"

namespace mlra {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.69314718055994531f;
// Lazy softmax reference: probabilities exp2(score - m_ref) stay below
// 2^kLazyLog2 = 256 (exact in fp32 accumulation and bf16 operands).
constexpr float kLazyLog2 = 8.0f;

struct SplitParams {
  const void* q_lat;
  const void* q_rope;
  const void* lat;
  const void* rope;
  const int32_t* table;
  const int32_t* seq_lens;
  float* part_o;    // [S][spl][NB][rows][DC]
  float* part_lse;  // [S][spl][NB][rows]
  unsigned* status;  // workspace status word (MLRA_DEVSTATUS_* bits)
  // in-kernel merge: per-sequence slots of kSyncSlots publication counters
  // then kSyncSlots verdict counters; the outputs; the bounds of its waits
  uint64_t* sync;
  void* out;
  float* lse;
  int64_t short_ticks, long_ticks;  // 10 ns ticks (s_memrealtime)
  int64_t lsb, lst, lsbr, rsb, rst;
  int32_t S, Q, H, rows, NB, DC, DR, spl, tps, max_blocks, num_blocks, lcap, causal;
  int32_t nrt;        // workgroups per split: row groups or branch groups (1 or 2)
  int32_t wait_polls;  // bound of the LDS waits
  int32_t concat;
  float score_scale;  // scale * log2(e): scores kept in base-2 units
  float out_rescale;
};

struct CombineParams {
  const float* part_o;
  const float* part_lse;
  const int32_t* seq_lens;
  void* out;
  float* lse;
  int32_t S, Q, H, rows, NB, DC, spl, tps, lcap, concat;
  float out_rescale;
};

__device__ __forceinline__ int seq_len_of(const int32_t* seq_lens, int s, int lcap) {
  int L = seq_lens[s];
  return L < 0 ? 0 : (L > lcap ? lcap : L);
}

__device__ __forceinline__ int clamp_block(int b, int num_blocks) {
  return (b < 0 || b >= num_blocks) ? 0 : b;
}

__device__ __forceinline__ float wave_max_halves(float x) {
  // max over lanes l and l^32 (the two k-groups of a 32x32 MFMA column)
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float wave_sum_halves(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Workgroup barrier that orders LDS only: it does not wait for this wave's
// outstanding global loads (a plain __syncthreads() would, which would stall
// the software pipeline on its prefetches).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// ---------------------------------------------------------------------------
// LDS helpers of the bf16 split kernel
// ---------------------------------------------------------------------------
// LDS transpose read (gfx950 ds_read_b64_tr_b16): within each 16-lane group,
// lane j supplies the address of 4 bf16 at row j/4, column 4*(j%4) of a 4x16
// block; lane i receives column i, rows 0..3 of that block.
__device__ __forceinline__ i16x4 lds_read_tr(const unsigned char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) i16x4*)(const_cast<unsigned char*>(p)));
}

// Staged rows are padded so that every LDS address is a per-lane base plus a
// compile-time offset: latent rows get 2 spare 16-byte chunks, RoPE rows 1
// (stage_lpitch, stage_rpitch). With 64 four-byte banks a 16-byte row read
// serves 16 lanes per pass, and at these pitches 16 consecutive rows meet
// each bank twice (a two-way conflict; the transpose reads likewise). An
// unpadded layout with chunk swizzles free of conflicts (the prefill
// kernel's) measured no faster here: the loader waves set the pace.

// ---------------------------------------------------------------------------
// bf16 split kernel: loader and compute waves
// ---------------------------------------------------------------------------
// A wave that issues loads while its CU's memory pipeline is full stalls in
// issue, and a wave that waits for its own loads idles: both cost a wave that
// also computes. Here the roles are split. Of the eight waves of a workgroup
// (two per SIMD), the four loader waves stream every 32-token sub-tile of the
// split into a ring of LDS slots, keeping PL sub-tiles each in flight in
// registers; the four compute waves (one per SIMD) take ready slots and never
// touch global memory in their loop. Loader l loads part l of every sub-tile
// (every fourth of its 16-byte-per-lane load instructions, all branches and
// the shared RoPE key once), so the RoPE key is read once per token.
//
// A workgroup holds NBW branches (branch group grp: branches NBW*grp ...)
// and RT 32-row tiles of query rows (the 512-wide latent: row group grp); a
// slot holds the NBW latents and the RoPE key of one sub-tile, so every
// cache byte of the split is read once per workgroup. Latents wider than 128
// are split into WD slices of 128 columns, one compute wave each: a wave
// scores its slice (and its share of the RoPE key), the WD partial scores
// meet through LDS, and each wave accumulates P . C over its own columns.
//
// Slot hand-off uses two cumulative LDS counters per slot: ready (loader parts
// written, 4 per use) and consumed (compute waves done, NCW = NBW * RT * WD
// per use). A loader refills slot j % NSLOT for sub-tile j only when the
// previous occupant was consumed NCW times; a compute wave reads it once it
// is ready 4 times. Every wait is a bounded spin (it ends even if the protocol were
// broken, leaving wrong results rather than a hung GPU).
//
// Compute wave c takes slice c % WD of the (branch, row tile) pair
// (c / WD) % NP (branch pair % NBW, row tile pair / NBW) and sub-tiles
// j = c / NCW + WT*i (WT = 4 / NCW); per sub-tile it runs S^T = C . Q^T
// (MFMA, A = slot rows, B = query rows in registers), the online softmax,
// and O^T += C^T . P^T (A = transpose reads of the slot). With WT > 1 the
// token streams of a triple merge (m, l, O) at the end without a workgroup
// barrier: every stream but the one holding the split's last sub-tile leaves
// its state as a record in a dedicated LDS area, counts it on an LDS counter
// and exits; that last stream waits for them and merges the records with its
// own registers in a fixed stream order (so the partial does not depend on
// which stream finished first) and writes it.
// A wait that gives up (after `polls` polls, by default a few million: far
// longer than any wait here) marks the wave's `expired`; the wave reports it
// once, when it leaves the kernel, as MLRA_DEVSTATUS_WAIT_EXPIRED in the
// workspace status word, so a broken hand-off is reported, not silent.
// (An atomic after every wait measured 0.7 us slower at B=16, T=8192.)
__device__ __forceinline__ void set_status(unsigned* status, unsigned bit) {
  if ((threadIdx.x & 63) == 0)
    __hip_atomic_fetch_or(status, bit, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void lds_wait_geq(const int* flag, int target, int polls, bool& expired) {
  int it = 0;
  for (; it < polls; ++it) {
    if (__hip_atomic_load(flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) >= target) break;
    __builtin_amdgcn_s_sleep(1);
  }
  if (it == polls) expired |= __hip_atomic_load(flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) < target;
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}
__device__ __forceinline__ void report_expired(unsigned* status, bool expired) {
  if (expired) set_status(status, MLRA_DEVSTATUS_WAIT_EXPIRED);
}
__device__ __forceinline__ void lds_signal(int* flag) {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  if ((threadIdx.x & 63) == 0)
    __hip_atomic_fetch_add(flag, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

// ---------------------------------------------------------------------------
// In-kernel merge of a sequence's splits
// ---------------------------------------------------------------------------
// When the whole call runs as one round of workgroups (one per CU) and every
// sequence's workgroups are dealt to one XCD (workgroup ids congruent modulo
// kXcdSlots), the workgroups of a sequence merge their own partial results
// instead of a second kernel doing it. The XCD's L2 is shared by its CUs, so
// a partial or counter stored with ordinary stores is visible to the
// sequence's other workgroups once the stores are acknowledged; reads that
// must not hit this CU's L1 use the sc1 (agent-scope) bit.
//
// Every workgroup of sequence s owns a publication counter and a verdict
// counter in the workspace header (slot rr: its index within the sequence).
// All counters of a sequence advance in lock step, by one per call: a
// workgroup reads its own counter N at the start, and after its partial is
// stored publishes N+1 in its slot and in every slot no workgroup of this
// call owns (so a later call with more workgroups finds them level). Values
// carry the XCD id; a workgroup waits until every slot shows N+1 and all
// XCD ids equal its own, then merges its share (chunk rr) of the sequence's
// outputs. It writes its verdict: merging, gave up waiting, or found
// another XCD. A workgroup that gives up after a short bound leaves its
// chunk to the sequence's last workgroup (rr = per - 1), which is dealt to
// its XCD after all others of the sequence, so it only waits for workgroups
// that already run; it waits with a long bound, reads every verdict and
// merges the chunks given up. Chunks that cannot be merged (workgroups on
// different XCDs, or a long wait expired) are written as NaN and flagged in
// the status word. A counter never goes back, so stale values never look
// fresh; a header that was not zeroed leaves the slots uneven, which shows
// as NaN and a flag rather than as wrong numbers.
__device__ __forceinline__ uint64_t sync_load(const uint64_t* a) {
  return __hip_atomic_load(a, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Counters are published with plain stores: they stay in the XCD's L2,
// where the sequence's other workgroups (same XCD) poll them with sc1 loads.
// A workgroup on another XCD would not see them (its wait expires) or, if an
// eviction wrote one back, would see a foreign XCD id: never stale data.
__device__ __forceinline__ void sync_store(uint64_t* a, uint64_t v) {
  *reinterpret_cast<volatile uint64_t*>(a) = v;
}
// A publication slot holds (count << 8) | XCD id: the workgroup's count.
__device__ __forceinline__ uint64_t own_count(const uint64_t* sync, int s, int rr) {
  return sync_load(sync + (size_t)s * (kSyncSlotBytes / 8) + rr) >> 8;
}
// XCC (XCD) id of the executing CU: hardware register 20 (HW_REG_XCC_ID), bits [3:0].
__device__ __forceinline__ unsigned xcc_id() { return __builtin_amdgcn_s_getreg(6164) & 15u; }

__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, 0x7fffffff, 0x00020000);
}

__device__ __forceinline__ void store_bf16x4(__bf16* d, f32x4 v) {
  typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
  *reinterpret_cast<bf16x4*>(d) = bf16x4{(__bf16)v[0], (__bf16)v[1], (__bf16)v[2], (__bf16)v[3]};
}

// Merge the splits of sequence s for output items [i0, i1) (an item is four
// columns of one row: of the branch sum, or of one branch with CONCAT),
// thread tid of nthr; nan_fill writes NaN instead. Splits are merged in
// order with a running log-sum-exp, 16 splits' loads in flight at a time.
// The partials are read with plain loads: this CU has not touched those
// lines in this kernel (its L1 holds no stale copy), so they come from the
// XCD's L2, where their writers' acknowledged stores are.
__device__ void merge_items(const SplitParams& p, int s, int nsplit, int i0, int i1, int tid,
                            int nthr, bool nan_fill) {
  const int C4 = p.DC >> 2;
  const int64_t seq_rows = (int64_t)p.spl * p.NB * p.rows;  // partial rows of one sequence
  const __amdgpu_buffer_rsrc_t ro = buffer_rsrc(p.part_o + (int64_t)s * seq_rows * p.DC);
  const __amdgpu_buffer_rsrc_t rl = buffer_rsrc(p.part_lse + (int64_t)s * seq_rows);
  __bf16* const out = static_cast<__bf16*>(p.out);
  for (int it = i0 + tid; it < i1; it += nthr) {
    const int c4 = it % C4, rb = it / C4;
    const int row = p.concat ? rb / p.NB : rb;
    const int b0 = p.concat ? rb % p.NB : 0, b1 = p.concat ? b0 + 1 : p.NB;
    const int64_t orow = (int64_t)s * p.rows + row;
    f32x4 tot = {0.f, 0.f, 0.f, 0.f};
    for (int b = b0; b < b1; ++b) {
      float m = -INFINITY, den = 0.f;
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      for (int k0 = 0; k0 < nsplit && !nan_fill; k0 += 16) {
        float l[16];
        f32x4 v[16];
#pragma unroll
        for (int u = 0; u < 16; ++u) {
          const int pr = (min(k0 + u, nsplit - 1) * p.NB + b) * p.rows + row;
          l[u] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rl, pr * 4, 0, 0));
          v[u] = __builtin_bit_cast(
              f32x4, __builtin_amdgcn_raw_buffer_load_b128(ro, (pr * p.DC + 4 * c4) * 4, 0, 0));
        }
        // all 32 loads leave before the first wait (one round trip, not two)
        __builtin_amdgcn_sched_barrier(0);
        float mb = m;
#pragma unroll
        for (int u = 0; u < 16; ++u)
          if (k0 + u < nsplit) mb = fmaxf(mb, l[u]);
        if (mb == -INFINITY) continue;  // no visible token so far
        const float sc = expf(m - mb);
        den *= sc;
        acc *= sc;
#pragma unroll
        for (int u = 0; u < 16; ++u)
          if (k0 + u < nsplit) {
            const float w = expf(l[u] - mb);
            den += w;
            acc += v[u] * w;
          }
        m = mb;
      }
      const f32x4 o = acc * (den > 0.f ? 1.f / den : 0.f);
      const float lse_b = nan_fill ? NAN : (den > 0.f ? m + logf(den) : -INFINITY);
      if (c4 == 0) p.lse[orow * p.NB + b] = lse_b;
      if (p.concat)
        store_bf16x4(out + (orow * p.NB + b) * p.DC + 4 * c4,
                     nan_fill ? f32x4{NAN, NAN, NAN, NAN} : o * p.out_rescale);
      else
        tot += o;
    }
    if (!p.concat)
      store_bf16x4(out + orow * p.DC + 4 * c4,
                   nan_fill ? f32x4{NAN, NAN, NAN, NAN} : tot * p.out_rescale);
  }
}

// The merge protocol (above) for workgroup rr of per of sequence s. Called by
// the compute waves (cw 0-3) once their partial is stored; cw 0 drives. With
// solo, only cw 0 runs (a workgroup with no tokens of its own) and merges
// with its 64 lanes. N is the workgroup's own counter, read at its start.
template <int NCW>
__device__ void fused_merge(const SplitParams& p, int s, int rr, int per, int nsplit, uint64_t N,
                            int cw, int lane, bool solo, int* stored, int* go, int* godec,
                            bool& expired) {
  const uint64_t next = N + 1;
  uint64_t* const flags = p.sync + (size_t)s * (kSyncSlotBytes / 8);
  uint64_t* const verd = flags + kSyncSlots;
  const unsigned xcc = xcc_id();
  const bool designated = rr == per - 1;
  const int items = p.rows * (p.concat ? p.NB : 1) * (p.DC >> 2);
  const int csz = (items + per - 1) / per;
  auto lo = [&](int c) { return min(c * csz, items); };
  auto hi = [&](int c) { return min((c + 1) * csz, items); };
  int dec = 0;  // 1: merge own chunk; 2: gave up waiting; 3: another XCD found
  if (cw == 0) {
    if (!solo) lds_wait_geq(stored, NCW, p.wait_polls, expired);  // every partial writer's stores acknowledged
    if (lane == 0)
      for (int q = rr; q < kSyncSlots; q += per) sync_store(flags + q, (next << 8) | xcc);
    const uint64_t bound = designated ? p.long_ticks : p.short_ticks;
    const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
    bool all = false, same = false;
    for (;;) {
      const uint64_t f = lane < per ? sync_load(flags + lane) : ((next << 8) | xcc);
      if (__builtin_amdgcn_ballot_w64((f >> 8) != next) == 0) {
        all = true;
        same = __builtin_amdgcn_ballot_w64((f & 0xff) != xcc) == 0;
        break;
      }
      if (__builtin_amdgcn_s_memrealtime() - t0 > bound) break;
      __builtin_amdgcn_s_sleep(2);
    }
    dec = !all ? 2 : (same ? 1 : 3);
    if (lane == 0)
      for (int q = rr; q < kSyncSlots; q += per)
        sync_store(verd + q, (next << 2) | (uint64_t)(q == rr ? dec : 1));
    if (!solo) {
      if (lane == 0) *godec = dec;
      lds_signal(go);
    }
  } else {
    lds_wait_geq(go, 1, p.wait_polls, expired);
    dec = *godec;
  }
  // The sequence's last workgroup reads the others' verdicts; its first read
  // is issued before its own chunk, so the two overlap.
  uint64_t v = (next << 2) | 1;
  if (cw == 0 && designated && lane < per && lane != rr) v = sync_load(verd + lane);
  if (dec == 1) merge_items(p, s, nsplit, lo(rr), hi(rr), solo ? lane : cw * 64 + lane, solo ? 64 : 256, false);
  if (cw != 0 || !designated) return;
  // Chunks the others gave up.
  if (dec != 1) {
    merge_items(p, s, nsplit, lo(rr), hi(rr), lane, 64, true);
    set_status(p.status, MLRA_DEVSTATUS_MERGE_FAILED);
  }
  const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
  while (__builtin_amdgcn_ballot_w64((v >> 2) != next) != 0) {
    if (__builtin_amdgcn_s_memrealtime() - t0 > (uint64_t)p.long_ticks) break;
    __builtin_amdgcn_s_sleep(2);
    if (lane < per && lane != rr) v = sync_load(verd + lane);
  }
  const int state = (v >> 2) == next ? (int)(v & 3) : 0;  // 0: no verdict in time
  for (int q = 0; q < per; ++q) {
    if (q == rr) continue;
    const int sq = __builtin_amdgcn_readlane(state, q);
    if (sq == 1) continue;  // merged by its own workgroup
    const bool can = dec == 1 && sq == 2;
    merge_items(p, s, nsplit, lo(q), hi(q), lane, 64, !can);
    if (!can) set_status(p.status, MLRA_DEVSTATUS_MERGE_FAILED);
  }
}

template <int NBW, int RT, int WD, int DC, int DR, int NSLOT, int PL, bool FUSED>
__global__ void __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
mlra_split_pc(SplitParams p) {
  constexpr int NP = NBW * RT;   // (branch, row tile) pairs
  constexpr int NCW = NP * WD;   // compute waves per token stream
  constexpr int WT = 4 / NCW;    // token streams
  constexpr int DCW = DC / WD, DRW = DR / WD;  // a compute wave's slice of the dims
  constexpr int NL = DCW / 16, NR = DRW / 16, NDT = DCW / 32;
  constexpr int LCHW = DCW / 8, RCHW = DRW / 8;
  constexpr int LCH = DC / 8, RCH = DR / 8;
  constexpr int LQ = kSub * LCH / 64, RQ = kSub * RCH / 64;  // load instructions per sub-tile part
  constexpr int NLOAD = NBW * LQ + RQ;                       // per sub-tile
  constexpr int P = (NLOAD + 3) / 4;                         // per loader per sub-tile
  constexpr int LP = stage_lpitch(DC), RP = stage_rpitch(DR);
  constexpr PcLds lay = pc_lds(NBW, RT, WD, DC, DR);
  static_assert(NCW == 1 || NCW == 2 || NCW == 4, "compute waves");
  static_assert(NR >= 1 && RCHW >= 2, "RoPE slice of at least one k-step");
  static_assert(lay.nslot == NSLOT && NSLOT >= 2, "slot count");
  static_assert(lay.total <= 160 * 1024, "LDS");
  static_assert((PL - 1) * P <= 63, "outstanding loads fit the counter");
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  int* const ready = reinterpret_cast<int*>(smem + lay.flags);
  int* const consumed = ready + NSLOT;
  int* const qdone = consumed + NSLOT;
  int* const recorded = qdone + 1;    // [4] merge records written, per compute wave of a stream
  int* const exchanged = recorded + 4;  // [4] partial scores written, per compute wave
  int* const stored = exchanged + 4;    // in-kernel merge: partial writers done
  int* const go = stored + 1;           // in-kernel merge: the driving wave's decision made
  int* const godec = go + 1;            // ... and what it is
  int* const tabl = reinterpret_cast<int*>(smem + lay.table);

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 31, g = lane >> 5;
  bool expired = false;       // a wait of this wave gave up (reported when it leaves)
  int k, s, bo = 0, rb0 = 0;  // bo, rb0: first branch and first query row of this workgroup
  int rr = 0;                 // in-kernel merge: index of this workgroup within its sequence
  const int per = p.spl * p.nrt;
  if constexpr (FUSED) {
    // Sequence s's workgroups are the ids congruent to s mod kXcdSlots (one
    // XCD), split-major within the sequence.
    const int id = blockIdx.x, jx = id / kXcdSlots;
    s = id % kXcdSlots + kXcdSlots * (jx / per);
    rr = jx % per;
    k = rr / p.nrt;
    const int grp = rr % p.nrt;
    const int nbg = p.NB / NBW;
    bo = (grp % nbg) * NBW;
    rb0 = (grp / nbg) * RT * kSub;
  } else if (p.nrt == 1) {
    k = blockIdx.x;
    s = blockIdx.y;
  } else {
    // G groups per split: ids 8G*c + 8g + i (g < G) are dealt to one XCD
    // together. Group g = row group * (NB / NBW) + branch group.
    const int G = p.nrt;
    const int id = blockIdx.x;
    const int pr = (id / (8 * G)) * 8 + (id & 7);
    if (pr >= p.S * p.spl) return;
    const int grp = (id >> 3) % G;
    const int nbg = p.NB / NBW;
    bo = (grp % nbg) * NBW;
    rb0 = (grp / nbg) * RT * kSub;
    s = pr / p.spl;
    k = pr % p.spl;
  }
  const int NBT = RT == 1 ? NBW : p.NB;  // branches of the call (one group with one row tile)
  const int t0 = k * p.tps;
  // query and cache bases moved to the workgroup's first branch
  const __bf16* __restrict__ qlat = static_cast<const __bf16*>(p.q_lat) + bo * DC;
  const __bf16* __restrict__ qrop = static_cast<const __bf16*>(p.q_rope);
  const __bf16* __restrict__ lat = static_cast<const __bf16*>(p.lat) + bo * p.lsbr;
  const __bf16* __restrict__ rope = static_cast<const __bf16*>(p.rope);

  // Prologue. Loader waves read the split's first 64 block ids into a
  // register and issue their first PL sub-tiles at once; compute waves stage
  // the split's block ids and the query rows (coalesced) in LDS, over the
  // ring's last slots, and clear the counters. The first cache loads thus
  // leave as soon as the block table arrives, not after the queries, and the
  // first slots are filled without waiting for the queries to be read.
  const int L_raw = p.seq_lens[s];
  const int64_t tab_base = (int64_t)s * p.max_blocks;
  const bool is_loader = wave >= 4;
  const int ld = wave & 3;
  constexpr int LAT_B = kSub * LP * 16;  // one branch's latent rows in a slot
  u32x4 buf[PL][P];
  // Load instruction x of a sub-tile (x = q*4 + ld, wrapping: loaders with
  // fewer real loads repeat one, writing the same bytes twice): branch
  // latent x / LQ instruction x % LQ, or RoPE instruction x - NBW*LQ.
  auto issue = [&](int j, int phys, u32x4 (&d)[P]) {
    const int sub = (j & 1) * kSub;
    const char* lb = reinterpret_cast<const char*>(lat) + ((int64_t)phys * p.lsb + (int64_t)sub * p.lst) * 2;
    const char* rb = reinterpret_cast<const char*>(rope) + ((int64_t)phys * p.rsb + (int64_t)sub * p.rst) * 2;
#pragma unroll
    for (int q = 0; q < P; ++q) {
      const int x = (q * 4 + ld) % NLOAD;
      const bool isl = x < NBW * LQ;
      const int bb = isl ? x / LQ : 0, ql = isl ? x % LQ : x - NBW * LQ;
      const uint32_t off = isl ? (uint32_t)(bb * p.lsbr * 2 + (ql * (64 / LCH) + lane / LCH) * p.lst * 2 + (lane % LCH) * 16)
                               : (uint32_t)((ql * (64 / RCH) + lane / RCH) * p.rst * 2 + (lane % RCH) * 16);
      d[q] = ld16((isl ? lb : rb) + off);
    }
  };
  int L, nsub;
  auto sizes = [&]() {
    L = L_raw < 0 ? 0 : (L_raw > p.lcap ? p.lcap : L_raw);
    const int ntiles = (L + kBlock - 1) / kBlock;
    nsub = t0 >= ntiles ? 0 : 2 * (min(t0 + p.tps, ntiles) - t0);  // sub-tiles of this split
  };
  f32x16 acc[NDT];
  float m_run = -INFINITY, l_run = 0.f;
  uint64_t n_own = 0;  // in-kernel merge: this workgroup's counter at its start
  const int cw = wave & 3;                // compute waves: index
  const int wd = cw % WD;                 // latent slice
  const int pi = (cw / WD) % NP;          // (branch, row tile) pair
  const int b = pi % NBW;                 // its branch within the group
  const int row0 = (pi / NBW) * kSub;     // its first query row in the workgroup
  const int strm = cw / NCW;              // token stream
  // Each role synchronises once with the other (s_barrier counts waves)
  // inside its own branch, so no register of one role is live in the other.
  if (is_loader) {
    const int tab0 = p.table[tab_base + min(t0 + lane, p.max_blocks - 1)];
    sizes();
    if (nsub == 0) return;  // uniform over the workgroup
#pragma unroll
    for (int i = 0; i < PL; ++i) {
      const int phys = i < nsub ? clamp_block(__builtin_amdgcn_readlane(tab0, (i >> 1) & 63), p.num_blocks) : 0;
      issue(i, phys, buf[i]);
    }
    lds_barrier();
    // ---------------- loader ----------------
    auto write = [&](int j, u32x4 (&d)[P]) {
      const int slot = j % NSLOT;
      // first pass: slots from qslot on hold the staged query rows until
      // every compute wave has read its own into registers
      if (j >= lay.qslot && j < NSLOT) lds_wait_geq(qdone, 4, p.wait_polls, expired);
      lds_wait_geq(consumed + slot, (j / NSLOT) * NCW, p.wait_polls, expired);  // previous occupant done
      unsigned char* sb = smem + slot * lay.slot_bytes;
      const int tok0 = (t0 + (j >> 1)) * kBlock + (j & 1) * kSub;
#pragma unroll
      for (int q = 0; q < P; ++q) {
        const int x = (q * 4 + ld) % NLOAD;
        const bool isl = x < NBW * LQ;
        const int bb = isl ? x / LQ : 0, ql = isl ? x % LQ : x - NBW * LQ;
        const int row = isl ? ql * (64 / LCH) + lane / LCH : ql * (64 / RCH) + lane / RCH;
        const int dst = isl ? bb * LAT_B + (row * LP + lane % LCH) * 16
                            : NBW * LAT_B + (row * RP + lane % RCH) * 16;
        *reinterpret_cast<u32x4*>(sb + dst) = tok0 + row < L ? d[q] : u32x4{};
      }
      lds_signal(ready + slot);
    };
    auto phys_of = [&](int j) { return j < nsub ? tabl[min(j >> 1, kPcMaxTiles - 1)] : 0; };
    // Steady state: write j, issue j + PL into the same registers (every
    // written sub-tile here is < nsub); then the last PL without new loads.
    // (Issuing fewer sub-tiles first and ramping up to PL was measured
    // slower: the memory system is best fed from the start.)
    int j0 = 0;
    for (; j0 + PL < nsub; j0 += PL) {
#pragma unroll
      for (int i = 0; i < PL; ++i) {
        const int j = j0 + i;
        write(j, buf[i]);
        issue(j + PL, phys_of(j + PL), buf[i]);
      }
    }
#pragma unroll
    for (int i = 0; i < PL; ++i)
      if (j0 + i < nsub) write(j0 + i, buf[i]);
  } else {
    constexpr int TK = (kPcMaxTiles + 255) / 256;
    int tv[TK];
#pragma unroll
    for (int kt = 0; kt < TK; ++kt)
      tv[kt] = p.table[tab_base + min(t0 + kt * 256 + (int)threadIdx.x, p.max_blocks - 1)];
    // in-kernel merge: the driving wave reads its own counter now, so the
    // load is long done when the merge starts
    if constexpr (FUSED)
      if (wave == 0) n_own = own_count(p.sync, s, rr);
    // query rows of the workgroup: latent [NBW][RT*32 rows][LP chunks], then
    // RoPE [RT*32][RP]
    constexpr int QR = RT * kSub;
    constexpr int QL_CH = NBW * QR * LCH;
    constexpr int Q_CH = QL_CH + QR * RCH;
    constexpr int QK = (Q_CH + 255) / 256;
    u32x4 qv[QK];
    int qdst[QK];
#pragma unroll
    for (int kq = 0; kq < QK; ++kq) {
      const int x = kq * 256 + threadIdx.x;
      const bool is_lat = x < QL_CH;
      const bool is_rope = !is_lat && x < Q_CH;
      const int bb = x / (QR * LCH), rem = x % (QR * LCH);
      const int rl = rem / LCH, cl = rem % LCH;
      const int xr = is_rope ? x - QL_CH : 0;
      const int rr = xr / RCH, cr = xr % RCH;
      const int r = rb0 + (is_lat ? rl : rr);
      const bool live = (is_lat || is_rope) && r < p.rows;
      const int rs = live ? r : 0;
      const int64_t head = ((int64_t)s * p.Q + rs / p.H) * p.H + rs % p.H;
      const __bf16* src = is_lat ? qlat + (head * NBT + (is_lat ? bb : 0)) * DC + cl * 8
                                 : qrop + head * DR + cr * 8;
      const u32x4 v = ld16(src);
      qv[kq] = live ? v : u32x4{};
      qdst[kq] = is_lat ? lay.qoff + ((bb * QR + rl) * LP + cl) * 16
                        : (is_rope ? lay.qoff + NBW * QR * LP * 16 + (rr * RP + cr) * 16 : -1);
    }
    sizes();
    if (nsub == 0) {  // uniform over the workgroup
      if constexpr (FUSED) {
        if (wave == 0) {
          const int nsplit = min((L + kBlock * p.tps - 1) / (kBlock * p.tps), p.spl);
          fused_merge<NCW>(p, s, rr, per, nsplit, own_count(p.sync, s, rr), 0, lane, true, nullptr,
                           nullptr, nullptr, expired);
          report_expired(p.status, expired);
        }
      }
      return;
    }
#pragma unroll
    for (int kt = 0; kt < TK; ++kt) tabl[kt * 256 + threadIdx.x] = clamp_block(tv[kt], p.num_blocks);
#pragma unroll
    for (int kq = 0; kq < QK; ++kq)
      if (qdst[kq] >= 0) *reinterpret_cast<u32x4*>(smem + qdst[kq]) = qv[kq];
    if (threadIdx.x < 2 * NSLOT + 12) ready[threadIdx.x] = 0;  // every counter
    lds_barrier();
    // ---------------- compute ----------------
    // this wave's slice of the query row (the k order of the score MFMAs:
    // lane half g takes chunks g*LCHW/2 + st of the slice)
    const unsigned char* const qb =
        smem + lay.qoff + ((b * QR + row0 + n) * LP + wd * LCHW + g * (LCHW / 2)) * 16;
    const unsigned char* const qrb =
        smem + lay.qoff + NBW * QR * LP * 16 + ((row0 + n) * RP + wd * RCHW + g * (RCHW / 2)) * 16;
    auto rd16 = [](const unsigned char* a) {
      return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(a));
    };
    bf16x8 qL[NL], qR[NR];
#pragma unroll
    for (int st = 0; st < NL; ++st) qL[st] = rd16(qb + st * 16);
#pragma unroll
    for (int st = 0; st < NR; ++st) qR[st] = rd16(qrb + st * 16);
    lds_signal(qdone);
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) acc[dt] = f32x16{};
    const int row = rb0 + row0 + n;
    const int jr = row < p.rows ? row / p.H : 0;
    const int vis = p.causal ? L - (p.Q - 1 - jr) : L;
    const int min_vis = p.causal ? L - (p.Q - 1) : L;
    const int a_l = (n * LP + wd * LCHW + g * (LCHW / 2)) * 16 + b * LAT_B;  // S^T A operand, row n
    const int a_r = (n * RP + wd * RCHW + g * (RCHW / 2)) * 16 + NBW * LAT_B;
    const int a_t = b * LAT_B + (4 * (lane >> 5) + ((lane & 15) >> 2)) * LP * 16 +
                    (wd * DCW + 16 * ((lane >> 4) & 1) + 4 * (lane & 3)) * 2;
    // Pieces of a sub-tile's work, shared by both loop forms below.
    bf16x8 aR[NR], aL[NL], aT[2][NDT];
    auto slot_at = [&](int j) { return smem + (j % NSLOT) * lay.slot_bytes; };
    auto wait_ready = [&](int j) {
      lds_wait_geq(ready + j % NSLOT, (j / NSLOT + 1) * 4, p.wait_polls, expired);
    };
    auto read_a = [&](const unsigned char* sb) {  // score operands (A = slot rows)
#pragma unroll
      for (int st = 0; st < NR; ++st) aR[st] = rd16(sb + a_r + st * 16);
#pragma unroll
      for (int st = 0; st < NL; ++st) aL[st] = rd16(sb + a_l + st * 16);
    };
    auto read_t = [&](const unsigned char* sb, int h2) {  // C^T operands of P . C
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        const i16x4 lo = lds_read_tr(sb + a_t + (16 * h2) * LP * 16 + dt * 64);
        const i16x4 hi = lds_read_tr(sb + a_t + (16 * h2 + 8) * LP * 16 + dt * 64);
        aT[h2][dt] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      }
    };
    // The WD waves of a (branch, row tile) pair hold partial scores over
    // their slices: each leaves its part in the exchange area (double
    // buffered by the stream's sub-tile parity), and all of them add the WD
    // parts in slice order, so they hold bit-identical scores and take the
    // same softmax decisions. A part is overwritten two sub-tiles later,
    // after its readers have signalled the sub-tile in between.
    auto exchange = [&](int u, f32x16 sc) {
      f32x4* const X = reinterpret_cast<f32x4*>(smem + lay.xchg) + (u & 1) * 4 * 4 * 64;
#pragma unroll
      for (int q = 0; q < 4; ++q)
        X[(cw * 4 + q) * 64 + lane] = f32x4{sc[4 * q], sc[4 * q + 1], sc[4 * q + 2], sc[4 * q + 3]};
      lds_signal(exchanged + cw);
#pragma unroll
      for (int w = 0; w < WD; ++w)
        if (w != wd) lds_wait_geq(exchanged + cw - wd + w, u + 1, p.wait_polls, expired);
      f32x16 tot = f32x16{};
#pragma unroll
      for (int w = 0; w < WD; ++w) {
        f32x16 part = sc;
        if (w != wd) {
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const f32x4 v = X[((cw - wd + w) * 4 + q) * 64 + lane];
            part[4 * q] = v[0];
            part[4 * q + 1] = v[1];
            part[4 * q + 2] = v[2];
            part[4 * q + 3] = v[3];
          }
        }
        tot = w == 0 ? part : tot + part;
      }
      return tot;
    };
    auto mask = [&](f32x16& sc, int tb) {
      if (tb + kSub > min_vis) {  // uniform
        // element r holds token tb + 4g + 8(r/4) + r%4: compare the constant
        // part against a per-lane limit
        const int lim = vis - tb - 4 * g;
#pragma unroll
        for (int r = 0; r < 16; ++r) sc[r] = 8 * (r >> 2) + (r & 3) < lim ? sc[r] : -INFINITY;
      }
    };
    // Online softmax against a lazily moved reference maximum: the reference
    // moves only when a row maximum exceeds it by more than kLazyLog2 (log2
    // units). Returns whether any lane moved it with a running sum behind it
    // (then O must be scaled by alpha before this sub-tile's P . C).
    auto softmax = [&](const f32x16& sc, bf16x8 (&pB)[2], float& alpha) {
      float mx = -INFINITY;
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sc[r]);
      mx = wave_max_halves(mx) * p.score_scale;
      const bool first = m_run == -INFINITY;
      const bool grow = first ? mx > -INFINITY : mx > m_run + kLazyLog2;
      alpha = grow ? __builtin_amdgcn_exp2f(m_run - mx) : 1.f;
      m_run = grow ? mx : m_run;
      l_run *= alpha;
      const float m_use = m_run == -INFINITY ? 0.f : m_run;
      float ps[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float pe = __builtin_amdgcn_exp2f(fmaf(sc[8 * h2 + e], p.score_scale, -m_use));
          ps[e & 3] += pe;
          pB[h2][e] = (__bf16)pe;
        }
      l_run += (ps[0] + ps[1]) + (ps[2] + ps[3]);
      return grow && !first;
    };
    auto rescale = [&](bool moved, float alpha) {
      if (__builtin_amdgcn_ballot_w64(moved)) {
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) acc[dt] *= alpha;
      }
    };
    auto pv = [&](const bf16x8 (&pB)[2]) {
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
          acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aT[h2][dt], pB[h2], acc[dt], 0, 0, 0);
    };
    if constexpr (WT == 1) {
      // One token stream per wave: a software pipeline across sub-tiles.
      // Iteration j holds the scores of sub-tile j (from the previous
      // iteration) and keeps slot j until its C^T reads are done; it issues
      // the score MFMAs of sub-tile j + 1 first and runs the softmax of
      // sub-tile j on the vector ALU while they execute, then P . C of
      // sub-tile j. A wave thus holds two slots at a time.
      auto score1 = [&]() {  // S^T = C . Q^T, one accumulator chain
        f32x16 sc = f32x16{};
#pragma unroll
        for (int st = 0; st < NR; ++st) sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aR[st], qR[st], sc, 0, 0, 0);
#pragma unroll
        for (int st = 0; st < NL; ++st) sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aL[st], qL[st], sc, 0, 0, 0);
        return sc;
      };
      wait_ready(0);
      read_a(slot_at(0));
      f32x16 S = score1();
      for (int j = 0; j < nsub; ++j) {
        const unsigned char* sb = slot_at(j);
        const bool more = j + 1 < nsub;  // uniform
        if constexpr (WD > 1) S = exchange(j, S);
        mask(S, (t0 + (j >> 1)) * kBlock + (j & 1) * kSub);
        read_t(sb, 0);
        read_t(sb, 1);
        if (more) wait_ready(j + 1);
        // past the last sub-tile the next scores are computed from this
        // (still held) slot and dropped
        read_a(more ? slot_at(j + 1) : sb);
        __builtin_amdgcn_sched_barrier(0);
        const f32x16 Sn = score1();
        bf16x8 pB[2];
        float alpha;
        const bool moved = softmax(S, pB, alpha);
        // interleave: each score MFMA followed by a share of the softmax
#pragma unroll
        for (int i = 0; i < NR + NL; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
          __builtin_amdgcn_sched_group_barrier(0x002, 8, 0);  // VALU
        }
        __builtin_amdgcn_sched_barrier(0);
        rescale(moved, alpha);
        pv(pB);
        lds_signal(consumed + j % NSLOT);  // its C^T reads are done (P . C used them)
        S = Sn;
      }
    } else {
      for (int j = strm; j < nsub; j += WT) {
        const unsigned char* sb = slot_at(j);
        wait_ready(j);
        // LDS reads are batched ahead of the MFMAs that use them: the score
        // operands (A = slot rows) first, then the C^T operands of P.C
        // (transpose reads) in two halves slotted between the score MFMAs.
        // LDS returns in order, so each MFMA waits only for its own operand,
        // and at most 15 reads are outstanding past any wait (the counter's
        // limit; beyond it the wait would be for every read).
        read_a(sb);
        __builtin_amdgcn_sched_barrier(0);
        f32x16 sc = f32x16{}, sd = f32x16{};
#pragma unroll
        for (int st = 0; st < NR; ++st) sd = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aR[st], qR[st], sd, 0, 0, 0);
        read_t(sb, 0);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int st = 0; st < NL; ++st) {
          if (st % 2 == 0)
            sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aL[st], qL[st], sc, 0, 0, 0);
          else
            sd = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aL[st], qL[st], sd, 0, 0, 0);
        }
        read_t(sb, 1);
        __builtin_amdgcn_sched_barrier(0);
        // every read of the slot is issued: hand it back once they complete
        __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
        lds_signal(consumed + j % NSLOT);
        sc += sd;
        if constexpr (WD > 1) sc = exchange(j / WT, sc);
        mask(sc, (t0 + (j >> 1)) * kBlock + (j & 1) * kSub);
        bf16x8 pB[2];
        float alpha;
        const bool moved = softmax(sc, pB, alpha);
        rescale(moved, alpha);
        pv(pB);
      }
    }
    l_run = wave_sum_halves(l_run);
  }

  const int64_t slotp = (int64_t)s * p.spl + k;
  if (wave >= 4) {  // loaders
    report_expired(p.status, expired);
    return;
  }
  if constexpr (WT == 1) {
    const int row = rb0 + row0 + n;
    if (row < p.rows) {
      const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
      const int64_t ri = (slotp * NBT + bo + b) * p.rows + row;
      float* o = p.part_o + ri * DC + wd * DCW;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int q = 0; q < 4; ++q)
          *reinterpret_cast<f32x4*>(o + dt * 32 + 8 * q + 4 * g) =
              f32x4{acc[dt][4 * q], acc[dt][4 * q + 1], acc[dt][4 * q + 2], acc[dt][4 * q + 3]} * inv;
      if (g == 0 && wd == 0) p.part_lse[ri] = l_run > 0.f ? (m_run + __log2f(l_run)) * kLn2 : -INFINITY;
    }
    if constexpr (FUSED) {  // partial acknowledged by the L2 before the merge uses it
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      lds_signal(stored);
    }
  } else {
    // Merge the WT token streams of each compute wave's triple (see above).
    constexpr int REC = NDT * 4 + 1;  // 64-lane f32x4 rows per record
    const int tri = cw % NCW;  // (branch, row tile, slice) within a stream
    f32x4* const M = reinterpret_cast<f32x4*>(smem + lay.merge) + tri * (WT - 1) * REC * 64;
    // The stream holding the split's last sub-tile (it finishes last) merges;
    // stream mst + r (mod WT) writes record r - 1.
    const int mst = (nsub - 1) % WT;
    const int r = (strm - mst + WT) % WT;
    if (r > 0) {
      f32x4* my = M + (r - 1) * REC * 64;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int q = 0; q < 4; ++q)
          my[(dt * 4 + q) * 64 + lane] =
              f32x4{acc[dt][4 * q], acc[dt][4 * q + 1], acc[dt][4 * q + 2], acc[dt][4 * q + 3]};
      my[(REC - 1) * 64 + lane] = f32x4{m_run, l_run, 0.f, 0.f};
      lds_signal(recorded + tri);
      if constexpr (!FUSED) {
        report_expired(p.status, expired);
        return;
      }
    } else {
    // Stream mst merges the others' records with its own registers in the
    // order mst, mst + 1, ... (fixed by the split's sub-tile count, so the
    // result does not depend on which stream finished first). The others
    // took the sub-tiles before its last one, so this wait is short, and it
    // always ends.
    lds_wait_geq(recorded + tri, WT - 1, p.wait_polls, expired);
    float ms[WT], ls[WT];
    ms[0] = m_run;
    ls[0] = l_run;
#pragma unroll
    for (int w = 1; w < WT; ++w) {
      const f32x4 ml = M[((w - 1) * REC + REC - 1) * 64 + lane];
      ms[w] = ml[0];
      ls[w] = ml[1];
    }
    float mm = -INFINITY;
#pragma unroll
    for (int w = 0; w < WT; ++w) mm = fmaxf(mm, ms[w]);
    const float m_use = mm == -INFINITY ? 0.f : mm;
    float wsc[WT];
    float l = 0.f;
#pragma unroll
    for (int w = 0; w < WT; ++w) {
      wsc[w] = __builtin_amdgcn_exp2f(ms[w] - m_use);
      l += ls[w] * wsc[w];
    }
    const int row = rb0 + row0 + n;
    if (row < p.rows) {
      const float inv = l > 0.f ? 1.f / l : 0.f;
      const int64_t ri = (slotp * NBT + bo + b) * p.rows + row;
      float* o = p.part_o + ri * DC + wd * DCW;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          f32x4 v = f32x4{acc[dt][4 * q], acc[dt][4 * q + 1], acc[dt][4 * q + 2], acc[dt][4 * q + 3]} *
                    wsc[0];
#pragma unroll
          for (int w = 1; w < WT; ++w) v += M[((w - 1) * REC + dt * 4 + q) * 64 + lane] * wsc[w];
          *reinterpret_cast<f32x4*>(o + dt * 32 + 8 * q + 4 * g) = v * inv;
        }
      if (g == 0 && wd == 0) p.part_lse[ri] = l > 0.f ? (mm + __log2f(l)) * kLn2 : -INFINITY;
    }
    if constexpr (FUSED) {  // partial acknowledged by the L2 before the merge uses it
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      lds_signal(stored);
    }
    }
  }
  if constexpr (FUSED) {
    const int nsplit = min((L + kBlock * p.tps - 1) / (kBlock * p.tps), p.spl);
    fused_merge<NCW>(p, s, rr, per, nsplit, n_own, cw, lane, false, stored, go, godec, expired);
  }
  report_expired(p.status, expired);
}

// ---------------------------------------------------------------------------
// fp32 split kernel (vector ALU): one wave per (query row, branch) pair
// ---------------------------------------------------------------------------
template <int NDC>
__global__ void __launch_bounds__(256) mlra_split_valu(SplitParams p) {
  const int lane = threadIdx.x & 63;
  const int pair = blockIdx.z * 4 + (threadIdx.x >> 6);
  const int k = blockIdx.x;
  const int s = blockIdx.y;
  const int L = seq_len_of(p.seq_lens, s, p.lcap);
  const int ntiles = (L + kBlock - 1) / kBlock;
  const int t0 = k * p.tps;
  if (t0 >= ntiles || pair >= p.rows * p.NB) return;
  const int t1 = min(t0 + p.tps, ntiles);
  const int row = pair / p.NB, b = pair % p.NB;
  const int j = row / p.H, h = row % p.H;
  const int V = p.causal ? L - (p.Q - 1 - j) : L;
  const int tend = min(t1 * kBlock, V);

  const float* qlat = static_cast<const float*>(p.q_lat);
  const float* qrop = static_cast<const float*>(p.q_rope);
  const float* lat = static_cast<const float*>(p.lat);
  const float* rope = static_cast<const float*>(p.rope);
  const int64_t qb = ((((int64_t)s * p.Q + j) * p.H + h) * p.NB + b) * p.DC;
  float q[NDC];
#pragma unroll
  for (int i = 0; i < NDC; ++i) q[i] = qlat[qb + lane + 64 * i];
  const float qr = lane < p.DR ? qrop[(((int64_t)s * p.Q + j) * p.H + h) * p.DR + lane] : 0.f;

  float m = -INFINITY, l = 0.f, acc[NDC];
#pragma unroll
  for (int i = 0; i < NDC; ++i) acc[i] = 0.f;
  // kU tokens per step: their loads are all issued before the first is used
  // (indices clamped to the last visible token; the extra ones are skipped).
  constexpr int kU = 8;
  for (int tb = t0 * kBlock; tb < tend; tb += kU) {
    float c[kU][NDC], dot[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int t = min(tb + u, tend - 1);
      const int phys = clamp_block(p.table[(int64_t)s * p.max_blocks + t / kBlock], p.num_blocks);
      const int slot = t % kBlock;
      const float* cp = lat + (int64_t)phys * p.lsb + (int64_t)slot * p.lst + (int64_t)b * p.lsbr;
#pragma unroll
      for (int i = 0; i < NDC; ++i) c[u][i] = cp[lane + 64 * i];
      dot[u] = lane < p.DR ? rope[(int64_t)phys * p.rsb + (int64_t)slot * p.rst + lane] : 0.f;
    }
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      float d = 0.f;
#pragma unroll
      for (int i = 0; i < NDC; ++i) d = fmaf(q[i], c[u][i], d);
      if (lane < p.DR) d = fmaf(qr, dot[u], d);
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) d += __shfl_xor(d, off);
      dot[u] = d;
    }
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      if (tb + u >= tend) break;  // uniform
      // one value for the whole wave (the butterfly's rounding differs per lane)
      const float x = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(dot[u]))) *
                      p.score_scale;
      const float m_new = fmaxf(m, x);
      const float alpha = __builtin_amdgcn_exp2f(m - m_new);
      const float w = __builtin_amdgcn_exp2f(x - m_new);
      l = l * alpha + w;
#pragma unroll
      for (int i = 0; i < NDC; ++i) acc[i] = acc[i] * alpha + w * c[u][i];
      m = m_new;
    }
  }
  const int64_t ri = (((int64_t)s * p.spl + k) * p.NB + b) * p.rows + row;
  const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
  for (int i = 0; i < NDC; ++i) p.part_o[ri * p.DC + lane + 64 * i] = acc[i] * inv;
  if (lane == 0) p.part_lse[ri] = l > 0.f ? (m + __log2f(l)) * kLn2 : -INFINITY;
}

// ---------------------------------------------------------------------------
// combine: log-sum-exp merge of the splits, branch sum / concat, rescale
// ---------------------------------------------------------------------------
__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x = fmaxf(x, __shfl_xor(x, off));
  return x;
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off);
  return x;
}

template <typename OutT, int VPL>
__device__ __forceinline__ void store_vpl(OutT* dst, const float* v);

template <>
__device__ __forceinline__ void store_vpl<float, 1>(float* d, const float* v) { d[0] = v[0]; }
template <>
__device__ __forceinline__ void store_vpl<float, 2>(float* d, const float* v) {
  *reinterpret_cast<float2*>(d) = make_float2(v[0], v[1]);
}
template <>
__device__ __forceinline__ void store_vpl<float, 4>(float* d, const float* v) {
  *reinterpret_cast<f32x4*>(d) = f32x4{v[0], v[1], v[2], v[3]};
}
template <>
__device__ __forceinline__ void store_vpl<float, 8>(float* d, const float* v) {
  *reinterpret_cast<f32x4*>(d) = f32x4{v[0], v[1], v[2], v[3]};
  *reinterpret_cast<f32x4*>(d + 4) = f32x4{v[4], v[5], v[6], v[7]};
}
template <int VPL>
__device__ __forceinline__ void store_bf16(__bf16* d, const float* v) {
  typedef __bf16 vec __attribute__((ext_vector_type(VPL)));
  vec o;
#pragma unroll
  for (int e = 0; e < VPL; ++e) o[e] = (__bf16)v[e];
  *reinterpret_cast<vec*>(d) = o;
}
template <>
__device__ __forceinline__ void store_vpl<__bf16, 1>(__bf16* d, const float* v) { d[0] = (__bf16)v[0]; }
template <>
__device__ __forceinline__ void store_vpl<__bf16, 2>(__bf16* d, const float* v) { store_bf16<2>(d, v); }
template <>
__device__ __forceinline__ void store_vpl<__bf16, 4>(__bf16* d, const float* v) { store_bf16<4>(d, v); }
template <>
__device__ __forceinline__ void store_vpl<__bf16, 8>(__bf16* d, const float* v) { store_bf16<8>(d, v); }

// One wave (one workgroup) per (sequence, query row). Lane k holds split k's
// lse; the weights exp(lse_k - max) are broadcast with readlane while lanes
// sum the split outputs over the feature range (VPL = DC/64 values per lane).
// The first split batch's loads are issued before seq_lens has arrived
// (splits past the sequence's count are masked with selects, so stale
// workspace contents can never reach the result).
template <int VPL>
__device__ __forceinline__ void load_vpl(float (&v)[VPL], const float* src) {
  if constexpr (VPL >= 4) {
#pragma unroll
    for (int e4 = 0; e4 < VPL; e4 += 4) {
      const f32x4 t = *reinterpret_cast<const f32x4*>(src + e4);
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e4 + e] = t[e];
    }
  } else if constexpr (VPL == 2) {
    const float2 t = *reinterpret_cast<const float2*>(src);
    v[0] = t.x;
    v[1] = t.y;
  } else {
    v[0] = src[0];
  }
}

// One workgroup per (sequence, query row), one wave per branch: wave b merges
// the splits of branch b (weights exp(lse_k - lse_b)), writes lse_b and, for
// CONCAT, its output slice; for SUM the branch outputs meet in LDS and wave 0
// adds them in branch order and applies out_rescale.
template <typename OutT, int VPL, int KB>  // KB: splits whose loads are in flight together
__global__ void __launch_bounds__(256) mlra_combine(CombineParams c) {
  __shared__ float red[4 * 512];
  const int lane = threadIdx.x & 63;
  const int b = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int pair = blockIdx.x;
  const int s = pair / c.rows, row = pair % c.rows;
  const int L_raw = c.seq_lens[s];
  const int j = row / c.H, h = row % c.H;
  const int64_t orow = ((int64_t)s * c.Q + j) * c.H + h;
  const int64_t kstride = (int64_t)c.NB * c.rows;  // between splits, in rows
  const int last = c.spl - 1;
  OutT* out = static_cast<OutT*>(c.out);

  const int64_t base = ((int64_t)s * c.spl * c.NB + b) * c.rows + row;
  const float* lse_p = c.part_lse + base;
  const float* o_p = c.part_o + base * c.DC + lane * VPL;
  // Unconditional loads (indices clamped into the plan's splits) so the
  // compiler keeps them all in flight; results past the sequence's split
  // count are discarded with selects.
  float v[KB][VPL];
#pragma unroll
  for (int u = 0; u < KB; ++u) load_vpl<VPL>(v[u], o_p + (int64_t)min(u, last) * kstride * c.DC);
  const float l0 = lse_p[(int64_t)min(lane, last) * kstride];
  const int L = L_raw < 0 ? 0 : (L_raw > c.lcap ? c.lcap : L_raw);
  const int nsplit = min((L + kBlock * c.tps - 1) / (kBlock * c.tps), c.spl);
  float M = lane < nsplit ? l0 : -INFINITY;
  for (int k0 = 64; k0 < nsplit; k0 += 64) {
    const float lk = lse_p[(int64_t)min(k0 + lane, last) * kstride];
    M = fmaxf(M, k0 + lane < nsplit ? lk : -INFINITY);
  }
  M = wave_max(M);
  float o[VPL];
#pragma unroll
  for (int e = 0; e < VPL; ++e) o[e] = 0.f;
  float lse_b = -INFINITY;
  if (M != -INFINITY) {
    float den = 0.f;
    for (int k0 = 0; k0 < nsplit; k0 += 64) {
      const float lk = k0 == 0 ? l0 : lse_p[(int64_t)min(k0 + lane, last) * kstride];
      const float w = k0 + lane < nsplit ? expf(lk - M) : 0.f;
      den += w;
      const int kn = min(64, nsplit - k0);
      for (int q0 = 0; q0 < kn; q0 += KB) {
        if (k0 + q0 > 0) {
#pragma unroll
          for (int u = 0; u < KB; ++u)
            load_vpl<VPL>(v[u], o_p + (int64_t)min(k0 + q0 + u, last) * kstride * c.DC);
        }
#pragma unroll
        for (int u = 0; u < KB; ++u) {
          const bool use = q0 + u < kn;
          const float wq =
              __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w), min(q0 + u, 63)));
#pragma unroll
          for (int e = 0; e < VPL; ++e) o[e] = use ? fmaf(wq, v[u][e], o[e]) : o[e];
        }
      }
    }
    den = wave_sum(den);
    const float inv = 1.f / den;
#pragma unroll
    for (int e = 0; e < VPL; ++e) o[e] *= inv;
    lse_b = M + logf(den);
  }
  if (lane == 0) c.lse[orow * c.NB + b] = lse_b;
  if (c.concat) {
#pragma unroll
    for (int e = 0; e < VPL; ++e) o[e] *= c.out_rescale;
    store_vpl<OutT, VPL>(out + (orow * c.NB + b) * c.DC + lane * VPL, o);
    return;
  }
  if (c.NB > 1) {
#pragma unroll
    for (int e = 0; e < VPL; ++e) red[b * 64 * VPL + lane * VPL + e] = o[e];
    __syncthreads();
    if (b != 0) return;
    float tot[VPL];
#pragma unroll
    for (int e = 0; e < VPL; ++e) tot[e] = 0.f;
    for (int bb = 0; bb < c.NB; ++bb)
#pragma unroll
      for (int e = 0; e < VPL; ++e) tot[e] += red[bb * 64 * VPL + lane * VPL + e];
#pragma unroll
    for (int e = 0; e < VPL; ++e) o[e] = tot[e];
  }
#pragma unroll
  for (int e = 0; e < VPL; ++e) o[e] *= c.out_rescale;
  store_vpl<OutT, VPL>(out + orow * c.DC + lane * VPL, o);
}

// Column-sliced combine, for calls with few (sequence, query row) pairs and
// many splits (one long sequence): one workgroup per (sequence, row, CC-column
// slice), one wave per branch. Lane (kp, c) = (lane / CC, lane % CC) merges
// column c of the splits k = kp (mod 64 / CC) with a private running
// log-sum-exp, 32 splits' loads in flight per step; the split phases then
// merge through lane exchanges. Same result as mlra_combine up to the order
// of the fp32 sums.
__device__ __forceinline__ void lse_merge(float& m, float& d, float& o, float m2, float d2, float o2) {
  const float mm = fmaxf(m, m2);
  const float mu = mm == -INFINITY ? 0.f : mm;
  const float a = expf(m - mu), b = expf(m2 - mu);
  d = d * a + d2 * b;
  o = o * a + o2 * b;
  m = mm;
}
template <typename OutT, int kCombCols>
__global__ void __launch_bounds__(256) mlra_combine_cols(CombineParams c) {
  constexpr int KP = 64 / kCombCols;  // split phases per wave
  constexpr int U = 32;               // splits per lane per step
  __shared__ float red[4 * kCombCols];
  const int lane = threadIdx.x & 63;
  const int b = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int pair = blockIdx.x, slice = blockIdx.y;
  const int s = pair / c.rows, row = pair % c.rows;
  const int L_raw = c.seq_lens[s];
  const int j = row / c.H, h = row % c.H;
  const int64_t orow = ((int64_t)s * c.Q + j) * c.H + h;
  const int64_t kstride = (int64_t)c.NB * c.rows;  // between splits, in rows
  const int last = c.spl - 1;
  const int64_t base = ((int64_t)s * c.spl * c.NB + b) * c.rows + row;
  const float* lse_p = c.part_lse + base;
  const int col = slice * kCombCols + lane % kCombCols, kp = lane / kCombCols;
  const float* o_p = c.part_o + base * c.DC + col;
  const int L = L_raw < 0 ? 0 : (L_raw > c.lcap ? c.lcap : L_raw);
  const int nsplit = min((L + kBlock * c.tps - 1) / (kBlock * c.tps), c.spl);

  float m = -INFINITY, d = 0.f, o = 0.f;
  for (int k0 = 0; k0 < nsplit; k0 += KP * U) {
    float v[U], lk[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {  // clamped, unconditional: all in flight
      const int64_t k = min(k0 + kp + KP * u, last);
      v[u] = o_p[k * kstride * c.DC];
      lk[u] = lse_p[k * kstride];
    }
    // Splits past the sequence's count were never written in this call:
    // select them away (a zero weight times stale data could be NaN).
    float mc = m;
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (k0 + kp + KP * u < nsplit) mc = fmaxf(mc, lk[u]);
    const float mu = mc == -INFINITY ? 0.f : mc;
    const float sc = expf(m - mu);
    d *= sc;
    o *= sc;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const bool use = k0 + kp + KP * u < nsplit;
      const float w = expf(lk[u] - mu);
      d = use ? d + w : d;
      o = use ? fmaf(w, v[u], o) : o;
    }
    m = mc;
  }
#pragma unroll
  for (int off = kCombCols; off < 64; off <<= 1)
    lse_merge(m, d, o, __shfl_xor(m, off), __shfl_xor(d, off), __shfl_xor(o, off));
  const float lse_b = d > 0.f ? m + logf(d) : -INFINITY;
  o = d > 0.f ? o / d : 0.f;
  if (slice == 0 && lane == 0) c.lse[orow * c.NB + b] = lse_b;
  OutT* out = static_cast<OutT*>(c.out);
  if (c.concat) {
    if (kp == 0) out[(orow * c.NB + b) * c.DC + col] = (OutT)(o * c.out_rescale);
    return;
  }
  if (c.NB > 1) {
    if (kp == 0) red[b * kCombCols + lane] = o;
    __syncthreads();
    if (b != 0) return;
    float tot = 0.f;
    for (int bb = 0; bb < c.NB; ++bb) tot += red[bb * kCombCols + lane % kCombCols];
    o = tot;
  }
  if (kp == 0) out[orow * c.DC + col] = (OutT)(o * c.out_rescale);
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
template <int NBW, int RT, int DC, int DR, bool FUSED>
static hipError_t launch_pc_as(const SplitParams& sp, const mlra_decode_plan& plan,
                               hipStream_t stream) {
  constexpr int WD = pc_wd(DC);
  constexpr PcLds lay = pc_lds(NBW, RT, WD, DC, DR);
  constexpr int PL = pc_pl(NBW, DC, DR);
  auto kern = mlra_split_pc<NBW, RT, WD, DC, DR, lay.nslot, PL, FUSED>;
  static std::atomic<unsigned long long> lds_allowed{0};  // per instance, per device
  const hipError_t e = allow_dynamic_lds(reinterpret_cast<const void*>(kern), lay.total, lds_allowed);
  if (e != hipSuccess) return e;
  const dim3 grid =
      FUSED ? dim3((uint32_t)((int64_t)sp.S * plan.splits_per_seq * sp.nrt))
            : (sp.nrt == 1 ? dim3(plan.splits_per_seq, sp.S)
                           : dim3((uint32_t)(((int64_t)sp.S * plan.splits_per_seq + 7) / 8 * 8 * sp.nrt)));
  hipLaunchKernelGGL(kern, grid, dim3(512), lay.total, stream, sp);
  return hipGetLastError();
}

template <int NBW, int RT, int DC, int DR>
static hipError_t launch_pc(const SplitParams& sp, const mlra_decode_plan& plan,
                            hipStream_t stream, bool fused) {
  return fused ? launch_pc_as<NBW, RT, DC, DR, true>(sp, plan, stream)
               : launch_pc_as<NBW, RT, DC, DR, false>(sp, plan, stream);
}

template <int NBW, int RT, int DC>
static hipError_t pc_dr(const SplitParams& sp, const mlra_decode_plan& plan, hipStream_t st, bool f) {
  if (sp.DR == 64) return launch_pc<NBW, RT, DC, 64>(sp, plan, st, f);
  if constexpr (DC <= 128) return launch_pc<NBW, RT, DC, 32>(sp, plan, st, f);
  return hipErrorInvalidValue;  // wide latents take the 64-wide RoPE key only
}

template <int NBW, int RT>
static hipError_t pc_dc(const SplitParams& sp, const mlra_decode_plan& plan, hipStream_t st, bool f) {
  if (sp.DC == 128) return pc_dr<NBW, RT, 128>(sp, plan, st, f);
  if (sp.DC == 64) return pc_dr<NBW, RT, 64>(sp, plan, st, f);
  return hipErrorInvalidValue;
}

// (branches per workgroup, row tiles, latent width) as the planner chose them
static hipError_t pc_nb(const SplitParams& sp, const mlra_decode_plan& plan, hipStream_t st, bool f) {
  const int nbw = pc_nbw(sp.NB, sp.rows, sp.DC), rt = pc_rt(sp.rows, sp.DC);
  if (sp.nrt != pc_groups(sp.NB, sp.rows, sp.DC)) return hipErrorInvalidValue;
  if (sp.DC == 512) {  // one branch, four slices
    if (nbw == 1 && rt == 1 && sp.DR == 64) return launch_pc<1, 1, 512, 64>(sp, plan, st, f);
    return hipErrorInvalidValue;
  }
  if (sp.DC == 256) {  // two slices
    if (sp.DR != 64) return hipErrorInvalidValue;
    if (rt == 1 && nbw == 1) return launch_pc<1, 1, 256, 64>(sp, plan, st, f);
    if (rt == 1 && nbw == 2) return launch_pc<2, 1, 256, 64>(sp, plan, st, f);
    if (rt == 2 && nbw == 1) return launch_pc<1, 2, 256, 64>(sp, plan, st, f);
    return hipErrorInvalidValue;
  }
  if (rt == 1) {
    switch (nbw) {
      case 1: return pc_dc<1, 1>(sp, plan, st, f);
      case 2: return pc_dc<2, 1>(sp, plan, st, f);
      case 4: return pc_dc<4, 1>(sp, plan, st, f);
    }
  } else if (rt == 2) {
    switch (nbw) {
      case 1: return pc_dc<1, 2>(sp, plan, st, f);
      case 2: return pc_dc<2, 2>(sp, plan, st, f);
    }
  } else if (rt == 4 && nbw == 1) {
    return pc_dc<1, 4>(sp, plan, st, f);
  }
  return hipErrorInvalidValue;
}

static hipError_t launch_split(const SplitParams& sp, const KernelShape& ks,
                               const mlra_decode_plan& plan, hipStream_t st, bool fused) {
  if (ks.variant == kVariantPcBf16) return pc_nb(sp, plan, st, fused);
  dim3 grid(plan.splits_per_seq, sp.S, (sp.rows * sp.NB + 3) / 4);
  switch (sp.DC / 64) {
    case 1: hipLaunchKernelGGL(mlra_split_valu<1>, grid, dim3(256), 0, st, sp); break;
    case 2: hipLaunchKernelGGL(mlra_split_valu<2>, grid, dim3(256), 0, st, sp); break;
    case 4: hipLaunchKernelGGL(mlra_split_valu<4>, grid, dim3(256), 0, st, sp); break;
    case 8: hipLaunchKernelGGL(mlra_split_valu<8>, grid, dim3(256), 0, st, sp); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int VPL, int KB>
static void launch_combine_kb(bool bf16, dim3 grid, const CombineParams& cp, hipStream_t st) {
  const dim3 block(64 * cp.NB);  // one wave per branch
  if (bf16)
    hipLaunchKernelGGL((mlra_combine<__bf16, VPL, KB>), grid, block, 0, st, cp);
  else
    hipLaunchKernelGGL((mlra_combine<float, VPL, KB>), grid, block, 0, st, cp);
}

// Loads in flight per wave: enough for every split when there are few (loads
// past the split count are wasted), at most 64 registers of partials.
template <int VPL>
static void launch_combine(bool bf16, dim3 grid, const CombineParams& cp, hipStream_t st) {
  constexpr int kMax = 64 / VPL;
  if (cp.spl <= 8 || kMax <= 8)
    launch_combine_kb<VPL, 8>(bf16, grid, cp, st);
  else if (cp.spl <= 16 || kMax <= 16)
    launch_combine_kb<VPL, (kMax < 16 ? kMax : 16)>(bf16, grid, cp, st);
  else
    launch_combine_kb<VPL, (kMax < 32 ? kMax : 32)>(bf16, grid, cp, st);
}

static int device_cus(int* out) { return device_cu_count(out); }

// Process-wide bound of the split kernel's waits set by
// mlra_testing_set_wait_limit (< 0: the defaults).
static std::atomic<int> g_wait_limit{-1};

// Zero the first `words` 16-byte words at p (grid-stride).
__global__ void __launch_bounds__(256) zero_words(u32x4* p, int64_t words) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < words; i += (int64_t)gridDim.x * 256)
    p[i] = u32x4{0u, 0u, 0u, 0u};
}


// Which kernels one call enqueues: the split kernel (partial results of
// every split into the workspace), the combine kernel, or both.
enum Phase { kPartials = 1, kCombine = 2, kBoth = 3 };


static mlra_status decode(int phases, const void* q_latent, const void* q_rope,
                          const void* latent_cache, const void* rope_cache,
                          const int32_t* block_table, const int32_t* seq_lens, int32_t n_branch,
                          float scale, float out_rescale, void* out, float* lse,
                          const mlra_decode_dims* dims, void* workspace, size_t workspace_bytes,
                          void* stream) {
  Resolved r;
  mlra_status st = resolve_dims(dims, n_branch, &r);
  if (st != MLRA_OK) return st;
  const bool do_split = phases & kPartials, do_combine = phases & kCombine;
  if (!seq_lens || (do_split && (!q_latent || !q_rope || !latent_cache || !rope_cache ||
                                 !block_table)) ||
      (do_combine && (!out || !lse)))
    return MLRA_ERR_NULL_PTR;
  if (!workspace) return MLRA_ERR_WORKSPACE;
  if ((do_split && (!std::isfinite(scale) || !(scale > 0.f))) ||
      (do_combine && !std::isfinite(out_rescale)))
    return MLRA_ERR_BAD_DIMS;
  if (!aligned4(seq_lens) || !aligned16(workspace) ||
      (do_split && (!aligned16(q_latent) || !aligned16(q_rope) || !aligned16(latent_cache) ||
                    !aligned16(rope_cache) || !aligned4(block_table))) ||
      (do_combine && (!aligned16(out) || !aligned4(lse))))
    return MLRA_ERR_ALIGNMENT;
  const KernelShape ks = choose_shape(r);
  int cus = 0;
  if (device_cus(&cus) != 0) return MLRA_ERR_HIP;
  mlra_decode_plan plan;
  st = plan_call(r, ks, cus, dims->num_splits, dims->sum_seq_lens, &plan);
  if (st != MLRA_OK) return st;
  if (!workspace || workspace_bytes < plan.workspace_bytes) return MLRA_ERR_WORKSPACE;

  const int64_t slots = (int64_t)r.S * plan.splits_per_seq * r.NB * r.rows;
  char* const ws = static_cast<char*>(workspace);
  float* part_o = reinterpret_cast<float*>(ws + kWsHeaderBytes);
  float* part_lse = reinterpret_cast<float*>(ws + kWsHeaderBytes + ((slots * r.DC * 4 + 255) / 256) * 256);
  // the split kernel merges the splits itself when the plan allows it and
  // the call runs both halves
  const bool fused = plan.fused_merge && phases == kBoth;
  SplitParams sp;
  sp.q_lat = q_latent;
  sp.q_rope = q_rope;
  sp.lat = latent_cache;
  sp.rope = rope_cache;
  sp.table = block_table;
  sp.seq_lens = seq_lens;
  sp.part_o = part_o;
  sp.part_lse = part_lse;
  sp.lsb = r.lsb;
  sp.lst = r.lst;
  sp.lsbr = r.lsbr;
  sp.rsb = r.rsb;
  sp.rst = r.rst;
  sp.S = r.S;
  sp.Q = r.Q;
  sp.H = r.H;
  sp.rows = r.rows;
  sp.NB = r.NB;
  sp.DC = r.DC;
  sp.DR = r.DR;
  sp.spl = plan.splits_per_seq;
  sp.tps = plan.tiles_per_split;
  sp.max_blocks = r.max_blocks;
  sp.num_blocks = r.num_blocks;
  sp.lcap = r.lcap;
  sp.causal = r.causal;
  sp.nrt = ks.NRT;
  sp.score_scale = scale * kLog2e;
  sp.status = reinterpret_cast<unsigned*>(ws);
  sp.sync = reinterpret_cast<uint64_t*>(ws + kWsStatusBytes);
  sp.out = out;
  sp.lse = lse;
  sp.concat = r.reduce == MLRA_BRANCH_CONCAT;
  sp.out_rescale = out_rescale;
  {
    // Bounds of the in-kernel merge's waits, in 10 ns ticks. Short: 100 us
    // plus twice the time a split's tiles take at 8 GB/s per CU (far more than
    // any spread between workgroups of one sequence); long: 100 ms more.
    const int64_t tile_bytes = (int64_t)kBlock * (r.NB * r.DC + r.DR) * 2;
    sp.short_ticks = 10000 + 2 * (int64_t)plan.tiles_per_split * tile_bytes / 80;
    sp.long_ticks = 10000000 + 10 * sp.short_ticks;
    const int lim = g_wait_limit.load(std::memory_order_relaxed);
    sp.wait_polls = lim >= 0 ? lim : kDefaultWaitPolls;
    if (lim >= 0) sp.short_ticks = sp.long_ticks = lim;
  }
  hipStream_t hs = static_cast<hipStream_t>(stream);
  if (do_split && launch_split(sp, ks, plan, hs, fused) != hipSuccess) return MLRA_ERR_HIP;
  if (!do_combine || fused) return MLRA_OK;

  CombineParams cp;
  cp.part_o = part_o;
  cp.part_lse = part_lse;
  cp.seq_lens = seq_lens;
  cp.out = out;
  cp.lse = lse;
  cp.S = r.S;
  cp.Q = r.Q;
  cp.H = r.H;
  cp.rows = r.rows;
  cp.NB = r.NB;
  cp.DC = r.DC;
  cp.spl = plan.splits_per_seq;
  cp.tps = plan.tiles_per_split;
  cp.lcap = r.lcap;
  cp.concat = r.reduce == MLRA_BRANCH_CONCAT;
  cp.out_rescale = out_rescale;
  const bool bf = r.dtype == MLRA_BF16;
  // Few (sequence, row) pairs and many splits: slice the columns across
  // workgroups so that the partials are read by most of the CUs, with enough
  // split phases per wave that one step keeps a lane's loads in flight.
  if (2 * (int64_t)r.S * r.rows < plan.num_cus && plan.splits_per_seq >= 32) {
    const bool narrow = plan.splits_per_seq > 128;  // 8 columns, 8 split phases
    const dim3 grid((uint32_t)(r.S * r.rows), (uint32_t)(r.DC / (narrow ? 8 : 16)));
    const dim3 block(64 * r.NB);
    if (narrow) {
      if (bf) hipLaunchKernelGGL((mlra_combine_cols<__bf16, 8>), grid, block, 0, hs, cp);
      else hipLaunchKernelGGL((mlra_combine_cols<float, 8>), grid, block, 0, hs, cp);
    } else {
      if (bf) hipLaunchKernelGGL((mlra_combine_cols<__bf16, 16>), grid, block, 0, hs, cp);
      else hipLaunchKernelGGL((mlra_combine_cols<float, 16>), grid, block, 0, hs, cp);
    }
    return hipGetLastError() == hipSuccess ? MLRA_OK : MLRA_ERR_HIP;
  }
  dim3 cgrid(r.S * r.rows);
  switch (r.DC / 64) {
    case 1: launch_combine<1>(bf, cgrid, cp, hs); break;
    case 2: launch_combine<2>(bf, cgrid, cp, hs); break;
    case 4: launch_combine<4>(bf, cgrid, cp, hs); break;
    case 8: launch_combine<8>(bf, cgrid, cp, hs); break;
    default: return MLRA_ERR_UNSUPPORTED;
  }
  if (hipGetLastError() != hipSuccess) return MLRA_ERR_HIP;
  return MLRA_OK;
}

}  // namespace mlra

extern "C" mlra_status mlra_decode_make_plan(const mlra_decode_dims* dims, int32_t n_branch,
                                             int32_t num_cus, mlra_decode_plan* plan) {
  mlra::Resolved r;
  mlra_status st = mlra::resolve_dims(dims, n_branch, &r);
  if (st != MLRA_OK) return st;
  if (!plan) return MLRA_ERR_NULL_PTR;
  if (num_cus <= 0 && mlra::device_cus(&num_cus) != 0) return MLRA_ERR_HIP;
  return mlra::plan_call(r, mlra::choose_shape(r), num_cus, dims->num_splits,
                         dims->sum_seq_lens, plan);
}

extern "C" mlra_status mlra_decode_workspace_size(const mlra_decode_dims* dims,
                                                  int32_t n_branch, size_t* bytes) {
  if (!bytes) return MLRA_ERR_NULL_PTR;
  mlra_decode_plan plan;
  mlra_status st = mlra_decode_make_plan(dims, n_branch, 0, &plan);
  if (st != MLRA_OK) return st;
  *bytes = plan.workspace_bytes;
  return MLRA_OK;
}

extern "C" mlra_status mlra_decode_attention(const void* q_latent, const void* q_rope,
                                             const void* latent_cache, const void* rope_cache,
                                             const int32_t* block_table, const int32_t* seq_lens,
                                             int32_t n_branch, float scale, float out_rescale,
                                             void* out, float* lse, const mlra_decode_dims* dims,
                                             void* workspace, size_t workspace_bytes,
                                             void* stream) {
  return mlra::decode(mlra::kBoth, q_latent, q_rope, latent_cache, rope_cache, block_table,
                      seq_lens, n_branch, scale, out_rescale, out, lse, dims, workspace,
                      workspace_bytes, stream);
}

extern "C" mlra_status mla_decode_attention(const void* q_latent, const void* q_rope,
                                            const void* latent_cache, const void* rope_cache,
                                            const int32_t* block_table, const int32_t* seq_lens,
                                            float scale, void* out, float* lse,
                                            const mlra_decode_dims* dims, void* workspace,
                                            size_t workspace_bytes, void* stream) {
  return mlra::decode(mlra::kBoth, q_latent, q_rope, latent_cache, rope_cache, block_table,
                      seq_lens, 1, scale, 1.0f, out, lse, dims, workspace, workspace_bytes,
                      stream);
}

extern "C" mlra_status mlra_decode_partials(const void* q_latent, const void* q_rope,
                                            const void* latent_cache, const void* rope_cache,
                                            const int32_t* block_table, const int32_t* seq_lens,
                                            int32_t n_branch, float scale,
                                            const mlra_decode_dims* dims, void* workspace,
                                            size_t workspace_bytes, void* stream) {
  return mlra::decode(mlra::kPartials, q_latent, q_rope, latent_cache, rope_cache, block_table,
                      seq_lens, n_branch, scale, 1.0f, nullptr, nullptr, dims, workspace,
                      workspace_bytes, stream);
}

// ---------------------------------------------------------------------------
// Allocation-free entry point: the library's own device scratch
// ---------------------------------------------------------------------------
namespace mlra {
// Device scratch of mlra_decode_attention_static, zero when the code object
// is loaded (its header must start at zero), one copy per device that loads
// the library. Host code never uses this name as an address: each device's
// address comes from hipGetSymbolAddress (below).
constexpr size_t kStaticScratchBytes = (size_t)MLRA_STATIC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

// Device address of `scratch` on the current device, looked up once per
// device (with that device current) and kept; devices past 63 look it up on
// every call. Concurrent first calls store the same address.
static mlra_status static_scratch(void** ptr) {
  static std::atomic<void*> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return MLRA_ERR_HIP;
  if (dev >= 0 && dev < 64) {
    void* p = cache[dev].load(std::memory_order_acquire);
    if (p) {
      *ptr = p;
      return MLRA_OK;
    }
  }
  void* p = nullptr;
  if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MLRA_ERR_HIP;
  if (dev >= 0 && dev < 64) cache[dev].store(p, std::memory_order_release);
  *ptr = p;
  return MLRA_OK;
}
}  // namespace mlra

extern "C" mlra_status mlra_decode_attention_static(const void* q_latent, const void* q_rope,
                                                    const void* latent_cache,
                                                    const void* rope_cache,
                                                    const int32_t* block_table,
                                                    const int32_t* seq_lens, int32_t n_branch,
                                                    float scale, float out_rescale, void* out,
                                                    float* lse, const mlra_decode_dims* dims,
                                                    void* stream) {
  // the plan's workspace must fit the scratch (host-side, before any device work)
  mlra_decode_plan plan;
  mlra_status st = mlra_decode_make_plan(dims, n_branch, 0, &plan);
  if (st != MLRA_OK) return st;
  if (plan.workspace_bytes > mlra::kStaticScratchBytes) return MLRA_ERR_WORKSPACE;
  void* ws = nullptr;
  st = mlra::static_scratch(&ws);
  if (st != MLRA_OK) return st;
  return mlra::decode(mlra::kBoth, q_latent, q_rope, latent_cache, rope_cache, block_table,
                      seq_lens, n_branch, scale, out_rescale, out, lse, dims, ws,
                      mlra::kStaticScratchBytes, stream);
}

extern "C" mlra_status mlra_decode_workspace_init(void* workspace, size_t bytes, void* stream) {
  if (!workspace) return MLRA_ERR_NULL_PTR;
  if (bytes < (size_t)mlra::kWsHeaderBytes) return MLRA_ERR_WORKSPACE;
  if (!mlra::aligned16(workspace)) return MLRA_ERR_ALIGNMENT;
  const int64_t words = mlra::kWsHeaderBytes / 16;
  hipLaunchKernelGGL(mlra::zero_words, dim3((uint32_t)((words + 255) / 256)), dim3(256), 0,
                     static_cast<hipStream_t>(stream), static_cast<mlra::u32x4*>(workspace), words);
  return hipGetLastError() == hipSuccess ? MLRA_OK : MLRA_ERR_HIP;
}

extern "C" mlra_status mlra_decode_read_status(void* workspace, uint32_t* bits, int32_t clear,
                                               void* stream) {
  if (!workspace || !bits) return MLRA_ERR_NULL_PTR;
  if (!mlra::aligned16(workspace)) return MLRA_ERR_ALIGNMENT;
  hipStream_t hs = static_cast<hipStream_t>(stream);
  uint32_t v = 0;
  if (hipMemcpyAsync(&v, workspace, sizeof(v), hipMemcpyDeviceToHost, hs) != hipSuccess ||
      hipStreamSynchronize(hs) != hipSuccess)
    return MLRA_ERR_HIP;
  if (clear) {  // the status word's 16-byte word only
    hipLaunchKernelGGL(mlra::zero_words, dim3(1), dim3(256), 0, hs,
                       static_cast<mlra::u32x4*>(workspace), (int64_t)1);
    if (hipGetLastError() != hipSuccess) return MLRA_ERR_HIP;
  }
  *bits = v;
  return MLRA_OK;
}

extern "C" mlra_status mlra_testing_set_wait_limit(int32_t polls) {
  mlra::g_wait_limit.store(polls < 0 ? -1 : polls, std::memory_order_relaxed);
  return MLRA_OK;
}

extern "C" mlra_status mlra_decode_combine(const int32_t* seq_lens, int32_t n_branch,
                                           float out_rescale, void* out, float* lse,
                                           const mlra_decode_dims* dims, const void* workspace,
                                           size_t workspace_bytes, void* stream) {
  return mlra::decode(mlra::kCombine, nullptr, nullptr, nullptr, nullptr, nullptr, seq_lens,
                      n_branch, 1.0f, out_rescale, out, lse, dims, const_cast<void*>(workspace),
                      workspace_bytes, stream);
}
