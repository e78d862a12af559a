// Chunked-prefill MLRA attention over the paged latent cache, bf16 on MFMA.
//
// The same scores and outputs as decode (wispaper.ai blog "MLRA: Breaking
// the Sharding Bottleneck in Latent Attention", "The Core Insight: Sum of
// Branches, Not Sum of Keys": one softmax per latent branch, the branch
// outputs summed after attention; "Mathematical Calibration: Scaling the
// Latents": a fixed factor on the summed output), for a chunk of Q new query
// tokens per sequence instead of one or two. Token j of the chunk sits at
// position L - Q + j and sees every cached token up to its own position
// (the cached context, then the chunk's earlier tokens and itself).
//
// With many queries per key the work is bound by matrix throughput rather
// than by HBM (per query row and visible token the kernel does 640 flops at
// DC = 128, DR = 64, and reads nothing new). What MLRA changes is the key: every head of a query token scores the same cached
// latent and RoPE key (absorbed form), so a workgroup's rows -- 8 query
// tokens x 32 heads at H = 32 -- share one stream of cache tiles. Each
// 64-token tile is read from HBM (or L2) once per workgroup, loaded straight
// into LDS, and used by all 8 waves (two per SIMD), each holding 32 query
// rows in registers.
//
// Per wave and 32-token sub-tile:
//   S^T = [c ; k_r] [q_lat ; q_rope]^T        32x32x16 bf16 MFMA, K = DC + DR
//   online softmax per row (column of S^T), lazily rescaled
//   O^T += c^T P^T                            32x32x16 bf16 MFMA, transposed LDS reads
// software-pipelined by one sub-tile: the score MFMAs of sub-tile j are
// issued between the vector instructions that turn the scores of sub-tile
// j-1 into probabilities, so the matrix products overlap the softmax inside
// one wave's instruction stream while the SIMD's other wave covers its waits.
//
// Outputs: with one split and no branch sum (one branch, or CONCAT) the
// kernel writes out and lse directly; otherwise it writes the decode
// kernels' partial layout and a merge kernel finishes (log-sum-exp over
// splits, branch sum, output factor).
#include <algorithm>
#include <cmath>
#include <cstring>
#include <type_traits>

#include "mlra_device.h"
#include "mlra_internal.h"

namespace mlra {
namespace {

constexpr float kPfLog2e = 1.4426950408889634f;
constexpr float kPfLn2 = 0.69314718055994531f;
// Lazy softmax reference: probabilities exp2(score - m_ref) stay below 2^8.
constexpr float kPfLazyLog2 = 8.0f;
constexpr int kPfRows = 256;              // query rows per workgroup
// 32-row tiles per wave (8 / kPfNT waves): 1, two waves per SIMD, measured
// 2-4% faster than one wave per SIMD holding two tiles (kPfNT = 2)
constexpr int kPfNT = 1;
constexpr int kPfTile = kBlock;           // tokens per staged tile = one cache block
constexpr int32_t kVariantPrefillBf16 = 8;  // mlra_decode_plan.kernel_variant of prefill
constexpr int kPfMaxTiles = 1024;           // 64-token tiles per split (block ids staged in LDS)

typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

// Items (sequence, row tile, split) that a workgroup ranks to dispatch them
// longest first: each compares every pair it owns, keys in 4 KB of LDS.
constexpr int kPfOrderMaxItems = 1024;

struct PrefillParams {
  const __bf16* q_lat;
  const __bf16* q_rope;
  const __bf16* lat;
  const __bf16* rope;
  const int32_t* table;
  const int32_t* seq_lens;
  __bf16* out;
  float* lse;
  float* part_o;    // [S][spl][NB][rows][DC]
  float* part_lse;  // [S][spl][NB][rows]
  int64_t lsb, lst, lsbr, rsb, rst;
  int32_t S, Q, H, rows, NB, RT, spl, tps, max_blocks, num_blocks, lcap, causal;
  int32_t direct;     // write out/lse here (one split, no branch sum)
  int32_t order;      // 1: dispatch (sequence, row tile, split) items longest first
  int32_t concat;     // out holds every branch
  float score_scale;  // scale * log2(e): scores kept in base-2 units
  float out_rescale;
};

struct MergeParams {
  const float* part_o;
  const float* part_lse;
  const int32_t* seq_lens;
  __bf16* out;
  float* lse;
  int32_t S, Q, H, rows, NB, DC, spl, tps, lcap, causal, concat;
  float out_rescale;
};

// Tokens row r = j*H + h of a chunk may attend to (may be <= 0).
__device__ __forceinline__ int pf_visible(int L, int Q, int H, int r, int causal) {
  return causal ? L - (Q - 1 - r / H) : L;
}

__device__ __forceinline__ int pf_clamp_block(int b, int num_blocks) {
  return (b < 0 || b >= num_blocks) ? 0 : b;
}

__device__ __forceinline__ float pf_max_halves(float x) {
  // max over lanes l and l^32 (the two k-groups of a 32x32 MFMA column)
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float pf_sum_halves(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Barrier that orders LDS only (it does not wait for outstanding global
// loads, which stay in flight across it).
__device__ __forceinline__ void pf_lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// gfx950 ds_read_b64_tr_b16: within each 16-lane group, lane j supplies the
// address of 4 bf16 at row j/4, column 4*(j%4) of a 4x16 block; lane i
// receives column i, rows 0..3 of that block.
__device__ __forceinline__ i16x4 pf_read_tr(const unsigned char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) i16x4*)(const_cast<unsigned char*>(p)));
}

// 16 bytes per lane from global memory straight into LDS at lds_addr +
// 16 * lane (lds_addr wave-uniform, in M0). No register receives data;
// completion is counted by vmcnt, and the kernel waits for it explicitly
// before the barrier that publishes the tile. Written as asm rather than
// with the load-to-LDS builtin: with the builtin the compiler cannot tell
// the ring's buffers apart and waits for every tile load in flight before
// each LDS read, which serialises the prefetch.
__device__ __forceinline__ void pf_load_lds16(const void* src, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" : : "v"(src), "s"(lds_addr) : "memory", "m0");
}

__device__ __forceinline__ bf16x8 pf_rd16(const unsigned char* a) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(a));
}

// Staged tiles in LDS: a ring of four buffers, each latent rows [64][LP]
// then RoPE rows [64][RP] in 16-byte chunks (unpadded, chunks swizzled as
// above). Loads run two tiles ahead, and a wave still reads the previous
// sub-tile's value rows after the barrier that publishes the next tile:
// four buffers.
// Chunk swizzles of the staged rows: chunk c of latent row r sits at chunk
// c ^ lat_swz(r) of that row, chunk c of RoPE row r at c ^ rope_swz(r).
// With 64 LDS banks (16 chunks), a 16-byte row read serves 16 lanes at a
// time and an 8-byte transpose read 32 lanes; these swizzles put every
// such group on distinct banks (16 consecutive rows, one chunk; or 4
// consecutive rows, 4 consecutive chunks), which no single row padding
// achieves for both. Both have period 16 in r.
template <int LCH>
__device__ __forceinline__ int lat_swz(int r) {
  return LCH == 16 ? 4 * (r & 3) + ((r >> 2) & 3) : 4 * ((r >> 1) & 1) + ((r >> 2) & 3);
}
template <int RCH>
__device__ __forceinline__ int rope_swz(int r) {
  return RCH == 8 ? (r >> 1) & 7 : (r >> 2) & 3;
}

template <int DC, int DR>
struct PfLayout {
  static constexpr int LP = DC / 8, RP = DR / 8;  // unpadded rows, swizzled chunks
  static constexpr int LAT = kPfTile * LP * 16;
  static constexpr int BUF = LAT + kPfTile * RP * 16;
  static constexpr int NBUF = 4;
  static constexpr int LDS = NBUF * BUF;                     // tile ring
  static constexpr int TOTAL = LDS + kPfMaxTiles * 4;         // + block ids of a split
};

// NT 32-row tiles of queries per wave and 8/NT waves per workgroup (256
// rows either way): NT = 2 is one wave per SIMD holding 64 rows, every LDS
// operand feeding two tiles; NT = 1 is two waves per SIMD of 32 rows, so
// one wave's waits are filled by the other's work.
template <int DC, int DR, int NT>
__global__ void __launch_bounds__(64 * (8 / NT)) __attribute__((amdgpu_waves_per_eu(3 - NT, 3 - NT)))
mlra_prefill(PrefillParams p) {
  constexpr int W = 8 / NT, THREADS = 64 * W;
  constexpr int NL = DC / 16, NR = DR / 16, NDT = DC / 32;
  constexpr int LCH = DC / 8, RCH = DR / 8;
  using Lay = PfLayout<DC, DR>;
  constexpr int LP = Lay::LP, RP = Lay::RP, LAT = Lay::LAT, BUF = Lay::BUF;
  // A tile buffer is filled by direct global->LDS loads of 64 lanes x 16
  // bytes: load q covers buffer chunks 64q..64q+63; wave w issues loads
  // w, w + W, ... (NLW of the NLD; where W does not divide NLD the last ones
  // repeat load NLD-1, writing the same bytes again).
  constexpr int NLD = BUF / 1024;
  constexpr int NLW = (NLD + W - 1) / W;
  static_assert(BUF % 1024 == 0, "loads cover a buffer exactly");
  static_assert(Lay::TOTAL <= 160 * 1024, "LDS");
  static_assert(W * 32 * NT == kPfRows, "256 rows per workgroup");
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];

  // workgroup -> (split, branch, sequence, row tile). Items (sequence, row
  // tile, split) are numbered last row tile first (those see the most
  // tokens), then sequence, then split; the branches of an item take
  // consecutive workgroups.
  const int tid = threadIdx.x, lane = tid & 63;
  int item = blockIdx.x / p.NB;
  const int b = blockIdx.x % p.NB;
  if (p.order) {
    // With lengths that differ (ragged contexts), take items longest first:
    // every workgroup ranks all items by their visible tokens (ties in item
    // order, a strict total order the same in every workgroup) and takes
    // the one whose rank is its own item number. Keys live in the tile ring,
    // which no load has touched yet.
    const int G = p.S * p.RT * p.spl, G4 = (G + 3) / 4;
    int* const keys = reinterpret_cast<int*>(smem);
    int* const pick = keys + 4 * G4;
    for (int t = tid; t < 4 * G4; t += THREADS) {
      int key = -1;  // padding: below every real key
      if (t < G) {
        const int kt = t % p.spl, st = (t / p.spl) % p.S, rtt = p.RT - 1 - t / (p.spl * p.S);
        int Lt = p.seq_lens[st];
        Lt = Lt < 0 ? 0 : (Lt > p.lcap ? p.lcap : Lt);
        const int vm = max(0, pf_visible(Lt, p.Q, p.H, min(rtt * kPfRows + kPfRows, p.rows) - 1, p.causal));
        const int lo = kt * p.tps * kPfTile;
        key = max(0, min(lo + p.tps * kPfTile, vm) - lo);
      }
      keys[t] = key;
    }
    pf_lds_barrier();
    for (int t = tid; t < G; t += THREADS) {
      const int key = keys[t];
      int rank = 0;
      for (int u = 0; u < G4; ++u) {
        const int4 kk = reinterpret_cast<const int4*>(keys)[u];
        rank += (kk.x > key || (kk.x == key && 4 * u < t)) + (kk.y > key || (kk.y == key && 4 * u + 1 < t)) +
                (kk.z > key || (kk.z == key && 4 * u + 2 < t)) + (kk.w > key || (kk.w == key && 4 * u + 3 < t));
      }
      if (rank == item) *pick = t;
    }
    pf_lds_barrier();
    item = *pick;
    pf_lds_barrier();  // the ring is free again before any tile load
  }
  const int k = item % p.spl;
  const int s = (item / p.spl) % p.S;
  const int rt = p.RT - 1 - item / (p.spl * p.S);

  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 31, g = lane >> 5;
  int L = p.seq_lens[s];
  L = L < 0 ? 0 : (L > p.lcap ? p.lcap : L);
  const int r0 = rt * kPfRows;
  const int r_last = min(r0 + kPfRows, p.rows) - 1;
  const int vmax = max(0, pf_visible(L, p.Q, p.H, r_last, p.causal));
  // rows past the end see nothing, so a group holding some masks everywhere
  const int vmin = r0 + kPfRows <= p.rows ? pf_visible(L, p.Q, p.H, r0, p.causal) : 0;
  const int t_lo = k * p.tps * kPfTile;
  const int t_hi = min(t_lo + p.tps * kPfTile, vmax);
  const int nsub = t_hi > t_lo ? (t_hi - t_lo + 31) / 32 : 0;  // 32-token sub-tiles
  const int ntile = (nsub + 1) / 2;
  if (nsub == 0 && !p.direct) return;  // no row of this group has a token in the split
  // sub-tiles from jm on hold some token that some row of the group may not see
  const int jm = vmin - t_lo >= 32 ? (vmin - t_lo) / 32 : 0;

  // Row tile t of this wave: rows wr0 + 32t + n.
  const int wr0 = r0 + 32 * NT * wave;
  int row[NT], vis[NT];
  bool live[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    row[t] = wr0 + 32 * t + n;
    live[t] = row[t] < p.rows;
    vis[t] = live[t] ? pf_visible(L, p.Q, p.H, row[t], p.causal) : 0;
  }

  // Query rows in registers as the B operand of S^T: k-step st takes
  // features 8st..8st+7 (g = 0) and DC/2 + 8st.. (g = 1), the order the
  // staged rows are read in.
  bf16x8 qL[NT][NL], qR[NT][NR];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int64_t qrow = (int64_t)s * p.rows + (live[t] ? row[t] : 0);
    const __bf16* ql = p.q_lat + (qrow * p.NB + b) * DC + g * (DC / 2);
    const __bf16* qr = p.q_rope + qrow * DR + g * (DR / 2);
#pragma unroll
    for (int st = 0; st < NL; ++st) qL[t][st] = __builtin_bit_cast(bf16x8, live[t] ? ld16(ql + 8 * st) : u32x4{});
#pragma unroll
    for (int st = 0; st < NR; ++st) qR[t][st] = __builtin_bit_cast(bf16x8, live[t] ? ld16(qr + 8 * st) : u32x4{});
  }

  const int64_t tab_base = (int64_t)s * p.max_blocks;
  const int tile0 = t_lo / kPfTile;
  // The split's block ids, staged in LDS before any tile load: once tile
  // loads are in flight a vector load of the table would make the compiler
  // wait for all of them (it does not track them).
  int* const tabl = reinterpret_cast<int*>(smem + Lay::LDS);
  for (int i = tid; i < ntile; i += THREADS)
    tabl[i] = pf_clamp_block(p.table[tab_base + min(tile0 + i, p.max_blocks - 1)], p.num_blocks);
  auto block_of = [&](int i) { return __builtin_amdgcn_readfirstlane(tabl[i]); };
  const unsigned char* lat_b = reinterpret_cast<const unsigned char*>(p.lat) + (int64_t)b * p.lsbr * 2;
  const unsigned char* rope_b = reinterpret_cast<const unsigned char*>(p.rope);
  // Source of this lane's chunk in each of its loads: row, chunk, latent or RoPE.
  int lrow[NLW], lch[NLW];
  bool llat[NLW];
#pragma unroll
  for (int i = 0; i < NLW; ++i) {
    const int q = min(wave + W * i, NLD - 1);
    const int pos = 64 * q + lane;  // 16-byte chunk of the buffer
    llat[i] = pos < LAT / 16;
    const int pr = llat[i] ? pos : pos - LAT / 16;
    lrow[i] = llat[i] ? pr / LP : pr / RP;
    lch[i] = llat[i] ? (pr % LP) ^ lat_swz<LCH>(lrow[i]) : (pr % RP) ^ rope_swz<RCH>(lrow[i]);
  }
  // Tile i of the split into buffer dst: rows at or past vmax (which may
  // hold NaN) are loaded from the tile's last visible row instead; their
  // probabilities are exactly 0.
  const uint32_t lds_base = (uint32_t)(uintptr_t)((__attribute__((address_space(3))) unsigned char*)smem);
  auto issue = [&](int i, unsigned char* dst, int phys) {
    const unsigned char* lb = lat_b + (int64_t)phys * p.lsb * 2;
    const unsigned char* rb = rope_b + (int64_t)phys * p.rsb * 2;
    const int last = vmax - 1 - (tile0 + i) * kPfTile;  // >= 0: the tile holds a visible token
#pragma unroll
    for (int l = 0; l < NLW; ++l) {
      const int q = min(wave + W * l, NLD - 1);
      const int r = min(lrow[l], last);
      const unsigned char* src = llat[l] ? lb + (int64_t)r * p.lst * 2 + lch[l] * 16
                                         : rb + (int64_t)r * p.rst * 2 + lch[l] * 16;
      pf_load_lds16(src, lds_base + (uint32_t)(dst - smem) + 1024 * q);
    }
  };
  // wait until this wave's loads of the tile before the newest one (or of all) are in LDS
  auto wait_loads = [&](bool newer_in_flight) {
    if (newer_in_flight)
      __builtin_amdgcn_s_waitcnt(0x0F70 | NLW);  // vmcnt(NLW)
    else
      __builtin_amdgcn_s_waitcnt(0x0F70);        // vmcnt(0)
  };

  f32x16 acc[NT][NDT];
  float m[NT], l[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    m[t] = -INFINITY;
    l[t] = 0.f;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) acc[t][dt] = f32x16{};
  }

  // LDS byte offsets this lane reads inside a 32-token sub-tile (all
  // swizzles have period 16 in the row, so sub-tiles and the row halves
  // 16..31 reuse them): S^T A operands (token row n, k-step st), and the
  // transposed C^T operands (rows r0 + 8*half (+16), feature tile dt).
  int a_l[NL], a_r[NR], a_t[2][NDT];
#pragma unroll
  for (int st = 0; st < NL; ++st) a_l[st] = (n * LP + ((g * (LCH / 2) + st) ^ lat_swz<LCH>(n))) * 16;
#pragma unroll
  for (int st = 0; st < NR; ++st) a_r[st] = LAT + (n * RP + ((g * (RCH / 2) + st) ^ rope_swz<RCH>(n))) * 16;
  {
    const int tr0 = 4 * (lane >> 5) + ((lane & 15) >> 2);
    const int lc0 = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
#pragma unroll
    for (int half = 0; half < 2; ++half)
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
        a_t[half][dt] = (tr0 + 8 * half) * LP * 16 +
                        (((lc0 + 4 * dt) ^ lat_swz<LCH>(tr0 + 8 * half)) * 16) + (lane & 1) * 8;
  }

  // S^T of the wave's row tiles for sub-tile u of the tile at buf.
  auto scores = [&](const unsigned char* buf, int u, f32x16 (&sc)[NT]) {
    bf16x8 aR[NR], aL[NL];
    const unsigned char* sl = buf + u * 32 * LP * 16;
    const unsigned char* sr = buf + u * 32 * RP * 16;
#pragma unroll
    for (int st = 0; st < NR; ++st) aR[st] = pf_rd16(sr + a_r[st]);
#pragma unroll
    for (int st = 0; st < NL; ++st) aL[st] = pf_rd16(sl + a_l[st]);
#pragma unroll
    for (int t = 0; t < NT; ++t) sc[t] = f32x16{};
#pragma unroll
    for (int st = 0; st < NR; ++st)
#pragma unroll
      for (int t = 0; t < NT; ++t) sc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aR[st], qR[t][st], sc[t], 0, 0, 0);
#pragma unroll
    for (int st = 0; st < NL; ++st)
#pragma unroll
      for (int t = 0; t < NT; ++t) sc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aL[st], qL[t][st], sc[t], 0, 0, 0);
  };
  // Row maxima of a sub-tile (first token tb), in base-2 units, then the
  // lazily moved reference maximum: rescale only when a row maximum exceeds
  // it by more than kPfLazyLog2 (log2 units). With MASK, tokens at or past
  // a row's visible length become -inf first; element r of lane (n, g)
  // holds token tb + 4g + 8(r/4) + r%4.
  auto settle = [&](f32x16 (&sc)[NT], int tb, auto mask) {
    float mx[NT];
    bool first[NT], grow[NT], any = false, rescale = false;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      if constexpr (decltype(mask)::value) {
        const int lim = vis[t] - tb - 4 * g;
#pragma unroll
        for (int r = 0; r < 16; ++r) sc[t][r] = 8 * (r >> 2) + (r & 3) < lim ? sc[t][r] : -INFINITY;
      }
      float x = -INFINITY;
#pragma unroll
      for (int r = 0; r < 16; ++r) x = fmaxf(x, sc[t][r]);
      mx[t] = pf_max_halves(x) * p.score_scale;
      first[t] = m[t] == -INFINITY;
      grow[t] = first[t] ? mx[t] > -INFINITY : mx[t] > m[t] + kPfLazyLog2;
      any = any || grow[t];
      rescale = rescale || (grow[t] && !first[t]);
    }
    if (__builtin_amdgcn_ballot_w64(any)) {
      float al[NT];
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        al[t] = grow[t] ? __builtin_amdgcn_exp2f(m[t] - mx[t]) : 1.f;
        m[t] = grow[t] ? mx[t] : m[t];
        l[t] *= al[t];
      }
      if (__builtin_amdgcn_ballot_w64(rescale)) {
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
          for (int dt = 0; dt < NDT; ++dt) acc[t][dt] *= al[t];
      }
    }
  };
  // Probabilities of a sub-tile against the reference, as the B operand of
  // O^T += C^T P^T, and their sums.
  auto probs = [&](const f32x16 (&sc)[NT], bf16x8 (&pb)[NT][2]) {
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const float m_use = m[t] == -INFINITY ? 0.f : m[t];
      float ps[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float pe = __builtin_amdgcn_exp2f(fmaf(sc[t][8 * h2 + e], p.score_scale, -m_use));
          ps[e & 3] += pe;
          pb[t][h2][e] = (__bf16)pe;
        }
      l[t] += (ps[0] + ps[1]) + (ps[2] + ps[3]);
    }
  };
  // O^T += C^T P^T for the wave's row tiles; value rows (the sub-tile's latent) at vl.
  auto values = [&](const unsigned char* vl, const bf16x8 (&pb)[NT][2]) {
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        const i16x4 lo = pf_read_tr(vl + a_t[0][dt] + (16 * h2) * LP * 16);
        const i16x4 hi = pf_read_tr(vl + a_t[1][dt] + (16 * h2) * LP * 16);
        const bf16x8 at = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
        for (int t = 0; t < NT; ++t)
          acc[t][dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(at, pb[t][h2], acc[t][dt], 0, 0, 0);
      }
  };

  if (nsub > 0) {
    // Software pipeline over 32-token sub-tiles j: iteration j computes the
    // scores of j while the probabilities of j-1 are formed and multiplied
    // into the outputs, so the vector work of one sub-tile runs beside the
    // matrix work of the next. Tile i (sub-tiles 2i, 2i+1) sits in buffer
    // i % 4; its loads leave at the start of iteration 2i-4 (two tiles
    // ahead), and at the start of iteration 2i each wave waits for its own
    // loads of it and a barrier publishes them. The buffer those loads
    // write last held tile i-4, whose last reads were in iteration 2i-6,
    // before the barrier of iteration 2i-4 that precedes them.
    pf_lds_barrier();  // block ids staged
    issue(0, smem, block_of(0));
    if (ntile > 1) issue(1, smem + BUF, block_of(1));
    wait_loads(ntile > 1);
    pf_lds_barrier();
    // the transition into tile 0: tile 2 leaves now
    if (ntile > 2) issue(2, smem + 2 * BUF, block_of(2));
    int phys_next = ntile > 3 ? block_of(3) : 0;
    f32x16 sc[NT];
    scores(smem, 0, sc);
    if (jm == 0)
      settle(sc, t_lo, std::true_type{});
    else
      settle(sc, t_lo, std::false_type{});
    int cur = 0, prev = 0;  // buffers of sub-tiles j and j-1
    auto step = [&](int j, auto mask) {
      prev = cur;
      if ((j & 1) == 0) {
        const int t = j >> 1;
        cur = (cur + 1) & 3;
        wait_loads(t + 1 < ntile);
        pf_lds_barrier();
        if (t + 2 < ntile) {
          issue(t + 2, smem + ((cur + 2) & 3) * BUF, phys_next);
          phys_next = t + 3 < ntile ? block_of(t + 3) : 0;
        }
      }
      f32x16 nsc[NT];
      scores(smem + cur * BUF, j & 1, nsc);
      bf16x8 pb[NT][2];
      probs(sc, pb);
      values(smem + prev * BUF + ((j - 1) & 1) * 32 * LP * 16, pb);
#pragma unroll
      for (int t = 0; t < NT; ++t) sc[t] = nsc[t];
      settle(sc, t_lo + 32 * j, mask);
    };
    const int j1 = min(max(jm, 1), nsub);
    for (int j = 1; j < j1; ++j) step(j, std::false_type{});
    for (int j = j1; j < nsub; ++j) step(j, std::true_type{});
    bf16x8 pb[NT][2];
    probs(sc, pb);
    values(smem + cur * BUF + ((nsub - 1) & 1) * 32 * LP * 16, pb);
  }

  // O^T element (dt, r) of lane (n, g) is feature dt*32 + 8(r/4) + 4g + r%4 of row n
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const float lt = pf_sum_halves(l[t]);
    if (!live[t]) continue;
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    const float lse_v = lt > 0.f ? (m[t] + __log2f(lt)) * kPfLn2 : -INFINITY;
    if (p.direct) {
      const float f = inv * p.out_rescale;
      __bf16* o = p.out + ((int64_t)(s * (int64_t)p.rows + row[t]) * (p.concat ? p.NB : 1) +
                           (p.concat ? b : 0)) * DC;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          bf16x4 v;
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = (__bf16)(acc[t][dt][4 * q + e] * f);
          *reinterpret_cast<bf16x4*>(o + dt * 32 + 8 * q + 4 * g) = v;
        }
      if (g == 0) p.lse[((int64_t)s * p.rows + row[t]) * p.NB + b] = lse_v;
    } else {
      const int64_t ri = (((int64_t)s * p.spl + k) * p.NB + b) * p.rows + row[t];
      float* o = p.part_o + ri * DC;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int q = 0; q < 4; ++q)
          *reinterpret_cast<f32x4*>(o + dt * 32 + 8 * q + 4 * g) =
              f32x4{acc[t][dt][4 * q], acc[t][dt][4 * q + 1], acc[t][dt][4 * q + 2], acc[t][dt][4 * q + 3]} * inv;
      if (g == 0) p.part_lse[ri] = lse_v;
    }
  }
}

// Merge of split partials: one thread per (sequence, row, 4 features). Row r
// has tokens in splits k < ceil(V_r / (64 * tps)); each split's output is
// weighted by exp(lse_k - lse), lse = ln sum_k exp(lse_k). Branch outputs
// are summed (or kept apart) and multiplied by the output factor.
__global__ void __launch_bounds__(256) mlra_prefill_merge(MergeParams p) {
  const int dc4 = p.DC / 4;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (int64_t)p.S * p.rows * dc4) return;
  const int c4 = (int)(idx % dc4);
  const int64_t sr = idx / dc4;
  const int s = (int)(sr / p.rows), r = (int)(sr % p.rows);
  int L = p.seq_lens[s];
  L = L < 0 ? 0 : (L > p.lcap ? p.lcap : L);
  const int V = pf_visible(L, p.Q, p.H, r, p.causal);
  const int64_t span = (int64_t)p.tps * kPfTile;
  const int nv = V > 0 ? (int)std::min<int64_t>((V + span - 1) / span, p.spl) : 0;
  f32x4 sum = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int b = 0; b < p.NB; ++b) {
    float m = -INFINITY;
    for (int k = 0; k < nv; ++k)
      m = fmaxf(m, p.part_lse[(((int64_t)s * p.spl + k) * p.NB + b) * p.rows + r]);
    f32x4 o = f32x4{0.f, 0.f, 0.f, 0.f};
    float wsum = 0.f;
    if (m > -INFINITY) {
      for (int k = 0; k < nv; ++k) {
        const int64_t ri = (((int64_t)s * p.spl + k) * p.NB + b) * p.rows + r;
        const float lk = p.part_lse[ri];
        if (!(lk > -INFINITY)) continue;  // a split without visible tokens holds no output
        const float w = expf(lk - m);
        wsum += w;
        o += w * *reinterpret_cast<const f32x4*>(p.part_o + ri * p.DC + 4 * c4);
      }
      o *= 1.f / wsum;
    }
    if (c4 == 0) p.lse[sr * p.NB + b] = m > -INFINITY ? m + logf(wsum) : -INFINITY;
    if (p.concat) {
      bf16x4 v;
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = (__bf16)(o[e] * p.out_rescale);
      *reinterpret_cast<bf16x4*>(p.out + (sr * p.NB + b) * p.DC + 4 * c4) = v;
    } else {
      sum += o;
    }
  }
  if (!p.concat) {
    bf16x4 v;
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = (__bf16)(sum[e] * p.out_rescale);
    *reinterpret_cast<bf16x4*>(p.out + sr * p.DC + 4 * c4) = v;
  }
}

int64_t pf_cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

int pf_device_cus(int* out) { return device_cu_count(out); }

// Validation: the decode rules for everything but the query count (checked
// with one query row), then the prefill kernel's own limits.
mlra_status prefill_resolve(const mlra_decode_dims* d, int32_t n_branch, Resolved* r) {
  if (!d || !r) return MLRA_ERR_NULL_PTR;
  if (d->num_heads < 1 || d->q_len < 1) return MLRA_ERR_BAD_DIMS;
  mlra_decode_dims one = *d;
  one.q_len = 1;
  one.num_heads = 1;
  mlra_status st = resolve_dims(&one, n_branch, r);
  if (st != MLRA_OK) return st;
  if (d->dtype != MLRA_BF16) return MLRA_ERR_UNSUPPORTED;
  if (d->d_latent != 64 && d->d_latent != 128) return MLRA_ERR_UNSUPPORTED;
  const int64_t rows = (int64_t)d->num_heads * d->q_len;
  if (rows > (int64_t(1) << 26)) return MLRA_ERR_UNSUPPORTED;
  r->Q = d->q_len;
  r->H = d->num_heads;
  r->rows = (int32_t)rows;
  return MLRA_OK;
}

// Split plan: row tiles x sequences x branches workgroups; when they do not
// fill the CUs, sequences are also split along their tokens (at least two
// tiles per split), as decode does.
mlra_status prefill_plan(const Resolved& r, int32_t num_cus, int32_t num_splits,
                         mlra_decode_plan* plan, bool* direct) {
  if (num_cus < 1) return MLRA_ERR_BAD_DIMS;
  const int64_t RT = pf_cdiv(r.rows, kPfRows);
  const int64_t base = RT * r.S * r.NB;
  const int64_t max_tiles = std::max<int64_t>(1, pf_cdiv(r.lcap, kPfTile));
  int64_t want;
  if (num_splits > 0)
    want = num_splits;
  else if (base >= num_cus)
    want = 1;
  else
    want = std::min<int64_t>(pf_cdiv(num_cus, base), std::max<int64_t>(1, max_tiles / 2));
  // a split's block ids are staged in LDS: at most kPfMaxTiles tiles
  want = std::max<int64_t>(want, pf_cdiv(max_tiles, kPfMaxTiles));
  const int64_t tps = pf_cdiv(max_tiles, std::min<int64_t>(want, max_tiles));
  const int64_t spl = pf_cdiv(max_tiles, tps);
  if (base * spl > INT32_MAX) return MLRA_ERR_UNSUPPORTED;
  const bool dir = spl == 1 && (r.NB == 1 || r.reduce == MLRA_BRANCH_CONCAT);
  // the merge runs one thread per (sequence, row, 4 features)
  if (!dir && pf_cdiv((int64_t)r.S * r.rows * (r.DC / 4), 256) > INT32_MAX) return MLRA_ERR_UNSUPPORTED;
  mlra_decode_plan p;
  std::memset(&p, 0, sizeof(p));
  p.num_cus = num_cus;
  p.target_groups = (int32_t)(base * spl);
  p.waves_per_group = 8 / kPfNT;
  p.tiles_per_split = (int32_t)tps;
  p.splits_per_seq = (int32_t)spl;
  p.kernel_variant = kVariantPrefillBf16;
  p.lds_bytes = r.DC == 128 ? (r.DR == 64 ? PfLayout<128, 64>::TOTAL : PfLayout<128, 32>::TOTAL)
                            : (r.DR == 64 ? PfLayout<64, 64>::TOTAL : PfLayout<64, 32>::TOTAL);
  p.row_groups = (int32_t)RT;
  if (!dir) {
    const int64_t slots = (int64_t)r.S * spl * r.NB * r.rows;
    // after the header every workspace of the library starts with (it belongs
    // to decode calls, so one buffer can serve both)
    p.workspace_bytes = (size_t)(kWsHeaderBytes + pf_cdiv(slots * r.DC * 4, 256) * 256 +
                                 pf_cdiv(slots * 4, 256) * 256);
  }
  *plan = p;
  *direct = dir;
  return MLRA_OK;
}

template <int DC, int DR>
hipError_t launch_prefill(const PrefillParams& pp, int64_t groups, hipStream_t st) {
  constexpr uint32_t lds = PfLayout<DC, DR>::TOTAL;
  static std::atomic<unsigned long long> lds_allowed{0};  // per instance, per device
  const hipError_t attr = allow_dynamic_lds(reinterpret_cast<const void*>(&mlra_prefill<DC, DR, kPfNT>),
                                            (int)lds, lds_allowed);
  if (attr != hipSuccess) return attr;
  hipLaunchKernelGGL((mlra_prefill<DC, DR, kPfNT>), dim3((uint32_t)groups), dim3(64 * (8 / kPfNT)), lds,
                     st, pp);
  return hipGetLastError();
}

}  // namespace
}  // namespace mlra

extern "C" mlra_status mlra_prefill_make_plan(const mlra_decode_dims* dims, int32_t n_branch,
                                              int32_t num_cus, mlra_decode_plan* plan) {
  mlra::Resolved r;
  mlra_status st = mlra::prefill_resolve(dims, n_branch, &r);
  if (st != MLRA_OK) return st;
  if (!plan) return MLRA_ERR_NULL_PTR;
  if (num_cus <= 0 && mlra::pf_device_cus(&num_cus) != 0) return MLRA_ERR_HIP;
  bool direct = false;
  return mlra::prefill_plan(r, num_cus, dims->num_splits, plan, &direct);
}

extern "C" mlra_status mlra_prefill_workspace_size(const mlra_decode_dims* dims, int32_t n_branch,
                                                   size_t* bytes) {
  if (!bytes) return MLRA_ERR_NULL_PTR;
  mlra_decode_plan plan;
  mlra_status st = mlra_prefill_make_plan(dims, n_branch, 0, &plan);
  if (st != MLRA_OK) return st;
  *bytes = plan.workspace_bytes;
  return MLRA_OK;
}

extern "C" mlra_status mlra_prefill_attention(const void* q_latent, const void* q_rope,
                                              const void* latent_cache, const void* rope_cache,
                                              const int32_t* block_table, const int32_t* seq_lens,
                                              int32_t n_branch, float scale, float out_rescale,
                                              void* out, float* lse, const mlra_decode_dims* dims,
                                              void* workspace, size_t workspace_bytes,
                                              void* stream) {
  using namespace mlra;
  Resolved r;
  mlra_status st = prefill_resolve(dims, n_branch, &r);
  if (st != MLRA_OK) return st;
  if (!q_latent || !q_rope || !latent_cache || !rope_cache || !block_table || !seq_lens || !out ||
      !lse)
    return MLRA_ERR_NULL_PTR;
  if (!std::isfinite(scale) || !(scale > 0.f) || !std::isfinite(out_rescale))
    return MLRA_ERR_BAD_DIMS;
  if (!aligned16(q_latent) || !aligned16(q_rope) || !aligned16(latent_cache) ||
      !aligned16(rope_cache) || !aligned4(block_table) || !aligned4(seq_lens) ||
      !aligned16(out) || !aligned4(lse) || (workspace && !aligned16(workspace)))
    return MLRA_ERR_ALIGNMENT;
  int cus = 0;
  if (pf_device_cus(&cus) != 0) return MLRA_ERR_HIP;
  mlra_decode_plan plan;
  bool direct = false;
  st = prefill_plan(r, cus, dims->num_splits, &plan, &direct);
  if (st != MLRA_OK) return st;
  if (plan.workspace_bytes > 0 && (!workspace || workspace_bytes < plan.workspace_bytes))
    return MLRA_ERR_WORKSPACE;

  const int64_t slots = (int64_t)r.S * plan.splits_per_seq * r.NB * r.rows;
  PrefillParams pp;
  pp.q_lat = static_cast<const __bf16*>(q_latent);
  pp.q_rope = static_cast<const __bf16*>(q_rope);
  pp.lat = static_cast<const __bf16*>(latent_cache);
  pp.rope = static_cast<const __bf16*>(rope_cache);
  pp.table = block_table;
  pp.seq_lens = seq_lens;
  pp.out = static_cast<__bf16*>(out);
  pp.lse = lse;
  char* const wsp = direct ? nullptr : static_cast<char*>(workspace) + kWsHeaderBytes;  // past the header
  pp.part_o = direct ? nullptr : reinterpret_cast<float*>(wsp);
  pp.part_lse = direct ? nullptr : reinterpret_cast<float*>(wsp + pf_cdiv(slots * r.DC * 4, 256) * 256);
  pp.lsb = r.lsb;
  pp.lst = r.lst;
  pp.lsbr = r.lsbr;
  pp.rsb = r.rsb;
  pp.rst = r.rst;
  pp.S = r.S;
  pp.Q = r.Q;
  pp.H = r.H;
  pp.rows = r.rows;
  pp.NB = r.NB;
  pp.RT = plan.row_groups;
  pp.spl = plan.splits_per_seq;
  pp.tps = plan.tiles_per_split;
  pp.max_blocks = r.max_blocks;
  pp.num_blocks = r.num_blocks;
  pp.lcap = r.lcap;
  pp.causal = r.causal;
  pp.direct = direct ? 1 : 0;
  // Longest-first dispatch unless the length hint says every sequence has the
  // same length (then the fixed order is already longest first), and only
  // while ranking the items stays cheap for every workgroup.
  const int64_t items = (int64_t)r.S * plan.row_groups * plan.splits_per_seq;
  const bool uniform = dims->sum_seq_lens > 0 && dims->sum_seq_lens == (int64_t)r.S * r.lcap;
  pp.order = items <= kPfOrderMaxItems && !uniform ? 1 : 0;
  pp.concat = r.reduce == MLRA_BRANCH_CONCAT ? 1 : 0;
  pp.score_scale = scale * kPfLog2e;
  pp.out_rescale = out_rescale;
  hipStream_t hs = static_cast<hipStream_t>(stream);
  const int64_t groups = (int64_t)plan.target_groups;
  hipError_t e;
  if (r.DC == 128)
    e = r.DR == 64 ? launch_prefill<128, 64>(pp, groups, hs) : launch_prefill<128, 32>(pp, groups, hs);
  else
    e = r.DR == 64 ? launch_prefill<64, 64>(pp, groups, hs) : launch_prefill<64, 32>(pp, groups, hs);
  if (e != hipSuccess) return MLRA_ERR_HIP;
  if (direct) return MLRA_OK;

  MergeParams mp;
  mp.part_o = pp.part_o;
  mp.part_lse = pp.part_lse;
  mp.seq_lens = seq_lens;
  mp.out = pp.out;
  mp.lse = lse;
  mp.S = r.S;
  mp.Q = r.Q;
  mp.H = r.H;
  mp.rows = r.rows;
  mp.NB = r.NB;
  mp.DC = r.DC;
  mp.spl = plan.splits_per_seq;
  mp.tps = plan.tiles_per_split;
  mp.lcap = r.lcap;
  mp.causal = r.causal;
  mp.concat = pp.concat;
  mp.out_rescale = out_rescale;
  const int64_t threads = (int64_t)r.S * r.rows * (r.DC / 4);
  hipLaunchKernelGGL(mlra_prefill_merge, dim3((uint32_t)pf_cdiv(threads, 256)), dim3(256), 0, hs, mp);
  return hipGetLastError() == hipSuccess ? MLRA_OK : MLRA_ERR_HIP;
}
