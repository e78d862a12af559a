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
// This is the regime the FlashAttention-3 pages describe for prefill: many
// queries per key, bound by matrix throughput rather than by HBM. What MLRA
// changes is the key: every head of a query token scores the same cached
// latent and RoPE key (absorbed form), so a workgroup's rows -- 8 query
// tokens x 32 heads at H = 32 -- share one stream of cache tiles. Each
// 64-token tile is read from HBM (or L2) once per workgroup, staged in LDS,
// and used by all 8 waves; one wave holds 32 query rows in registers.
//
// Per wave and 32-token sub-tile (the loop body of the decode kernels):
//   S^T = [c ; k_r] [q_lat ; q_rope]^T        32x32x16 bf16 MFMA, K = DC + DR
//   online softmax per row (column of S^T), lazily rescaled
//   O^T += c^T P^T                            32x32x16 bf16 MFMA, transposed LDS reads
// Rows of one wave share a query token when H is a multiple of 32, so the
// causal edge is wave-uniform there; elsewhere each lane masks its own row.
//
// Outputs: with one split and no branch sum (one branch, or CONCAT) the
// kernel writes out and lse directly; otherwise it writes the decode
// kernels' partial layout and a merge kernel finishes (log-sum-exp over
// splits, branch sum, output factor).
#include <algorithm>
#include <cmath>
#include <cstring>

#include "mlra_device.h"
#include "mlra_internal.h"

namespace mlra {
namespace {

constexpr float kPfLog2e = 1.4426950408889634f;
constexpr float kPfLn2 = 0.69314718055994531f;
// Lazy softmax reference: probabilities exp2(score - m_ref) stay below 2^8.
constexpr float kPfLazyLog2 = 8.0f;
constexpr int kPfWaves = 8;               // two per SIMD
constexpr int kPfThreads = 64 * kPfWaves;
constexpr int kPfRows = 32 * kPfWaves;    // query rows per workgroup
constexpr int kPfTile = kBlock;           // tokens per staged tile = one cache block
constexpr int32_t kVariantPrefillBf16 = 8;  // mlra_decode_plan.kernel_variant of prefill

typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

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

__device__ __forceinline__ bf16x8 pf_rd16(const unsigned char* a) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(a));
}

// Staged tile in LDS: latent rows [64][LP] then RoPE rows [64][RP], in
// 16-byte chunks. Latent rows carry 2 spare chunks and RoPE rows 1, the
// pitches under which the decode kernels' row reads (8 lanes, one chunk of
// 8 consecutive rows) and 16-lane transpose reads (4 rows x 32 bytes) land
// on distinct banks.
template <int DC, int DR>
struct PfLayout {
  static constexpr int LP = DC / 8 + 2, RP = DR / 8 + 1;
  static constexpr int LAT = kPfTile * LP * 16;
  static constexpr int BUF = LAT + kPfTile * RP * 16;
  static constexpr int LDS = 2 * BUF;  // double buffered
};

template <int DC, int DR>
__global__ void __launch_bounds__(kPfThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
mlra_prefill(PrefillParams p) {
  constexpr int NL = DC / 16, NR = DR / 16, NDT = DC / 32;
  constexpr int LCH = DC / 8, RCH = DR / 8;
  using Lay = PfLayout<DC, DR>;
  constexpr int LP = Lay::LP, RP = Lay::RP, LAT = Lay::LAT, BUF = Lay::BUF;
  constexpr int NCH = kPfTile * (LCH + RCH);              // 16-byte chunks per tile
  constexpr int CPT = (NCH + kPfThreads - 1) / kPfThreads;  // per thread
  static_assert((kPfTile * LCH) % kPfThreads == 0, "latent/RoPE split is uniform per load");
  static_assert(Lay::LDS <= 64 * 1024, "LDS");
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];

  // workgroup -> (split, branch, sequence, row tile); the last row tiles,
  // which see the most tokens, are dispatched first
  int id = blockIdx.x;
  const int k = id % p.spl;
  id /= p.spl;
  const int b = id % p.NB;
  id /= p.NB;
  const int s = id % p.S;
  const int rt = p.RT - 1 - id / p.S;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 31, g = lane >> 5;
  int L = p.seq_lens[s];
  L = L < 0 ? 0 : (L > p.lcap ? p.lcap : L);
  const int r0 = rt * kPfRows;
  const int vmax = max(0, pf_visible(L, p.Q, p.H, min(r0 + kPfRows, p.rows) - 1, p.causal));
  const int t_lo = k * p.tps * kPfTile;
  const int t_hi = min(t_lo + p.tps * kPfTile, vmax);
  const int ntile = t_hi > t_lo ? (t_hi - t_lo + kPfTile - 1) / kPfTile : 0;
  if (ntile == 0 && !p.direct) return;  // no row of this group has a token in the split

  // this lane's row, its visible length, and the wave's extremes (rows past
  // the end see nothing)
  const int wr0 = r0 + 32 * wave;
  const int row = wr0 + n;
  const bool live = row < p.rows;
  const int vis = live ? pf_visible(L, p.Q, p.H, row, p.causal) : 0;
  const int wmin = wr0 + 31 < p.rows ? pf_visible(L, p.Q, p.H, wr0, p.causal) : 0;
  const int wmax = wr0 < p.rows ? pf_visible(L, p.Q, p.H, min(wr0 + 31, p.rows - 1), p.causal) : 0;

  // Query rows in registers as the B operand of S^T: k-step st takes
  // features 8st..8st+7 (g = 0) and DC/2 + 8st.. (g = 1), the order the
  // staged rows are read in.
  const int64_t qrow = (int64_t)s * p.rows + (live ? row : 0);
  const __bf16* ql = p.q_lat + (qrow * p.NB + b) * DC + g * (DC / 2);
  const __bf16* qr = p.q_rope + qrow * DR + g * (DR / 2);
  bf16x8 qL[NL], qR[NR];
#pragma unroll
  for (int st = 0; st < NL; ++st) qL[st] = __builtin_bit_cast(bf16x8, live ? ld16(ql + 8 * st) : u32x4{});
#pragma unroll
  for (int st = 0; st < NR; ++st) qR[st] = __builtin_bit_cast(bf16x8, live ? ld16(qr + 8 * st) : u32x4{});

  // Tile loads: thread tid moves chunks tid, tid + 512, ... of a tile.
  // Offsets inside a block, and the LDS destinations, are fixed per thread.
  uint32_t goff[CPT], loff[CPT];
  int gtok[CPT];
  bool isl[CPT], has[CPT];
#pragma unroll
  for (int c = 0; c < CPT; ++c) {
    const int x = c * kPfThreads + tid;
    has[c] = x < NCH;
    isl[c] = x < kPfTile * LCH;
    const int y = x - kPfTile * LCH;
    gtok[c] = isl[c] ? x / LCH : y / RCH;
    goff[c] = isl[c] ? (uint32_t)(gtok[c] * p.lst * 2 + (x % LCH) * 16)
                     : (uint32_t)(gtok[c] * p.rst * 2 + (y % RCH) * 16);
    loff[c] = isl[c] ? (uint32_t)((gtok[c] * LP + x % LCH) * 16)
                     : (uint32_t)(LAT + (gtok[c] * RP + y % RCH) * 16);
  }
  const int64_t tab_base = (int64_t)s * p.max_blocks;
  const int tile0 = t_lo / kPfTile;
  // block ids of 64 consecutive tiles, one per lane, the next 64 in flight
  auto tab_load = [&](int i) { return p.table[tab_base + min(tile0 + i + lane, p.max_blocks - 1)]; };
  int tabA = 0, tabB = 0;
  if (ntile > 0) {
    tabA = tab_load(0);
    tabB = ntile > 64 ? tab_load(64) : 0;
  }
  const unsigned char* lat_b = reinterpret_cast<const unsigned char*>(p.lat) + (int64_t)b * p.lsbr * 2;
  const unsigned char* rope_b = reinterpret_cast<const unsigned char*>(p.rope);
  u32x4 buf[CPT];
  auto issue = [&](int i) {  // tile i of the split: global -> registers
    if (i > 0 && (i & 63) == 0) {
      tabA = tabB;
      tabB = i + 64 < ntile ? tab_load(i + 64) : 0;
    }
    const int phys = pf_clamp_block(__builtin_amdgcn_readlane(tabA, i & 63), p.num_blocks);
    const unsigned char* lb = lat_b + (int64_t)phys * p.lsb * 2;
    const unsigned char* rb = rope_b + (int64_t)phys * p.rsb * 2;
#pragma unroll
    for (int c = 0; c < CPT; ++c)
      if (has[c]) buf[c] = ld16((isl[c] ? lb : rb) + goff[c]);
  };
  auto stage = [&](int i, unsigned char* dst) {  // registers -> LDS, rows past vmax zeroed
    const int tok0 = (tile0 + i) * kPfTile;
#pragma unroll
    for (int c = 0; c < CPT; ++c)
      if (has[c]) *reinterpret_cast<u32x4*>(dst + loff[c]) = tok0 + gtok[c] < vmax ? buf[c] : u32x4{};
  };

  f32x16 acc[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) acc[dt] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;

  const int a_l = (n * LP + g * (LCH / 2)) * 16;  // S^T A operand: token row n
  const int a_r = (n * RP + g * (RCH / 2)) * 16;
  const int a_t = (4 * (lane >> 5) + ((lane & 15) >> 2)) * LP * 16 +
                  (16 * ((lane >> 4) & 1) + 4 * (lane & 3)) * 2;

  // One 32-token sub-tile: latent rows at sl, RoPE rows at sr, first token tb.
  auto sub_tile = [&](const unsigned char* sl, const unsigned char* sr, int tb) {
    // LDS reads batched ahead of the MFMAs that use them (the score operands
    // first, then the transposed value operands in two halves between the
    // score MFMAs); at most 15 reads outstanding past any wait.
    bf16x8 aR[NR], aL[NL], aT[2][NDT];
    auto read_t = [&](int h2) {
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        const i16x4 lo = pf_read_tr(sl + a_t + (16 * h2) * LP * 16 + dt * 64);
        const i16x4 hi = pf_read_tr(sl + a_t + (16 * h2 + 8) * LP * 16 + dt * 64);
        aT[h2][dt] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      }
    };
#pragma unroll
    for (int st = 0; st < NR; ++st) aR[st] = pf_rd16(sr + a_r + st * 16);
#pragma unroll
    for (int st = 0; st < NL; ++st) aL[st] = pf_rd16(sl + a_l + st * 16);
    __builtin_amdgcn_sched_barrier(0);
    f32x16 sc = f32x16{}, sd = f32x16{};
#pragma unroll
    for (int st = 0; st < NR; ++st) sd = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aR[st], qR[st], sd, 0, 0, 0);
    read_t(0);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int st = 0; st < NL; ++st) {
      if (st % 2 == 0)
        sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aL[st], qL[st], sc, 0, 0, 0);
      else
        sd = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aL[st], qL[st], sd, 0, 0, 0);
    }
    read_t(1);
    __builtin_amdgcn_sched_barrier(0);
    sc += sd;
    if (tb + 32 > wmin) {  // uniform: some row of the wave stops inside this sub-tile
      // element r holds token tb + 4g + 8(r/4) + r%4
      const int lim = vis - tb - 4 * g;
#pragma unroll
      for (int r = 0; r < 16; ++r) sc[r] = 8 * (r >> 2) + (r & 3) < lim ? sc[r] : -INFINITY;
    }
    float mx = -INFINITY;
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sc[r]);
    mx = pf_max_halves(mx) * p.score_scale;
    const bool first = m_run == -INFINITY;
    const bool grow = first ? mx > -INFINITY : mx > m_run + kPfLazyLog2;
    if (__builtin_amdgcn_ballot_w64(grow)) {
      const float alpha = grow ? __builtin_amdgcn_exp2f(m_run - mx) : 1.f;
      m_run = grow ? mx : m_run;
      l_run *= alpha;
      if (__builtin_amdgcn_ballot_w64(grow && !first)) {
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) acc[dt] *= alpha;
      }
    }
    const float m_use = m_run == -INFINITY ? 0.f : m_run;
    bf16x8 pB[2];
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
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
        acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aT[h2][dt], pB[h2], acc[dt], 0, 0, 0);
  };

  if (ntile > 0) {
    // Tile i+1 is in registers while tile i is computed from LDS; it is
    // staged into the other buffer after the compute, and the barrier that
    // follows both publishes it and frees the buffer just computed on.
    issue(0);
    stage(0, smem);
    if (ntile > 1) issue(1);
    pf_lds_barrier();
    for (int i = 0; i < ntile; ++i) {
      const unsigned char* tb_base = smem + (i & 1) * BUF;
      const int t0 = (tile0 + i) * kPfTile;
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        if (t0 + 32 * u >= wmax) break;  // uniform: the wave's rows see no further token
        sub_tile(tb_base + u * 32 * LP * 16, tb_base + LAT + u * 32 * RP * 16, t0 + 32 * u);
      }
      if (i + 1 < ntile) {
        stage(i + 1, smem + ((i + 1) & 1) * BUF);
        if (i + 2 < ntile) issue(i + 2);
      }
      pf_lds_barrier();
    }
  }

  l_run = pf_sum_halves(l_run);
  if (!live) return;
  const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
  const float lse_v = l_run > 0.f ? (m_run + __log2f(l_run)) * kPfLn2 : -INFINITY;
  // O^T element (dt, r) of lane (n, g) is feature dt*32 + 8(r/4) + 4g + r%4 of row n
  if (p.direct) {
    const float f = inv * p.out_rescale;
    __bf16* o = p.out + ((int64_t)(s * (int64_t)p.rows + row) * (p.concat ? p.NB : 1) +
                         (p.concat ? b : 0)) * DC;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        bf16x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = (__bf16)(acc[dt][4 * q + e] * f);
        *reinterpret_cast<bf16x4*>(o + dt * 32 + 8 * q + 4 * g) = v;
      }
    if (g == 0) p.lse[((int64_t)s * p.rows + row) * p.NB + b] = lse_v;
  } else {
    const int64_t ri = (((int64_t)s * p.spl + k) * p.NB + b) * p.rows + row;
    float* o = p.part_o + ri * DC;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        *reinterpret_cast<f32x4*>(o + dt * 32 + 8 * q + 4 * g) =
            f32x4{acc[dt][4 * q], acc[dt][4 * q + 1], acc[dt][4 * q + 2], acc[dt][4 * q + 3]} * inv;
    if (g == 0) p.part_lse[ri] = lse_v;
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

int pf_device_cus(int* out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return -1;
  static int cache[64] = {0};
  if (dev >= 0 && dev < 64 && cache[dev] > 0) {
    *out = cache[dev];
    return 0;
  }
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus < 1)
    return -1;
  if (dev >= 0 && dev < 64) cache[dev] = cus;
  *out = cus;
  return 0;
}

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
  const int64_t tps = pf_cdiv(max_tiles, std::min<int64_t>(want, max_tiles));
  const int64_t spl = pf_cdiv(max_tiles, tps);
  if (base * spl > INT32_MAX) return MLRA_ERR_UNSUPPORTED;
  const bool dir = spl == 1 && (r.NB == 1 || r.reduce == MLRA_BRANCH_CONCAT);
  mlra_decode_plan p;
  std::memset(&p, 0, sizeof(p));
  p.num_cus = num_cus;
  p.target_groups = (int32_t)(base * spl);
  p.waves_per_group = kPfWaves;
  p.tiles_per_split = (int32_t)tps;
  p.splits_per_seq = (int32_t)spl;
  p.kernel_variant = kVariantPrefillBf16;
  p.lds_bytes = r.DC == 128 ? (r.DR == 64 ? PfLayout<128, 64>::LDS : PfLayout<128, 32>::LDS)
                            : (r.DR == 64 ? PfLayout<64, 64>::LDS : PfLayout<64, 32>::LDS);
  p.row_groups = (int32_t)RT;
  if (!dir) {
    const int64_t slots = (int64_t)r.S * spl * r.NB * r.rows;
    p.workspace_bytes = (size_t)(pf_cdiv(slots * r.DC * 4, 256) * 256 + pf_cdiv(slots * 4, 256) * 256);
  }
  *plan = p;
  *direct = dir;
  return MLRA_OK;
}

template <int DC, int DR>
hipError_t launch_prefill(const PrefillParams& pp, int64_t groups, hipStream_t st) {
  constexpr uint32_t lds = PfLayout<DC, DR>::LDS;
  hipLaunchKernelGGL((mlra_prefill<DC, DR>), dim3((uint32_t)groups), dim3(kPfThreads), lds, st, pp);
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
  pp.part_o = direct ? nullptr : static_cast<float*>(workspace);
  pp.part_lse = direct ? nullptr
                       : reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                                  pf_cdiv(slots * r.DC * 4, 256) * 256);
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
