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
// the split kernel streams each cache byte exactly once:
//   * one workgroup per (sequence, split); a split is a run of 64-token tiles
//     (one cache block each); waves of the workgroup take a branch (NB), a
//     slice of the latent width (WD) and/or an interleaved share of the tiles
//     (WT);
//   * a wave loads 32-token sub-tiles with 16-byte loads straight into the A
//     operand of v_mfma_f32_32x32x16_bf16: lane (m, g) holds 8 consecutive
//     features of token m, so S^T = C . Q^T needs no shuffles;
//   * the score tile lands with the query row along the lanes, so the online
//     softmax is lane-local plus one v_permlane32_swap for the row max, and
//     the probabilities are already in B-operand order for O^T += C^T . P^T;
//   * C^T (tokens along K) is read back from a wave-private LDS copy of the
//     sub-tile written row-major with 16-byte stores;
//   * each (split, branch, row) writes a partial (output / l, lse); the combine
//     kernel merges the splits with the log-sum-exp rule, sums the branches
//     (or lays them side by side) and applies the output factor.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <cmath>

#include "mlra_internal.h"

namespace mlra {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.69314718055994531f;

struct SplitParams {
  const void* q_lat;
  const void* q_rope;
  const void* lat;
  const void* rope;
  const int32_t* table;
  const int32_t* seq_lens;
  float* part_o;    // [S][spl][NB][rows][DC]
  float* part_lse;  // [S][spl][NB][rows]
  int64_t lsb, lst, lsbr, rsb, rst;
  int32_t S, Q, H, rows, NB, DC, DR, spl, tps, max_blocks, num_blocks, lcap, causal;
  float score_scale;  // scale * log2(e): scores kept in base-2 units
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

__device__ __forceinline__ u32x4 ld16(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

// ---------------------------------------------------------------------------
// bf16 split kernel (MFMA)
// ---------------------------------------------------------------------------
template <int NL, int NR>
struct SubTile {
  u32x4 l[NL];  // latent: NL chunks of 8 bf16 (k-steps of S^T)
  u32x4 r[NR];  // RoPE key: NR chunks of 8 bf16
};

template <int NB, int DCW, int WD, int DR, int NT, int WT, int NPF>
__global__ void __launch_bounds__(64 * NB * WD * WT)
mlra_split_mfma(SplitParams p) {
  constexpr int DC = DCW * WD;
  constexpr int DRW = DR / WD;
  constexpr int NL = DCW / 16;
  constexpr int NR = DRW / 16;
  constexpr int NDT = DCW / 32;
  constexpr int LDW = DCW + kLdsPad;
  static_assert(NR >= 1 && NL >= 1 && NDT >= 1, "bad shape");
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int wd = wave % WD;
  const int b = (wave / WD) % NB;
  const int wt = wave / (WD * NB);
  const int n = lane & 31;
  const int g = lane >> 5;

  const int k = blockIdx.x;
  const int s = blockIdx.y;
  const int L = seq_len_of(p.seq_lens, s, p.lcap);
  const int ntiles = (L + kBlock - 1) / kBlock;
  const int t0 = k * p.tps;
  if (t0 >= ntiles) return;  // uniform over the workgroup: no barrier skipped
  const int t1 = min(t0 + p.tps, ntiles);

  const __bf16* __restrict__ qlat = static_cast<const __bf16*>(p.q_lat);
  const __bf16* __restrict__ qrop = static_cast<const __bf16*>(p.q_rope);
  const __bf16* __restrict__ lat = static_cast<const __bf16*>(p.lat);
  const __bf16* __restrict__ rope = static_cast<const __bf16*>(p.rope);

  // Query rows as the B operand of S^T = C . Q^T (zero for padding rows).
  bf16x8 qL[NT][NL], qR[NT][NR];
  int vis[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int row = nt * 32 + n;
    const bool ok = row < p.rows;
    const int j = ok ? row / p.H : 0;
    const int h = ok ? row % p.H : 0;
    vis[nt] = p.causal ? L - (p.Q - 1 - j) : L;
    const int64_t qb = ((((int64_t)s * p.Q + j) * p.H + h) * NB + b) * DC + wd * DCW + g * (DCW / 2);
    const int64_t rb = (((int64_t)s * p.Q + j) * p.H + h) * DR + wd * DRW + g * (DRW / 2);
#pragma unroll
    for (int st = 0; st < NL; ++st)
      qL[nt][st] = ok ? __builtin_bit_cast(bf16x8, ld16(qlat + qb + 8 * st)) : bf16x8{};
#pragma unroll
    for (int st = 0; st < NR; ++st)
      qR[nt][st] = ok ? __builtin_bit_cast(bf16x8, ld16(qrop + rb + 8 * st)) : bf16x8{};
  }

  f32x16 acc[NT][NDT];
  float m_run[NT], l_run[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    m_run[nt] = -INFINITY;
    l_run[nt] = 0.f;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) acc[nt][dt] = f32x16{};
  }

  // This wave's tiles: t0 + wt + WT*i for i < my_tiles (uniform across the
  // workgroup up to masking), two 32-token sub-tiles each.
  const int nu = 2 * ((t1 - t0 + WT - 1) / WT);
  const int nup = (nu + NPF - 1) / NPF * NPF;
  const int64_t tab_base = (int64_t)s * p.max_blocks;
  int tab = 0, tab_chunk = -1;

  __bf16* tile_lds = reinterpret_cast<__bf16*>(smem) + wave * (kSub * LDW);
  float* xchg = reinterpret_cast<float*>(smem + NB * WD * WT * kSub * LDW * 2);

  auto load = [&](int u, SubTile<NL, NR>& bf) {
    const int i = u >> 1;
    const int ti = t0 + wt + WT * i;
    const bool valid = (u < nu) && ti < t1;
    const int c = i >> 6;
    if (c != tab_chunk) {  // uniform: refresh 64 block ids at once
      const int tj = t0 + wt + WT * (c * 64 + lane);
      tab = tj < t1 ? p.table[tab_base + tj] : 0;
      tab_chunk = c;
    }
    const int phys = clamp_block(__builtin_amdgcn_readlane(tab, i & 63), p.num_blocks);
    const int slot = (u & 1) * kSub + n;
    const bool pred = valid && (ti * kBlock + slot) < L;
    const __bf16* lp = lat + (int64_t)phys * p.lsb + (int64_t)slot * p.lst +
                       (int64_t)b * p.lsbr + wd * DCW + g * (DCW / 2);
    const __bf16* rp = rope + (int64_t)phys * p.rsb + (int64_t)slot * p.rst + wd * DRW +
                       g * (DRW / 2);
    if (pred) {
#pragma unroll
      for (int st = 0; st < NL; ++st) bf.l[st] = ld16(lp + 8 * st);
#pragma unroll
      for (int st = 0; st < NR; ++st) bf.r[st] = ld16(rp + 8 * st);
    } else {
#pragma unroll
      for (int st = 0; st < NL; ++st) bf.l[st] = u32x4{};
#pragma unroll
      for (int st = 0; st < NR; ++st) bf.r[st] = u32x4{};
    }
  };

  auto compute = [&](int u, const SubTile<NL, NR>& bf) {
    const int i = u >> 1;
    const int ti = t0 + wt + WT * i;
    const bool valid = (u < nu) && ti < t1;
    const int tb = ti * kBlock + (u & 1) * kSub;

    // scores S^T[token][row], fp32 accumulate
    f32x16 sc[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      sc[nt] = f32x16{};
#pragma unroll
      for (int st = 0; st < NL; ++st)
        sc[nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, bf.l[st]),
                                                         qL[nt][st], sc[nt], 0, 0, 0);
#pragma unroll
      for (int st = 0; st < NR; ++st)
        sc[nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, bf.r[st]),
                                                         qR[nt][st], sc[nt], 0, 0, 0);
    }

    if constexpr (WD > 1) {
      // Sum the WD partial score tiles (each wave holds a slice of the
      // latent width) in a fixed order so every wave gets identical scores.
      const int grp = wt * NB + b;
      f32x4* X = reinterpret_cast<f32x4*>(xchg) + (u & 1) * (NB * WT * WD * NT * 4 * 64);
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int q = 0; q < 4; ++q)
          X[(((grp * WD + wd) * NT + nt) * 4 + q) * 64 + lane] =
              f32x4{sc[nt][4 * q], sc[nt][4 * q + 1], sc[nt][4 * q + 2], sc[nt][4 * q + 3]};
      __syncthreads();
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          f32x4 t = X[(((grp * WD + 0) * NT + nt) * 4 + q) * 64 + lane];
#pragma unroll
          for (int w = 1; w < WD; ++w) t += X[(((grp * WD + w) * NT + nt) * 4 + q) * 64 + lane];
          sc[nt][4 * q] = t[0];
          sc[nt][4 * q + 1] = t[1];
          sc[nt][4 * q + 2] = t[2];
          sc[nt][4 * q + 3] = t[3];
        }
    }

    // wave-private LDS copy of the latent sub-tile, row-major [32][LDW]
#pragma unroll
    for (int st = 0; st < NL; ++st)
      *reinterpret_cast<u32x4*>(tile_lds + n * LDW + g * (DCW / 2) + 8 * st) = bf.l[st];

    // online softmax per query row (row = lane column of the MFMA tile)
    bf16x8 pB[NT][2];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const int lim = valid ? vis[nt] : 0;
      float x[16];
      float mx = -INFINITY;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int tok = tb + 8 * (r >> 2) + 4 * g + (r & 3);
        x[r] = tok < lim ? sc[nt][r] * p.score_scale : -INFINITY;
        mx = fmaxf(mx, x[r]);
      }
      mx = wave_max_halves(mx);
      const float m_new = fmaxf(m_run[nt], mx);
      const float m_use = m_new == -INFINITY ? 0.f : m_new;
      const float alpha = __builtin_amdgcn_exp2f(m_run[nt] - m_use);
      float sum = 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        x[r] = __builtin_amdgcn_exp2f(x[r] - m_use);
        sum += x[r];
      }
      l_run[nt] = l_run[nt] * alpha + sum;
      m_run[nt] = m_new;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) acc[nt][dt] *= alpha;
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
        for (int e = 0; e < 8; ++e) pB[nt][h2][e] = (__bf16)x[8 * h2 + e];
    }

    // O^T[d][row] += C^T[d][t] . P^T[t][row]; K-slot e of lane group g in
    // half h2 is token 16*h2 + 8*(e/4) + 4*g + e%4, matching P's registers.
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        bf16x8 a;
        const __bf16* col = tile_lds + dt * 32 + n;
#pragma unroll
        for (int e = 0; e < 8; ++e)
          a[e] = col[(16 * h2 + 8 * (e >> 2) + 4 * g + (e & 3)) * LDW];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
          acc[nt][dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pB[nt][h2], acc[nt][dt], 0, 0, 0);
      }
    }
  };

  SubTile<NL, NR> buf[NPF];
#pragma unroll
  for (int i = 0; i < NPF; ++i) load(i, buf[i]);
  for (int u0 = 0; u0 < nup; u0 += NPF) {
#pragma unroll
    for (int i = 0; i < NPF; ++i) {
      compute(u0 + i, buf[i]);
      if (u0 + i + NPF < nup) load(u0 + i + NPF, buf[i]);
    }
  }

#pragma unroll
  for (int nt = 0; nt < NT; ++nt) l_run[nt] = wave_sum_halves(l_run[nt]);

  if constexpr (WT > 1) {
    // Merge the WT token-split waves of each (branch, width slice) in LDS.
    constexpr int REC = NT * NDT * 4 + 1;  // float4 records per lane
    __syncthreads();
    f32x4* M = reinterpret_cast<f32x4*>(smem);
    const int gi = b * WD + wd;
    if (wt > 0) {
      f32x4* my = M + ((wt - 1) * NB * WD + gi) * REC * 64;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
          for (int q = 0; q < 4; ++q)
            my[((nt * NDT + dt) * 4 + q) * 64 + lane] =
                f32x4{acc[nt][dt][4 * q], acc[nt][dt][4 * q + 1], acc[nt][dt][4 * q + 2],
                      acc[nt][dt][4 * q + 3]};
      my[(REC - 1) * 64 + lane] = f32x4{m_run[0], l_run[0], NT > 1 ? m_run[NT - 1] : 0.f,
                                        NT > 1 ? l_run[NT - 1] : 0.f};
    }
    __syncthreads();
    if (wt > 0) return;
#pragma unroll 1
    for (int w = 1; w < WT; ++w) {
      const f32x4* ot = M + ((w - 1) * NB * WD + gi) * REC * 64;
      const f32x4 ml = ot[(REC - 1) * 64 + lane];
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const float mw = nt == 0 ? ml[0] : ml[2];
        const float lw = nt == 0 ? ml[1] : ml[3];
        const float m_new = fmaxf(m_run[nt], mw);
        const float m_use = m_new == -INFINITY ? 0.f : m_new;
        const float a0 = __builtin_amdgcn_exp2f(m_run[nt] - m_use);
        const float a1 = __builtin_amdgcn_exp2f(mw - m_use);
        l_run[nt] = l_run[nt] * a0 + lw * a1;
        m_run[nt] = m_new;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const f32x4 v = ot[((nt * NDT + dt) * 4 + q) * 64 + lane];
#pragma unroll
            for (int e = 0; e < 4; ++e)
              acc[nt][dt][4 * q + e] = acc[nt][dt][4 * q + e] * a0 + v[e] * a1;
          }
      }
    }
  }

  // Partial (output / l, lse) of this split for each (branch, row).
  const int64_t slot = (int64_t)s * p.spl + k;
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int row = nt * 32 + n;
    if (row >= p.rows) continue;
    const float l = l_run[nt];
    const float inv = l > 0.f ? 1.f / l : 0.f;
    const int64_t ri = (slot * NB + b) * p.rows + row;
    float* o = p.part_o + ri * DC + wd * DCW;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        *reinterpret_cast<f32x4*>(o + dt * 32 + 8 * q + 4 * g) =
            f32x4{acc[nt][dt][4 * q], acc[nt][dt][4 * q + 1], acc[nt][dt][4 * q + 2],
                  acc[nt][dt][4 * q + 3]} * inv;
    if (g == 0 && wd == 0)
      p.part_lse[ri] = l > 0.f ? (m_run[nt] + __log2f(l)) * kLn2 : -INFINITY;
  }
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
  for (int t = t0 * kBlock; t < tend; ++t) {
    const int phys = clamp_block(p.table[(int64_t)s * p.max_blocks + t / kBlock], p.num_blocks);
    const int slot = t % kBlock;
    const float* cp = lat + (int64_t)phys * p.lsb + (int64_t)slot * p.lst + (int64_t)b * p.lsbr;
    float c[NDC];
    float dot = 0.f;
#pragma unroll
    for (int i = 0; i < NDC; ++i) {
      c[i] = cp[lane + 64 * i];
      dot = fmaf(q[i], c[i], dot);
    }
    if (lane < p.DR) dot = fmaf(qr, rope[(int64_t)phys * p.rsb + (int64_t)slot * p.rst + lane], dot);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) dot += __shfl_xor(dot, off);
    // one value for the whole wave (the butterfly's rounding differs per lane)
    const float x = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(dot))) *
                    p.score_scale;
    const float m_new = fmaxf(m, x);
    const float alpha = __builtin_amdgcn_exp2f(m - m_new);
    const float w = __builtin_amdgcn_exp2f(x - m_new);
    l = l * alpha + w;
#pragma unroll
    for (int i = 0; i < NDC; ++i) acc[i] = acc[i] * alpha + w * c[i];
    m = m_new;
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
template <typename OutT>
__device__ __forceinline__ void store4(OutT* dst, f32x4 v);

template <>
__device__ __forceinline__ void store4<float>(float* dst, f32x4 v) {
  *reinterpret_cast<f32x4*>(dst) = v;
}

template <>
__device__ __forceinline__ void store4<__bf16>(__bf16* dst, f32x4 v) {
  typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
  bf16x4 o = {(__bf16)v[0], (__bf16)v[1], (__bf16)v[2], (__bf16)v[3]};
  *reinterpret_cast<bf16x4*>(dst) = o;
}

template <typename OutT>
__global__ void __launch_bounds__(256) mlra_combine(CombineParams c) {
  const int tpr = c.DC / 4;
  const int row = blockIdx.x * (256 / tpr) + threadIdx.x / tpr;
  const int d4 = threadIdx.x % tpr;
  const int s = blockIdx.y;
  if (row >= c.rows) return;
  const int L = seq_len_of(c.seq_lens, s, c.lcap);
  const int ntiles = (L + kBlock - 1) / kBlock;
  const int nsplit = min((ntiles + c.tps - 1) / c.tps, c.spl);
  const int j = row / c.H, h = row % c.H;
  const int64_t orow = ((int64_t)s * c.Q + j) * c.H + h;
  OutT* out = static_cast<OutT*>(c.out);
  f32x4 tot = {};
  for (int b = 0; b < c.NB; ++b) {
    float M = -INFINITY;
    for (int k = 0; k < nsplit; ++k)
      M = fmaxf(M, c.part_lse[(((int64_t)s * c.spl + k) * c.NB + b) * c.rows + row]);
    f32x4 o = {};
    float lse_b = -INFINITY;
    if (M != -INFINITY) {
      float den = 0.f;
      for (int k = 0; k < nsplit; ++k) {
        const int64_t ri = (((int64_t)s * c.spl + k) * c.NB + b) * c.rows + row;
        const float w = expf(c.part_lse[ri] - M);
        den += w;
        o += w * *reinterpret_cast<const f32x4*>(c.part_o + ri * c.DC + 4 * d4);
      }
      o *= 1.f / den;
      lse_b = M + logf(den);
    }
    if (c.concat)
      store4<OutT>(out + (orow * c.NB + b) * c.DC + 4 * d4, o * c.out_rescale);
    else
      tot += o;
    if (d4 == 0) c.lse[orow * c.NB + b] = lse_b;
  }
  if (!c.concat) store4<OutT>(out + orow * c.DC + 4 * d4, tot * c.out_rescale);
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
template <int NB, int DC, int DR, int NT>
static hipError_t launch_mfma(const SplitParams& sp, const mlra_decode_plan& plan,
                              hipStream_t stream) {
  constexpr int WD = DC == 512 ? 4 : 1;
  constexpr int DCW = DC / WD;
  constexpr int WT = (NB == 1 && WD == 1) ? 4 : (NB == 2 ? 2 : 1);
  constexpr int NPF = 2;
  auto kern = mlra_split_mfma<NB, DCW, WD, DR, NT, WT, NPF>;
  const int lds = mfma_lds_bytes(NB, DCW, WD, NT, WT);
  if (lds > 64 * 1024) {
    static bool attr_set = false;  // per instance; benign race (idempotent call)
    if (!attr_set) {
      hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                         hipFuncAttributeMaxDynamicSharedMemorySize, lds);
      if (e != hipSuccess) return e;
      attr_set = true;
    }
  }
  dim3 grid(plan.splits_per_seq, sp.S);
  hipLaunchKernelGGL(kern, grid, dim3(64 * NB * WD * WT), lds, stream, sp);
  return hipGetLastError();
}

template <int NB, int DC, int NT>
static hipError_t dispatch_dr(const SplitParams& sp, const mlra_decode_plan& plan,
                              hipStream_t st) {
  if (sp.DR == 64) return launch_mfma<NB, DC, 64, NT>(sp, plan, st);
  if constexpr (DC != 512) return launch_mfma<NB, DC, 32, NT>(sp, plan, st);
  return hipErrorInvalidValue;
}

template <int NB, int NT>
static hipError_t dispatch_dc(const SplitParams& sp, const mlra_decode_plan& plan,
                              hipStream_t st) {
  switch (sp.DC) {
    case 64: return dispatch_dr<NB, 64, NT>(sp, plan, st);
    case 128: return dispatch_dr<NB, 128, NT>(sp, plan, st);
    case 512:
      if constexpr (NB == 1) return dispatch_dr<NB, 512, NT>(sp, plan, st);
      return hipErrorInvalidValue;
  }
  return hipErrorInvalidValue;
}

template <int NT>
static hipError_t dispatch_nb(const SplitParams& sp, const mlra_decode_plan& plan,
                              hipStream_t st) {
  switch (sp.NB) {
    case 1: return dispatch_dc<1, NT>(sp, plan, st);
    case 2: return dispatch_dc<2, NT>(sp, plan, st);
    case 4: return dispatch_dc<4, NT>(sp, plan, st);
  }
  return hipErrorInvalidValue;
}

static hipError_t launch_split(const SplitParams& sp, const KernelShape& ks,
                               const mlra_decode_plan& plan, hipStream_t st) {
  if (ks.variant == kVariantMfmaBf16)
    return ks.NT == 1 ? dispatch_nb<1>(sp, plan, st) : dispatch_nb<2>(sp, plan, st);
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

static int device_cus(int* out) {
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

static bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

static mlra_status decode(const void* q_latent, const void* q_rope, const void* latent_cache,
                          const void* rope_cache, const int32_t* block_table,
                          const int32_t* seq_lens, int32_t n_branch, float scale,
                          float out_rescale, void* out, float* lse, const mlra_decode_dims* dims,
                          void* workspace, size_t workspace_bytes, void* stream) {
  Resolved r;
  mlra_status st = resolve_dims(dims, n_branch, &r);
  if (st != MLRA_OK) return st;
  if (!q_latent || !q_rope || !latent_cache || !rope_cache || !block_table || !seq_lens ||
      !out || !lse)
    return MLRA_ERR_NULL_PTR;
  if (!std::isfinite(scale) || !std::isfinite(out_rescale)) return MLRA_ERR_BAD_DIMS;
  if (!aligned16(q_latent) || !aligned16(q_rope) || !aligned16(latent_cache) ||
      !aligned16(rope_cache) || !aligned16(out) || !aligned16(workspace) ||
      (reinterpret_cast<uintptr_t>(lse) & 3) || (reinterpret_cast<uintptr_t>(block_table) & 3) ||
      (reinterpret_cast<uintptr_t>(seq_lens) & 3))
    return MLRA_ERR_ALIGNMENT;
  const KernelShape ks = choose_shape(r);
  int cus = 0;
  if (device_cus(&cus) != 0) return MLRA_ERR_HIP;
  mlra_decode_plan plan;
  st = plan_call(r, ks, cus, dims->num_splits, dims->sum_seq_lens, &plan);
  if (st != MLRA_OK) return st;
  if (!workspace || workspace_bytes < plan.workspace_bytes) return MLRA_ERR_WORKSPACE;

  const int64_t slots = (int64_t)r.S * plan.splits_per_seq * r.NB * r.rows;
  float* part_o = static_cast<float*>(workspace);
  float* part_lse = reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                             ((slots * r.DC * 4 + 255) / 256) * 256);
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
  sp.score_scale = scale * kLog2e;
  hipStream_t hs = static_cast<hipStream_t>(stream);
  if (launch_split(sp, ks, plan, hs) != hipSuccess) return MLRA_ERR_HIP;

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
  const int rpb = 256 / (r.DC / 4);
  dim3 cgrid((r.rows + rpb - 1) / rpb, r.S);
  if (r.dtype == MLRA_BF16)
    hipLaunchKernelGGL(mlra_combine<__bf16>, cgrid, dim3(256), 0, hs, cp);
  else
    hipLaunchKernelGGL(mlra_combine<float>, cgrid, dim3(256), 0, hs, cp);
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
  return mlra::decode(q_latent, q_rope, latent_cache, rope_cache, block_table, seq_lens,
                      n_branch, scale, out_rescale, out, lse, dims, workspace, workspace_bytes,
                      stream);
}

extern "C" mlra_status mla_decode_attention(const void* q_latent, const void* q_rope,
                                            const void* latent_cache, const void* rope_cache,
                                            const int32_t* block_table, const int32_t* seq_lens,
                                            float scale, void* out, float* lse,
                                            const mlra_decode_dims* dims, void* workspace,
                                            size_t workspace_bytes, void* stream) {
  return mlra::decode(q_latent, q_rope, latent_cache, rope_cache, block_table, seq_lens, 1,
                      scale, 1.0f, out, lse, dims, workspace, workspace_bytes, stream);
}
