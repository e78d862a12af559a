"""Workload shapes for MLRA decode attention over a paged latent KV cache.

Each entry fixes the shapes, dtypes, cache placement and value distribution
of one decode workload. Nothing here computes attention; the shapes follow
the per-device KV load that the wispaper.ai blog "MLRA: Breaking the
Sharding Bottleneck in Latent Attention" describes in "The Core Insight: Sum
of Branches, Not Sum of Keys" (each branch keeps a latent of width dh, one
decoupled position key of width 0.5*dh is shared, so a 4-way tensor-parallel
rank loads 1.5*dh per token while MLA loads 4.5*dh).
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional, Tuple

BLOCK_SIZE = 64  # tokens per physical cache block


@dataclasses.dataclass(frozen=True)
class DecodeConfig:
    name: str
    num_seqs: int            # S: sequences decoded together
    q_len: int               # Q: new query tokens per sequence
    num_heads: int           # H: query heads per branch
    n_branch: int            # NB: latent branches held in the cache
    d_latent: int            # DC: latent width per branch
    d_rope: int              # DR: shared decoupled-RoPE key width
    dtype: str               # "fp32" or "bf16" for q, cache and out
    context: Optional[int]   # fixed context length (tokens in cache, incl. new ones)
    context_range: Optional[Tuple[int, int]] = None  # ragged: inclusive U{lo..hi}
    placement: str = "shuffled"   # "identity" (contiguous) or "shuffled" physical blocks
    causal: bool = True           # with Q > 1: query j sees t < L - (Q - 1 - j)
    outlier_frac: float = 0.0     # fraction of latent elements scaled by outlier_scale
    outlier_scale: float = 1.0
    seed: int = 0
    scale: float = 1.0            # softmax scale on the raw dot products
    out_rescale: float = 1.0      # variance-calibration factor on the attention output
    block_size: int = BLOCK_SIZE

    @property
    def rows(self) -> int:
        return self.num_heads * self.q_len

    def with_(self, **kw) -> "DecodeConfig":
        return dataclasses.replace(self, **kw)


def _mlra_scale(dc: int, dr: int) -> float:
    return 1.0 / math.sqrt(dc + dr)


# Tiny MLRA-4 decode in fp32, contiguous cache (identity block table).
TINY_MLRA4_FP32 = DecodeConfig(
    name="tiny_mlra4_fp32_s1_t256", num_seqs=1, q_len=1, num_heads=8, n_branch=4,
    d_latent=64, d_rope=32, dtype="fp32", context=256, placement="identity",
    seed=0, scale=_mlra_scale(64, 32), out_rescale=1.0 / math.sqrt(4))

# One tensor-parallel rank's share of MLRA-4: a single branch (latent 128) plus
# the shared RoPE key (64), i.e. 1.5*dh per token at dh = 128. The output factor
# stays 1/sqrt(4) so that the four ranks' outputs sum to the fused result.
MLRA4_TP_SHARE = DecodeConfig(
    name="mlra4_tp_share_b16_t8192", num_seqs=16, q_len=1, num_heads=32, n_branch=1,
    d_latent=128, d_rope=64, dtype="bf16", context=8192, seed=2,
    scale=_mlra_scale(128, 64), out_rescale=0.5)

# All four MLRA-4 branches fused on one GPU.
MLRA4_FUSED = DecodeConfig(
    name="mlra4_fused_b32_t16384", num_seqs=32, q_len=1, num_heads=32, n_branch=4,
    d_latent=128, d_rope=64, dtype="bf16", context=16384, seed=3,
    scale=_mlra_scale(128, 64), out_rescale=0.5)

# MLA-shaped comparison on identical token counts: one 512-wide latent + RoPE 64.
MLA_COMPARE = DecodeConfig(
    name="mla_b32_t16384", num_seqs=32, q_len=1, num_heads=32, n_branch=1,
    d_latent=512, d_rope=64, dtype="bf16", context=16384, seed=3,
    scale=_mlra_scale(512, 64), out_rescale=1.0)

# Long-context decode with 1% latent outliers scaled by 8.
LONG_CONTEXT = DecodeConfig(
    name="mlra4_long_b4_t131072", num_seqs=4, q_len=1, num_heads=32, n_branch=4,
    d_latent=128, d_rope=64, dtype="bf16", context=131072, seed=4,
    outlier_frac=0.01, outlier_scale=8.0,
    scale=_mlra_scale(128, 64), out_rescale=0.5)

# Ragged batch, 2 query tokens per sequence, causal among the new tokens.
RAGGED_Q2 = DecodeConfig(
    name="mlra4_ragged_b64_q2", num_seqs=64, q_len=2, num_heads=32, n_branch=4,
    d_latent=128, d_rope=64, dtype="bf16", context=None, context_range=(1024, 32768),
    seed=5, causal=True, scale=_mlra_scale(128, 64), out_rescale=0.5)

# MLRA-2: MLA's 512-wide latent in two branches of 256 plus the shared RoPE
# key; same cache bytes per token as MLRA-4 and MLA. Output factor 1/sqrt(2),
# the two-branch analogue of MLRA-4's 1/sqrt(4).
MLRA2_FUSED = DecodeConfig(
    name="mlra2_fused_b32_t16384", num_seqs=32, q_len=1, num_heads=32, n_branch=2,
    d_latent=256, d_rope=64, dtype="bf16", context=16384, seed=6,
    scale=_mlra_scale(256, 64), out_rescale=1.0 / math.sqrt(2))

# One sequence at 1M and 2M tokens of context (the latency-vs-length sweep's
# long end), all four MLRA-4 branches: split-K planning at extreme lengths.
MLRA4_B1_T1M = DecodeConfig(
    name="mlra4_b1_t1m", num_seqs=1, q_len=1, num_heads=32, n_branch=4,
    d_latent=128, d_rope=64, dtype="bf16", context=1 << 20, seed=7,
    scale=_mlra_scale(128, 64), out_rescale=0.5)
MLRA4_B1_T2M = DecodeConfig(
    name="mlra4_b1_t2m", num_seqs=1, q_len=1, num_heads=32, n_branch=4,
    d_latent=128, d_rope=64, dtype="bf16", context=1 << 21, seed=8,
    scale=_mlra_scale(128, 64), out_rescale=0.5)

# The headline share with four new query tokens per sequence (speculative
# decoding verifying three draft tokens: 128 query rows per sequence).
MLRA4_TP_SHARE_Q4 = MLRA4_TP_SHARE.with_(name="mlra4_tp_share_b16_t8192_q4", q_len=4, seed=13)

# Cache append at a large serving batch: 4096 sequences, 2 new tokens each,
# all four MLRA-4 branches (one head: the append does not read queries).
APPEND_B4096_Q2 = DecodeConfig(
    name="mlra4_append_b4096_q2", num_seqs=4096, q_len=2, num_heads=1, n_branch=4,
    d_latent=128, d_rope=64, dtype="bf16", context=64, seed=9,
    scale=_mlra_scale(128, 64), out_rescale=0.5)

# Chunked prefill on one tensor-parallel rank's share: 4 sequences, each
# adding a chunk of 2048 tokens after 6144 cached ones (8192 in all), causal.
# 65536 query rows (2048 tokens x 32 heads) per sequence share each token's
# latent and RoPE key.
MLRA4_TP_PREFILL = DecodeConfig(
    name="mlra4_tp_share_prefill_b4_c2048_t8192", num_seqs=4, q_len=2048, num_heads=32,
    n_branch=1, d_latent=128, d_rope=64, dtype="bf16", context=8192, seed=10,
    scale=_mlra_scale(128, 64), out_rescale=0.5)
# A whole 16384-token sequence prefilled at once (the chunk is the sequence).
MLRA4_TP_PREFILL_WHOLE = DecodeConfig(
    name="mlra4_tp_share_prefill_b1_t16384", num_seqs=1, q_len=16384, num_heads=32,
    n_branch=1, d_latent=128, d_rope=64, dtype="bf16", context=16384, seed=11,
    scale=_mlra_scale(128, 64), out_rescale=0.5)
# All four MLRA-4 branches, summed: chunks of 512 after ragged contexts.
MLRA4_FUSED_PREFILL = DecodeConfig(
    name="mlra4_fused_prefill_b4_c512", num_seqs=4, q_len=512, num_heads=32, n_branch=4,
    d_latent=128, d_rope=64, dtype="bf16", context=None, context_range=(512, 4096), seed=12,
    scale=_mlra_scale(128, 64), out_rescale=0.5)

ALL = [TINY_MLRA4_FP32, MLRA4_TP_SHARE, MLRA4_FUSED, LONG_CONTEXT, RAGGED_Q2]
# Variants and stress workloads beyond the five above.
EXTRA = [MLRA2_FUSED, MLRA4_B1_T1M, MLRA4_B1_T2M, APPEND_B4096_Q2, MLRA4_TP_SHARE_Q4]
# Chunked-prefill workloads (mlra_prefill_attention).
PREFILL = [MLRA4_TP_PREFILL, MLRA4_TP_PREFILL_WHOLE, MLRA4_FUSED_PREFILL]
BY_NAME = {c.name: c for c in ALL + [MLA_COMPARE] + EXTRA + PREFILL}
