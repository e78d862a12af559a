"""Seeded synthetic inputs for MLRA decode attention.

This module only draws and lays out numbers; it computes nothing of the
attention method. Both the HIP path and the CPU oracle take their inputs from
here, so the two sides see bit-identical values.

Recipe (one ``numpy.random.default_rng(seed)`` stream, draws in this order):
  1. ragged context lengths, U{lo..hi} inclusive (ragged workloads only);
  2. a permutation of the physical cache blocks ("shuffled" placement) or the
     identity ("identity" placement, i.e. a contiguous cache);
  3. latent cache, N(0, 1), shape [num_blocks][block][n_branch][d_latent];
  4. RoPE key cache, N(0, 1), shape [num_blocks][block][d_rope];
  5. latent queries, N(0, 1), shape [S][Q][H][n_branch][d_latent];
  6. RoPE queries, N(0, 1), shape [S][Q][H][d_rope];
  7. outlier mask (latent elements, Bernoulli(outlier_frac)), applied as x*scale.
All draws are float32; bf16 workloads then round every value to bf16 with
round-to-nearest-even, so the float32 arrays returned hold bf16-exact values.

Poison: cache rows past a sequence's length in its last block, and one spare
physical block that every unused block-table entry points to, are NaN. A
kernel that reads them into its arithmetic produces NaN and fails parity.
"""
from __future__ import annotations

import dataclasses
from typing import Dict

import numpy as np

from .configs import DecodeConfig


@dataclasses.dataclass
class DecodeInputs:
    cfg: DecodeConfig
    seq_lens: np.ndarray       # [S] int32, tokens in cache incl. the Q new ones
    block_table: np.ndarray    # [S][max_blocks_per_seq] int32
    latent_cache: np.ndarray   # [num_blocks][BS][NB][DC] float32 (dtype-exact)
    rope_cache: np.ndarray     # [num_blocks][BS][DR] float32 (dtype-exact)
    q_latent: np.ndarray       # [S][Q][H][NB][DC] float32 (dtype-exact)
    q_rope: np.ndarray         # [S][Q][H][DR] float32 (dtype-exact)
    poison_block: int          # physical block that unused table entries name

    @property
    def max_seq_len(self) -> int:
        return int(self.seq_lens.max()) if self.seq_lens.size else 0

    @property
    def num_blocks(self) -> int:
        return int(self.latent_cache.shape[0])


def round_to_bf16(x: np.ndarray, chunk: int = 1 << 24) -> np.ndarray:
    """Round float32 values to the nearest bf16 (ties to even), in place.

    Returns the same array (float32 dtype, bf16-exact values). Inputs are
    finite draws, so no NaN/Inf handling is needed.
    """
    assert x.dtype == np.float32
    flat = x.reshape(-1)
    u = flat.view(np.uint32)
    for lo in range(0, u.size, chunk):
        v = u[lo:lo + chunk]
        bias = ((v >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
        v += bias
        v &= np.uint32(0xFFFF0000)
    return x


def make_inputs(cfg: DecodeConfig, seed: int | None = None) -> DecodeInputs:
    rng = np.random.default_rng(cfg.seed if seed is None else seed)
    S, Q, H, NB = cfg.num_seqs, cfg.q_len, cfg.num_heads, cfg.n_branch
    DC, DR, BS = cfg.d_latent, cfg.d_rope, cfg.block_size

    # 1. context lengths
    if cfg.context_range is not None:
        lo, hi = cfg.context_range
        seq_lens = rng.integers(lo, hi + 1, size=S).astype(np.int32)
    else:
        seq_lens = np.full(S, int(cfg.context), dtype=np.int32)

    nblk = (seq_lens.astype(np.int64) + BS - 1) // BS
    max_blocks = max(int(nblk.max()) if S else 0, 1)
    num_blocks = int(nblk.sum()) + 1  # + the NaN poison block

    # 2. physical placement
    if cfg.placement == "identity":
        perm = np.arange(num_blocks, dtype=np.int64)
    elif cfg.placement == "shuffled":
        perm = rng.permutation(num_blocks)
    else:
        raise ValueError(f"unknown placement {cfg.placement!r}")
    poison_block = int(perm[-1])
    block_table = np.full((S, max_blocks), poison_block, dtype=np.int32)
    off = 0
    for s in range(S):
        n = int(nblk[s])
        block_table[s, :n] = perm[off:off + n]
        off += n

    # 3-6. values
    latent = rng.standard_normal((num_blocks, BS, NB, DC), dtype=np.float32)
    rope = rng.standard_normal((num_blocks, BS, DR), dtype=np.float32)
    q_latent = rng.standard_normal((S, Q, H, NB, DC), dtype=np.float32)
    q_rope = rng.standard_normal((S, Q, H, DR), dtype=np.float32)

    # 7. outliers (latent only)
    if cfg.outlier_frac > 0.0:
        for blk in range(0, num_blocks, 256):  # chunked to bound memory
            sl = latent[blk:blk + 256]
            mask = rng.random(sl.shape, dtype=np.float32) < cfg.outlier_frac
            sl[mask] *= np.float32(cfg.outlier_scale)

    if cfg.dtype == "bf16":
        for a in (latent, rope, q_latent, q_rope):
            round_to_bf16(a)
    elif cfg.dtype != "fp32":
        raise ValueError(f"unknown dtype {cfg.dtype!r}")

    # poison: rows past each sequence's end in its last block, and the spare block
    latent[poison_block] = np.nan
    rope[poison_block] = np.nan
    for s in range(S):
        L = int(seq_lens[s])
        if L % BS and L > 0:
            last = block_table[s, (L - 1) // BS]
            latent[last, L % BS:] = np.nan
            rope[last, L % BS:] = np.nan

    return DecodeInputs(cfg=cfg, seq_lens=seq_lens, block_table=block_table,
                        latent_cache=latent, rope_cache=rope, q_latent=q_latent,
                        q_rope=q_rope, poison_block=poison_block)


def make_append_inputs(cfg: DecodeConfig, seed: int | None = None):
    """New tokens for a cache append: projected branch latents [S][Q][NB][DC]
    and position keys [S][Q][DR], N(0, 1) float32 (the projection's output,
    not rounded), from their own stream (seed + 1000003), so the decode inputs
    of the same config are unchanged."""
    rng = np.random.default_rng((cfg.seed if seed is None else seed) + 1_000_003)
    S, Q = cfg.num_seqs, cfg.q_len
    lat = rng.standard_normal((S, Q, cfg.n_branch, cfg.d_latent), dtype=np.float32)
    rope = rng.standard_normal((S, Q, cfg.d_rope), dtype=np.float32)
    return lat, rope


def make_out_proj_inputs(m: int, k: int, d: int, seed: int):
    """Operands of the output projection: x [m][k] N(0, 1) and an absorbed
    weight w [d][k] N(0, 1/k), both rounded to bf16 (float32 arrays holding
    bf16-exact values)."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((m, k), dtype=np.float32)
    w = rng.standard_normal((d, k), dtype=np.float32) * np.float32(1.0 / np.sqrt(k))
    return round_to_bf16(x), round_to_bf16(w)


def to_device(inp: DecodeInputs, device="cuda") -> Dict[str, "object"]:
    """Copy the inputs to the device as torch tensors of the workload dtype."""
    import torch

    dt = torch.bfloat16 if inp.cfg.dtype == "bf16" else torch.float32

    def t(a):
        return torch.from_numpy(np.ascontiguousarray(a)).to(device).to(dt)

    return dict(
        q_latent=t(inp.q_latent), q_rope=t(inp.q_rope),
        latent_cache=t(inp.latent_cache), rope_cache=t(inp.rope_cache),
        block_table=torch.from_numpy(inp.block_table).to(device),
        seq_lens=torch.from_numpy(inp.seq_lens).to(device),
    )
