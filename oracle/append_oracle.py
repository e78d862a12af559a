"""Float64 CPU oracle for appending new tokens to the paged MLRA latent cache.

TEST INFRASTRUCTURE ONLY. Imported by ``tests/`` and the CPU-baseline leg of
``bench.py``; never by the product path.

What is appended, from the pages (cited by title and section):
  [BLOG]  wispaper.ai, "MLRA: Breaking the Sharding Bottleneck in Latent
          Attention" -- "The Core Insight: Sum of Branches, Not Sum of Keys":
          per token the cache holds one latent per branch and one decoupled
          position (RoPE) key shared by all branches; "Mathematical
          Calibration: Scaling the Latents": the latent states are multiplied
          by a fixed calibration factor (its formula is lost in the page text,
          so it is a caller argument here).
  [HN]    Hacker News thread on TransMLA: only the compressed latent (plus the
          decoupled position key) is cached, never full keys or values.

Readings taken where the pages are silent (each is listed in the design doc):
  * the new tokens arrive already down-projected (the dense projection is an
    ordinary GEMM upstream); the append multiplies the latents by the
    calibration factor and rotates the position key;
  * the rotation is the rotary position embedding of Su et al. (RoFormer):
    adjacent pairs (2i, 2i+1) turn by the angle p * base**(-2i/DR), base
    10000 by default;
  * seq_lens counts the new tokens, so token j of Q sits at position
    p = L - Q + j; positions below 0, past the block table, or whose block id
    lies outside the cache are not written;
  * bfloat16 caches hold the exact value rounded to nearest, ties to even.

Parity pins (tests/test_oracle_append.py):
  rope_rotate        -- hand-derived golden example (literal cosines and sines
                        of the angles); position 0 is the identity; pair norms
                        kept; rotations compose; scores depend only on the
                        position difference.
  round_to_bf16_f64  -- exact bf16 values unchanged; ties to even; agrees with
                        the seeded generator's float32 rounding on float32
                        inputs.
  cache_append       -- hand-derived golden example (whole cache before and
                        after); brute-force gather of every sequence after the
                        append; block-permutation invariance; skipped writes.
No function here is parity-unpinned.
"""
from __future__ import annotations

import numpy as np


def rope_rotate(x, pos, base: float = 10000.0) -> np.ndarray:
    """Rotary position embedding of a decoupled key at integer positions, float64.

    x [..., DR] (DR even), pos broadcast against x's leading dimensions.
    Pair (x[2i], x[2i+1]) turns by the angle pos * base**(-2i/DR):
        y[2i]   = x[2i] cos a - x[2i+1] sin a
        y[2i+1] = x[2i] sin a + x[2i+1] cos a
    """
    x = np.asarray(x, dtype=np.float64)
    DR = x.shape[-1]
    i = np.arange(DR // 2, dtype=np.float64)
    theta = float(base) ** (-2.0 * i / DR)
    a = np.asarray(pos, dtype=np.float64)[..., None] * theta
    c, s = np.cos(a), np.sin(a)
    xe, xo = x[..., 0::2], x[..., 1::2]
    y = np.empty(np.broadcast_shapes(x.shape, a.shape[:-1] + (DR,)))
    y[..., 0::2] = xe * c - xo * s
    y[..., 1::2] = xe * s + xo * c
    return y


def round_to_bf16_f64(x) -> np.ndarray:
    """Round float64 values to the nearest bfloat16 (8 significant bits), ties to even.

    Returned as float64 holding bf16-exact values. Written for the finite,
    normal-range values of the workloads (no overflow or subnormal handling).
    """
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)                     # x = m * 2**e, 0.5 <= |m| < 1
    return np.ldexp(np.rint(m * 256.0), e - 8)


def cache_append(latent_new, rope_new, latent_cache, rope_cache, block_table, seq_lens,
                 latent_scale: float, rope_base: float = 10000.0, block_size: int = 64,
                 to_bf16: bool = True):
    """Write the Q new tokens of every sequence into copies of the paged caches.

    Shapes: latent_new [S][Q][NB][DC], rope_new [S][Q][DR] (projected, the key
    not yet rotated), latent_cache [blocks][BS][NB][DC], rope_cache
    [blocks][BS][DR], block_table [S][max_blocks], seq_lens [S] (counting the
    new tokens). Token j of sequence s goes to position p = L - Q + j, i.e.
    block block_table[s][p // BS], slot p % BS:
        latent_cache[...] = latent_scale * latent_new[s, j]
        rope_cache[...]   = rope_rotate(rope_new[s, j], p, rope_base)
    Returns (latent_cache', rope_cache') as float64 arrays.
    """
    lat = np.array(latent_cache, dtype=np.float64)
    rope = np.array(rope_cache, dtype=np.float64)
    S, Q = latent_new.shape[:2]
    nblocks, max_blocks = lat.shape[0], block_table.shape[1]
    for s in range(S):
        L = int(seq_lens[s])
        for j in range(Q):
            p = L - Q + j
            if p < 0 or p // block_size >= max_blocks:
                continue
            blk = int(block_table[s, p // block_size])
            if blk < 0 or blk >= nblocks:
                continue
            c = float(latent_scale) * np.asarray(latent_new[s, j], dtype=np.float64)
            k = rope_rotate(rope_new[s, j], p, rope_base)
            if to_bf16:
                c, k = round_to_bf16_f64(c), round_to_bf16_f64(k)
            lat[blk, p % block_size] = c
            rope[blk, p % block_size] = k
    return lat, rope
