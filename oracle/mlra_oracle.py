"""Float64 CPU oracle for Multi-Head Low-Rank Attention (MLRA) decode.

TEST INFRASTRUCTURE ONLY. Imported by ``tests/``, ``__graft_entry__.smoke()``
and the CPU-baseline leg of ``bench.py``; never by the product path.

Sources (web pages; cited by title and section):
  [BLOG]   wispaper.ai, "MLRA: Breaking the Sharding Bottleneck in Latent
           Attention" -- sections "The Core Insight: Sum of Branches, Not Sum
           of Keys" (per-branch attention, outputs summed afterwards; 1.5*dh
           per-device load vs 4.5*dh for MLA) and "Mathematical Calibration:
           Scaling the Latents" (fixed rescale of the attention output).
  [ABS]    arXiv 2603.02188 "Multi-Head Low-Rank Attention", abstract (decode
           is bound by moving the KV cache from HBM to on-chip memory; MLA's
           single latent head cannot be partitioned).
  [HN]     Hacker News thread on TransMLA (MLA background: only the latent
           is cached, keys/values come from low-rank up-projections).

Notation: S sequences, Q new query tokens per sequence, H heads, NB branches,
DC latent width per branch, DR decoupled-RoPE key width, BS tokens per cache
block. seq_lens[s] = L counts the Q new tokens, already appended to the cache.

Readings taken where the pages are silent (each is listed in the design doc):
  * the decoupled RoPE key and its query are shared by all branches of a head
    (the blog's 1.5*dh per rank = one dh latent + one 0.5*dh shared key);
  * scores are scale * (q_b . c_b[t] + q_r . k_r[t]); lse is the natural log
    of sum_t exp(score), one value per (s, j, h, b);
  * causal among the Q new tokens: query j sees t < L - (Q - 1 - j);
  * a query that sees no token has output 0 and lse = -inf;
  * branch reduce "sum": out = out_rescale * sum_b o_b (branches share the
    value up-projection); "concat": out[..., b, :] = out_rescale * o_b (the
    exact form when each branch has its own value up-projection).

Parity pins (tests/test_oracle.py), per function:
  paged_gather            -- block-permutation invariance; identity table ==
                             contiguous slice.
  mlra_decode             -- brute force (mlra_decode_bruteforce) on tiny
                             shapes; equals the expanded form (mlra_expanded)
                             and torch SDPA on explicit keys/values; closed
                             forms (V=1, zero queries -> mean & ln V, constant
                             latent, V<=0, one dominant token); hand-derived
                             golden example; causal consistency; fused ==
                             sum of single-branch shares; negative control vs
                             MLA-style sum-before-softmax; Gaussian-tilting
                             statistics at full workload size.
                             Prefill regime (tests/test_oracle_prefill.py,
                             many causal query tokens): torch SDPA with its
                             own causal flag (whole-sequence prefill) and with
                             a position mask (a chunk after cached context);
                             chunked prefill == whole prefill; the first
                             token sees only itself; planted visibility
                             mistakes caught.
  mlra_decode_bruteforce  -- hand-derived golden example; closed forms.
  mlra_expanded           -- torch.nn.functional.scaled_dot_product_attention.
  mla_expanded            -- torch SDPA (one softmax over a single latent).
No function here is parity-unpinned.
"""
from __future__ import annotations

import math

import numpy as np


def paged_gather(cache: np.ndarray, table_row: np.ndarray, n_tokens: int,
                 block_size: int) -> np.ndarray:
    """Rows 0..n_tokens-1 of one sequence from a paged cache, as float64.

    Token t lives in physical block table_row[t // block_size] at slot
    t % block_size ([HN]: the cache holds one latent row per token; the
    paging is the block-table layout of the decode workload).
    """
    t = np.arange(n_tokens)
    phys = np.asarray(table_row)[t // block_size]
    return cache[phys, t % block_size].astype(np.float64)


def visible_length(seq_len: int, q_len: int, j: int, causal: bool) -> int:
    """Tokens query j of a sequence may attend to (causal among new tokens)."""
    return int(seq_len) - (q_len - 1 - j) if causal else int(seq_len)


def mlra_decode(q_latent, q_rope, latent_cache, rope_cache, block_table, seq_lens,
                scale, out_rescale, reduce="sum", causal=True, block_size=64):
    """Absorbed-form MLRA decode attention, float64.

    [BLOG] "The Core Insight": each latent branch b runs its own attention and
    the per-branch outputs are summed afterwards (MLA instead sums the branch
    up-projections into one key before a single softmax). With the key
    up-projection absorbed into the query ([HN]: only the latent is cached),
    branch b of head h scores token t as
        z_b[t] = scale * (q_latent[s,j,h,b] . c_b[t] + q_rope[s,j,h] . k_r[t])
    and its latent-space output is o_b = sum_t softmax(z_b)[t] * c_b[t].
    [BLOG] "Mathematical Calibration": the summed output is multiplied by a
    fixed factor (out_rescale).

    Shapes: q_latent [S][Q][H][NB][DC], q_rope [S][Q][H][DR],
    latent_cache [blocks][BS][NB][DC], rope_cache [blocks][BS][DR],
    block_table [S][max_blocks], seq_lens [S].
    Returns (out, lse): out [S][Q][H][DC] ("sum") or [S][Q][H][NB][DC]
    ("concat"); lse [S][Q][H][NB] natural log of sum_t exp(z_b[t]).
    """
    S, Q, H, NB, DC = q_latent.shape
    if reduce == "sum":
        out = np.zeros((S, Q, H, DC))
    elif reduce == "concat":
        out = np.zeros((S, Q, H, NB, DC))
    else:
        raise ValueError(reduce)
    lse = np.full((S, Q, H, NB), -np.inf)
    for s in range(S):
        L = int(seq_lens[s])
        if L <= 0:
            continue
        C = paged_gather(latent_cache, block_table[s], L, block_size)   # [L][NB][DC]
        KR = paged_gather(rope_cache, block_table[s], L, block_size)    # [L][DR]
        for j in range(Q):
            V = visible_length(L, Q, j, causal)
            if V <= 0:
                continue
            qr = np.asarray(q_rope[s, j], dtype=np.float64)              # [H][DR]
            rope_dot = qr @ KR[:V].T                                     # [H][V]
            for b in range(NB):
                qb = np.asarray(q_latent[s, j, :, b], dtype=np.float64)  # [H][DC]
                Cb = C[:V, b]                                            # [V][DC]
                z = scale * (qb @ Cb.T + rope_dot)                       # [H][V]
                m = z.max(axis=1, keepdims=True)
                e = np.exp(z - m)
                tot = e.sum(axis=1, keepdims=True)
                lse[s, j, :, b] = (m + np.log(tot))[:, 0]
                ob = (e / tot) @ Cb                                      # [H][DC]
                if reduce == "sum":
                    out[s, j] += out_rescale * ob
                else:
                    out[s, j, :, b] = out_rescale * ob
    return out, lse


def mlra_decode_bruteforce(q_latent, q_rope, latent_cache, rope_cache, block_table,
                           seq_lens, scale, out_rescale, reduce="sum", causal=True,
                           block_size=64):
    """The same definition as mlra_decode, as pure-Python scalar loops.

    Independent of mlra_decode: no NumPy arithmetic, math.exp / math.log on
    Python floats, softmax taken as exp(z - max) / sum, block lookups written
    inline. For tiny shapes only.
    """
    S, Q, H, NB, DC = np.shape(q_latent)
    DR = np.shape(q_rope)[3]
    qlat = np.asarray(q_latent).tolist()
    qrop = np.asarray(q_rope).tolist()
    lat = latent_cache
    rop = rope_cache
    if reduce == "sum":
        out = [[[[0.0] * DC for _ in range(H)] for _ in range(Q)] for _ in range(S)]
    else:
        out = [[[[[0.0] * DC for _ in range(NB)] for _ in range(H)] for _ in range(Q)]
               for _ in range(S)]
    lse = [[[[float("-inf")] * NB for _ in range(H)] for _ in range(Q)] for _ in range(S)]
    for s in range(S):
        L = int(seq_lens[s])
        for j in range(Q):
            V = L - (Q - 1 - j) if causal else L
            if V <= 0:
                continue
            for h in range(H):
                for b in range(NB):
                    zs = []
                    rows = []
                    for t in range(V):
                        blk = int(block_table[s][t // block_size])
                        slot = t % block_size
                        c = [float(x) for x in lat[blk][slot][b]]
                        kr = [float(x) for x in rop[blk][slot]]
                        dot = 0.0
                        for d in range(DC):
                            dot += float(qlat[s][j][h][b][d]) * c[d]
                        for d in range(DR):
                            dot += float(qrop[s][j][h][d]) * kr[d]
                        zs.append(scale * dot)
                        rows.append(c)
                    zmax = max(zs)
                    ws = [math.exp(z - zmax) for z in zs]
                    tot = sum(ws)
                    lse[s][j][h][b] = zmax + math.log(tot)
                    for d in range(DC):
                        acc = 0.0
                        for t in range(V):
                            acc += ws[t] * rows[t][d]
                        v = out_rescale * acc / tot
                        if reduce == "sum":
                            out[s][j][h][d] += v
                        else:
                            out[s][j][h][b][d] = v
    return np.array(out, dtype=np.float64), np.array(lse, dtype=np.float64)


def _softmax_attend(q, K, Vv, scale):
    """Plain softmax attention of one query over explicit keys and values."""
    z = scale * (K @ q)
    m = z.max()
    e = np.exp(z - m)
    tot = e.sum()
    return (e / tot) @ Vv, m + math.log(tot)


def mlra_expanded(q_nope, q_rope, latent_cache, rope_cache, block_table, seq_lens,
                  w_uk, w_uv, scale, out_rescale, causal=True, block_size=64):
    """MLRA in expanded (non-absorbed) form, float64.

    [BLOG] "The Core Insight": per branch b, materialise keys
        k_b[t] = [W_UK[h,b] c_b[t] ; k_r[t]]   and values  v_b[t] = W_UV[h,b] c_b[t],
    run plain softmax attention of q = [q_nope[s,j,h,b] ; q_rope[s,j,h]] over
    them, and sum the branch outputs afterwards; [BLOG] "Mathematical
    Calibration": multiply the sum by out_rescale.

    Shapes: q_nope [S][Q][H][NB][DN], w_uk [H][NB][DN][DC], w_uv [H][NB][DV][DC].
    Returns (y [S][Q][H][DV], y_branch [S][Q][H][NB][DV] before the sum and
    the rescale, lse [S][Q][H][NB]).
    """
    S, Q, H, NB, DN = q_nope.shape
    DV = w_uv.shape[2]
    y = np.zeros((S, Q, H, DV))
    yb = np.zeros((S, Q, H, NB, DV))
    lse = np.full((S, Q, H, NB), -np.inf)
    for s in range(S):
        L = int(seq_lens[s])
        if L <= 0:
            continue
        C = paged_gather(latent_cache, block_table[s], L, block_size)
        KR = paged_gather(rope_cache, block_table[s], L, block_size)
        for j in range(Q):
            V = visible_length(L, Q, j, causal)
            if V <= 0:
                continue
            for h in range(H):
                for b in range(NB):
                    keys = np.concatenate([C[:V, b] @ w_uk[h, b].T, KR[:V]], axis=1)
                    vals = C[:V, b] @ w_uv[h, b].T
                    q = np.concatenate([q_nope[s, j, h, b], q_rope[s, j, h]])
                    yb[s, j, h, b], lse[s, j, h, b] = _softmax_attend(q, keys, vals, scale)
                y[s, j, h] = out_rescale * yb[s, j, h].sum(axis=0)
    return y, yb, lse


def mla_expanded(q_nope, q_rope, latent_cache, rope_cache, block_table, seq_lens,
                 w_uk, w_uv, scale, causal=True, block_size=64):
    """Textbook MLA decode in expanded form, float64.

    [HN] (TransMLA background) and [ABS]: MLA caches one latent c[t] per token
    (a single latent head) plus a decoupled RoPE key; keys and values are
    low-rank up-projections k[t] = [W_UK[h] c[t] ; k_r[t]], v[t] = W_UV[h] c[t];
    one softmax per head, no branches and no output factor.

    Shapes: latent_cache [blocks][BS][DC] (single latent), q_nope [S][Q][H][DN],
    w_uk [H][DN][DC], w_uv [H][DV][DC]. Returns (y [S][Q][H][DV], lse [S][Q][H]).
    """
    S, Q, H, DN = q_nope.shape
    DV = w_uv.shape[1]
    y = np.zeros((S, Q, H, DV))
    lse = np.full((S, Q, H), -np.inf)
    for s in range(S):
        L = int(seq_lens[s])
        if L <= 0:
            continue
        C = paged_gather(latent_cache, block_table[s], L, block_size)
        KR = paged_gather(rope_cache, block_table[s], L, block_size)
        for j in range(Q):
            V = visible_length(L, Q, j, causal)
            if V <= 0:
                continue
            for h in range(H):
                keys = np.concatenate([C[:V] @ w_uk[h].T, KR[:V]], axis=1)
                vals = C[:V] @ w_uv[h].T
                q = np.concatenate([q_nope[s, j, h], q_rope[s, j, h]])
                y[s, j, h], lse[s, j, h] = _softmax_attend(q, keys, vals, scale)
    return y, lse
