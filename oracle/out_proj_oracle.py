"""Float64 CPU oracle for the output side of MLRA decode: the value
up-projection of every branch and the output projection, as one contraction.

TEST INFRASTRUCTURE ONLY. Imported by ``tests/`` and the CPU-baseline leg of
``bench.py``; never by the product path.

From the pages (cited by title and section):
  [BLOG]  wispaper.ai, "MLRA: Breaking the Sharding Bottleneck in Latent
          Attention" -- "The Core Insight: Sum of Branches, Not Sum of Keys":
          each branch attends on its own and the branch outputs are summed
          after attention; "Mathematical Calibration: Scaling the Latents": the
          summed output is multiplied by a fixed factor.
  [HN]    Hacker News thread on TransMLA: in MLA the value of a head is a
          low-rank up-projection of the cached latent, and the head outputs go
          through the usual output projection.

Readings taken where the pages are silent (each is listed in the design doc):
  * branch b of head h has its own value up-projection W_UV[h][b] (dv x DC),
    so the head's output is sum_b W_UV[h][b] @ o[h][b], where o[h][b] is the
    branch's latent-space attention output already multiplied by the output
    factor (the decode call's CONCAT result);
  * the output projection W_O (D x H*dv) maps the concatenated head outputs
    to the model width D;
  * the two are applied as one contraction over (h, b, c) with the absorbed
    weight W[n][(h, b, c)] = sum_d W_O[n][h*dv + d] * W_UV[h][b][d][c], rows
    stored [D][H*NB*DC] (output feature major).

Parity pins (tests/test_oracle_out_proj.py):
  absorb_weights   -- brute-force loops on tiny shapes; hand-derived golden
                      example.
  out_projection   -- the two-stage definition (per-head sum of branch
                      up-projections, then the output projection) with
                      independent random factors; brute-force loops;
                      hand-derived golden example; linearity.
No function here is parity-unpinned.
"""
from __future__ import annotations

import numpy as np


def absorb_weights(w_uv, w_o) -> np.ndarray:
    """W[n][(h, b, c)] = sum_d W_O[n][h*dv + d] * W_UV[h][b][d][c], float64.

    w_uv [H][NB][dv][DC], w_o [D][H*dv]. Returns [D][H*NB*DC].
    """
    w_uv = np.asarray(w_uv, dtype=np.float64)
    w_o = np.asarray(w_o, dtype=np.float64)
    H, NB, dv, DC = w_uv.shape
    D = w_o.shape[0]
    w = np.empty((D, H, NB, DC))
    for h in range(H):
        wo_h = w_o[:, h * dv:(h + 1) * dv]            # [D][dv]
        for b in range(NB):
            w[:, h, b, :] = wo_h @ w_uv[h, b]         # [D][DC]
    return w.reshape(D, H * NB * DC)


def out_projection(o_concat, w) -> np.ndarray:
    """y[s][j][n] = sum_{h,b,c} o[s][j][h][b][c] * W[n][(h, b, c)], float64.

    o_concat [S][Q][H][NB][DC] (the decode call's CONCAT output), w
    [D][H*NB*DC]. Returns [S][Q][D].
    """
    o = np.asarray(o_concat, dtype=np.float64)
    S, Q = o.shape[:2]
    x = o.reshape(S * Q, -1)
    return (x @ np.asarray(w, dtype=np.float64).T).reshape(S, Q, -1)
