"""GPU parity of the output projection (mlra_out_projection) against the
float64 oracle.

Bar: |y - ref| <= 2^-8 |ref| + 1e-3 * s, where s = sqrt(K) * rms(x) * rms(w) is
the size of a typical output: the bf16 output rounds to half a unit in the
last place (2^-9 relative) and float32 accumulation over K terms adds far less
than 1e-3 s.
"""
import numpy as np
import pytest
import torch

from latent_kv_cache_amd import api, configs
from latent_kv_cache_amd.inputs import make_inputs, make_out_proj_inputs, to_device
from oracle import absorb_weights, mlra_decode, out_projection

pytestmark = pytest.mark.gpu


def _say(msg):
    print(f"[gpu-case] {msg}", flush=True)


def _assert_close(y, ref, x, w):
    s = np.sqrt(x.shape[-1]) * np.sqrt(np.mean(x.astype(np.float64) ** 2)) * np.sqrt(
        np.mean(w.astype(np.float64) ** 2))
    err = np.abs(y - ref)
    bound = 2.0 ** -8 * np.abs(ref) + 1e-3 * s
    assert not np.isnan(y).any()
    assert (err <= bound).all(), f"max excess {(err - bound).max():.3e} (s={s:.3e})"


def _run(x, w):
    xd = torch.from_numpy(x).cuda().to(torch.bfloat16)
    wd = torch.from_numpy(w).cuda().to(torch.bfloat16)
    y = api.mlra_out_projection(xd, api.pack_out_projection_weight(wd))
    torch.cuda.synchronize()
    return y.float().cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("m,k,d", [(1, 512, 128), (16, 4096, 4096), (33, 512, 384), (64, 1024, 256),
                                   (100, 1536, 128), (128, 2048, 128), (7, 512, 4096),
                                   (20, 1024, 640), (32, 16384, 4096), (128, 16384, 256),
                                   (96, 16384, 4096)])  # x staged in sub-chunks inside the loop
def test_out_projection_shapes(m, k, d):
    x, w = make_out_proj_inputs(m, k, d, seed=m + k + d)
    _say(f"out-proj m={m} k={k} d={d}")
    y = _run(x, w)
    _assert_close(y, out_projection(x[:, None, None, None, :], w)[:, 0], x, w)


def test_packed_layout_and_determinism():
    k, d = 1024, 256
    x, w = make_out_proj_inputs(20, k, d, seed=8)
    wd = torch.from_numpy(w).cuda().to(torch.bfloat16)
    _say("out-proj packed layout")
    packed = api.pack_out_projection_weight(wd).view(torch.int16).cpu().numpy()
    wi = wd.view(torch.int16).cpu().numpy()
    # packed[g][kb][w][q][l][e] = W[128g + 16w + l%16][64kb + 32q + 8(l/16) + e]
    g, kb, tw, q, l, e = np.meshgrid(np.arange(d // 128), np.arange(k // 64), np.arange(8),
                                     np.arange(2), np.arange(64), np.arange(8), indexing="ij")
    expect = wi[128 * g + 16 * tw + l % 16, 64 * kb + 32 * q + 8 * (l // 16) + e]
    assert np.array_equal(packed.reshape(expect.shape), expect)
    assert np.array_equal(_run(x, w), _run(x, w))


def test_decode_then_out_projection_matches_the_oracle_chain():
    # MLRA-4 at full width for a few sequences: decode (CONCAT) -> output side,
    # with W absorbed from random per-branch value up-projections and W_O.
    cfg = configs.MLRA4_FUSED.with_(num_seqs=3, context=None, context_range=(500, 3000), seed=17)
    inp = make_inputs(cfg)
    d = to_device(inp)
    H, NB, DC, dv, D = cfg.num_heads, cfg.n_branch, cfg.d_latent, 128, 4096
    rng = np.random.default_rng(23)
    w_uv = rng.standard_normal((H, NB, dv, DC)) / np.sqrt(DC)
    w_o = rng.standard_normal((D, H * dv)) / np.sqrt(H * dv)
    w = absorb_weights(w_uv, w_o).astype(np.float32)
    _say("decode (concat) then out-proj")
    o, _ = api.mlra_decode_attention(d["q_latent"], d["q_rope"], d["latent_cache"],
                                     d["rope_cache"], d["block_table"], d["seq_lens"], NB,
                                     cfg.scale, cfg.out_rescale, reduce="concat",
                                     max_seq_len=inp.max_seq_len)
    wd = torch.from_numpy(w).cuda().to(torch.bfloat16)
    y = api.mlra_out_projection(o.contiguous(), api.pack_out_projection_weight(wd))
    torch.cuda.synchronize()
    y = y.float().cpu().numpy().astype(np.float64)
    # the projection alone, on the GPU's own decode output and bf16 weight
    o_h = o.float().cpu().numpy().astype(np.float64)
    w_h = wd.float().cpu().numpy().astype(np.float64)
    ref_proj = out_projection(o_h, w_h)
    x2 = o_h.reshape(o_h.shape[0] * o_h.shape[1], -1)
    _assert_close(y.reshape(-1, D), ref_proj.reshape(-1, D), x2, w_h)
    # and the whole chain against the float64 oracle (decode + exact weights)
    ro, _ = mlra_decode(inp.q_latent, inp.q_rope, inp.latent_cache, inp.rope_cache,
                        inp.block_table, inp.seq_lens, cfg.scale, cfg.out_rescale, "concat")
    ref = out_projection(ro, absorb_weights(w_uv, w_o))
    rel = np.linalg.norm(y - ref) / np.linalg.norm(ref)
    assert rel <= 1e-2, f"chain L2-rel {rel:.3e}"
