"""Pins for the float64 CPU oracle (no GPU).

Each test checks the oracle against something other than itself: brute-force
scalar loops, torch's scaled_dot_product_attention on explicitly materialised
keys and values, closed forms, a hand-derived worked example, invariants of
the method, and Gaussian exponential-tilting statistics at full workload size.
"""
import json
import math
import os

import numpy as np
import pytest
import torch
from hypothesis import given, settings, strategies as st, HealthCheck

from latent_kv_cache_amd import configs
from latent_kv_cache_amd.inputs import make_inputs
from oracle import (mla_expanded, mlra_decode, mlra_decode_bruteforce,
                    mlra_expanded, paged_gather)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _run(inp, reduce="sum", fn=mlra_decode, **kw):
    c = inp.cfg
    args = dict(scale=c.scale, out_rescale=c.out_rescale, reduce=reduce,
                causal=c.causal, block_size=c.block_size)
    args.update(kw)
    return fn(inp.q_latent, inp.q_rope, inp.latent_cache, inp.rope_cache,
              inp.block_table, inp.seq_lens, **args)


def _small(**kw):
    base = dict(name="small", num_seqs=2, q_len=1, num_heads=3, n_branch=2, d_latent=6,
                d_rope=3, dtype="fp32", context=37, block_size=8, seed=11,
                scale=0.4, out_rescale=0.5)
    base.update(kw)
    return configs.DecodeConfig(**base)


# --------------------------------------------------------------------------- brute force

def test_bruteforce_matches_vectorised_tiny_config():
    inp = make_inputs(configs.TINY_MLRA4_FP32)
    for reduce in ("sum", "concat"):
        o1, l1 = _run(inp, reduce)
        o2, l2 = _run(inp, reduce, fn=mlra_decode_bruteforce)
        np.testing.assert_allclose(o1, o2, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(l1, l2, rtol=1e-12, atol=1e-12)


@settings(max_examples=40, deadline=None, suppress_health_check=[HealthCheck.too_slow])
@given(S=st.integers(1, 3), Q=st.integers(1, 2), H=st.integers(1, 3),
       NB=st.sampled_from([1, 2, 4]), DC=st.integers(1, 6), DR=st.integers(1, 4),
       lo=st.integers(0, 40), span=st.integers(0, 40), BS=st.sampled_from([1, 4, 8]),
       seed=st.integers(0, 10_000), reduce=st.sampled_from(["sum", "concat"]),
       causal=st.booleans())
def test_bruteforce_matches_vectorised_random_shapes(S, Q, H, NB, DC, DR, lo, span, BS,
                                                     seed, reduce, causal):
    cfg = _small(num_seqs=S, q_len=Q, num_heads=H, n_branch=NB, d_latent=DC, d_rope=DR,
                 context=None, context_range=(lo, lo + span), block_size=BS, seed=seed,
                 causal=causal, scale=0.7)
    inp = make_inputs(cfg)
    o1, l1 = _run(inp, reduce)
    o2, l2 = _run(inp, reduce, fn=mlra_decode_bruteforce)
    np.testing.assert_allclose(o1, o2, rtol=1e-11, atol=1e-12)
    assert np.array_equal(np.isneginf(l1), np.isneginf(l2))
    fin = np.isfinite(l1)
    np.testing.assert_allclose(l1[fin], l2[fin], rtol=1e-11, atol=1e-12)
    assert not np.isnan(o1).any()


# --------------------------------------------------------------------------- golden

def _ev(x):
    if isinstance(x, list):
        return [_ev(v) for v in x]
    if isinstance(x, str):
        return float(eval(x, {"__builtins__": {}}, {"ln2": math.log(2), "ln3": math.log(3),
                                                    "ln9": math.log(9), "ln4": math.log(4),
                                                    "nan": float("nan")}))
    return float(x)


@pytest.mark.parametrize("fn", [mlra_decode, mlra_decode_bruteforce])
def test_hand_derived_golden_example(fn):
    g = json.load(open(os.path.join(GOLDEN, "hand_example.json")))
    arr = {k: np.array(_ev(g[k])) for k in ("q_latent", "q_rope", "latent_cache",
                                            "rope_cache")}
    table = np.array(g["block_table"], dtype=np.int32)
    lens = np.array(g["seq_lens"], dtype=np.int32)
    for reduce, key in (("sum", "expected_out_sum"), ("concat", "expected_out_concat")):
        out, lse = fn(arr["q_latent"], arr["q_rope"], arr["latent_cache"], arr["rope_cache"],
                      table, lens, scale=g["scale"], out_rescale=g["out_rescale"],
                      reduce=reduce, causal=True, block_size=g["block_size"])
        np.testing.assert_allclose(out, np.array(_ev(g[key])), rtol=1e-13, atol=1e-13)
        np.testing.assert_allclose(lse, np.array(_ev(g["expected_lse"])), rtol=1e-13)


# --------------------------------------------------------------------------- expanded form

def _updown(rng, H, NB, DN, DV, DC):
    w_uk = rng.standard_normal((H, NB, DN, DC)) / math.sqrt(DC)
    w_uv = rng.standard_normal((H, NB, DV, DC)) / math.sqrt(DC)
    return w_uk, w_uv


@pytest.mark.parametrize("Q,causal", [(1, True), (2, True), (2, False)])
def test_absorbed_equals_expanded(Q, causal):
    cfg = _small(q_len=Q, causal=causal, n_branch=4, context=None, context_range=(5, 40))
    inp = make_inputs(cfg)
    S, _, H, NB, DC = inp.q_latent.shape
    rng = np.random.default_rng(123)
    DN, DV = 5, 7
    w_uk, w_uv = _updown(rng, H, NB, DN, DV, DC)
    q_nope = rng.standard_normal((S, Q, H, NB, DN))
    q_lat = np.einsum("hbnc,sjhbn->sjhbc", w_uk, q_nope)  # absorb W_UK into the query
    y, yb, lse_e = mlra_expanded(q_nope, inp.q_rope, inp.latent_cache, inp.rope_cache,
                                 inp.block_table, inp.seq_lens, w_uk, w_uv, cfg.scale,
                                 cfg.out_rescale, causal=causal, block_size=cfg.block_size)
    oc, lse_a = mlra_decode(q_lat, inp.q_rope, inp.latent_cache, inp.rope_cache,
                            inp.block_table, inp.seq_lens, cfg.scale, 1.0, "concat",
                            causal, cfg.block_size)
    # per branch: W_UV o_b == y_b; concat(o_b) . vstack(W_UV^T) == sum_b y_b
    np.testing.assert_allclose(np.einsum("hbvc,sjhbc->sjhbv", w_uv, oc), yb,
                               rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(cfg.out_rescale * np.einsum("hbvc,sjhbc->sjhv", w_uv, oc), y,
                               rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(lse_a, lse_e, rtol=1e-12, atol=1e-12)
    # sum reduce is exact when the branches share the value up-projection
    w_shared = np.broadcast_to(w_uv[:, :1], w_uv.shape).copy()
    y2, _, _ = mlra_expanded(q_nope, inp.q_rope, inp.latent_cache, inp.rope_cache,
                             inp.block_table, inp.seq_lens, w_uk, w_shared, cfg.scale,
                             cfg.out_rescale, causal=causal, block_size=cfg.block_size)
    osum, _ = mlra_decode(q_lat, inp.q_rope, inp.latent_cache, inp.rope_cache,
                          inp.block_table, inp.seq_lens, cfg.scale, cfg.out_rescale, "sum",
                          causal, cfg.block_size)
    np.testing.assert_allclose(np.einsum("hvc,sjhc->sjhv", w_shared[:, 0], osum), y2,
                               rtol=1e-10, atol=1e-12)


def _sdpa(q, k, v, scale):
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float64))[None, None]
    return torch.nn.functional.scaled_dot_product_attention(
        t(q)[:, :, None], t(k), t(v), scale=scale)[0, 0, 0].numpy()


def test_expanded_equals_torch_sdpa():
    cfg = _small(q_len=2, n_branch=2, context=None, context_range=(9, 30))
    inp = make_inputs(cfg)
    S, Q, H, NB, DC = inp.q_latent.shape
    rng = np.random.default_rng(7)
    DN, DV = 4, 5
    w_uk, w_uv = _updown(rng, H, NB, DN, DV, DC)
    q_nope = rng.standard_normal((S, Q, H, NB, DN))
    y, yb, _ = mlra_expanded(q_nope, inp.q_rope, inp.latent_cache, inp.rope_cache,
                             inp.block_table, inp.seq_lens, w_uk, w_uv, cfg.scale,
                             cfg.out_rescale, causal=True, block_size=cfg.block_size)
    for s in range(S):
        L = int(inp.seq_lens[s])
        # gather through the block table independently of paged_gather
        lat = np.stack([inp.latent_cache[inp.block_table[s, t // 8], t % 8] for t in range(L)])
        kr = np.stack([inp.rope_cache[inp.block_table[s, t // 8], t % 8] for t in range(L)])
        for j in range(Q):
            V = L - (Q - 1 - j)
            for h in range(H):
                acc = 0
                for b in range(NB):
                    k = np.concatenate([lat[:V, b] @ w_uk[h, b].T, kr[:V]], axis=1)
                    v = lat[:V, b] @ w_uv[h, b].T
                    q = np.concatenate([q_nope[s, j, h, b], inp.q_rope[s, j, h]])
                    ref = _sdpa(q, k, v, cfg.scale)
                    np.testing.assert_allclose(yb[s, j, h, b], ref, rtol=1e-10, atol=1e-12)
                    acc = acc + ref
                np.testing.assert_allclose(y[s, j, h], cfg.out_rescale * acc, rtol=1e-10,
                                           atol=1e-12)


def test_single_branch_equals_textbook_mla():
    """n_branch = 1 with a 512-wide-style single latent is standard MLA."""
    cfg = _small(n_branch=1, d_latent=16, d_rope=4, context=45, out_rescale=1.0)
    inp = make_inputs(cfg)
    S, Q, H, _, DC = inp.q_latent.shape
    rng = np.random.default_rng(5)
    DN, DV = 6, 6
    w_uk = rng.standard_normal((H, DN, DC)) / 4
    w_uv = rng.standard_normal((H, DV, DC)) / 4
    q_nope = rng.standard_normal((S, Q, H, DN))
    single = inp.latent_cache[:, :, 0]                          # [blocks][BS][DC]
    y, lse_m = mla_expanded(q_nope, inp.q_rope, single, inp.rope_cache, inp.block_table,
                            inp.seq_lens, w_uk, w_uv, cfg.scale, block_size=cfg.block_size)
    q_lat = np.einsum("hnc,sjhn->sjhc", w_uk, q_nope)[:, :, :, None]
    o, lse_a = mlra_decode(q_lat, inp.q_rope, inp.latent_cache, inp.rope_cache,
                           inp.block_table, inp.seq_lens, cfg.scale, 1.0, "sum", True,
                           cfg.block_size)
    np.testing.assert_allclose(np.einsum("hvc,sjhc->sjhv", w_uv, o), y, rtol=1e-10,
                               atol=1e-12)
    np.testing.assert_allclose(lse_a[..., 0], lse_m, rtol=1e-12)
    # and MLA itself against torch SDPA for one head
    L = int(inp.seq_lens[0])
    lat = paged_gather(single, inp.block_table[0], L, 8)
    kr = paged_gather(inp.rope_cache, inp.block_table[0], L, 8)
    k = np.concatenate([lat @ w_uk[1].T, kr], axis=1)
    ref = _sdpa(np.concatenate([q_nope[0, 0, 1], inp.q_rope[0, 0, 1]]), k, lat @ w_uv[1].T,
                cfg.scale)
    np.testing.assert_allclose(y[0, 0, 1], ref, rtol=1e-10)


def test_negative_control_sum_after_differs_from_sum_before():
    """MLRA (softmax per branch, then sum) must differ from MLA over the
    concatenated latent (one softmax over the summed branch scores)."""
    cfg = _small(n_branch=4, d_latent=8, context=50)
    inp = make_inputs(cfg)
    o_mlra, _ = _run(inp, "concat", out_rescale=1.0)
    NBk = inp.latent_cache.shape[:2] + (1, 4 * 8)
    cat_cache = inp.latent_cache.reshape(NBk)
    S, Q, H = inp.q_latent.shape[:3]
    cat_q = inp.q_latent.reshape(S, Q, H, 1, 32)
    o_mla, _ = mlra_decode(cat_q, inp.q_rope, cat_cache, inp.rope_cache, inp.block_table,
                           inp.seq_lens, cfg.scale, 1.0, "sum", True, cfg.block_size)
    diff = np.abs(o_mla.reshape(o_mlra.shape) - o_mlra).max()
    assert diff > 1e-3


# --------------------------------------------------------------------------- closed forms

def test_closed_form_single_visible_token():
    cfg = _small(context=1, n_branch=2)
    inp = make_inputs(cfg)
    o, lse = _run(inp, "concat", out_rescale=1.0)
    blk = inp.block_table[:, 0]
    for s in range(cfg.num_seqs):
        c = inp.latent_cache[blk[s], 0].astype(np.float64)          # [NB][DC]
        kr = inp.rope_cache[blk[s], 0].astype(np.float64)
        for h in range(cfg.num_heads):
            np.testing.assert_allclose(o[s, 0, h], c, rtol=1e-14)
            z = cfg.scale * (np.sum(inp.q_latent[s, 0, h] * c, axis=1)
                             + np.dot(inp.q_rope[s, 0, h], kr))
            np.testing.assert_allclose(lse[s, 0, h], z, rtol=1e-12)


def test_closed_form_zero_queries_give_mean_and_log_length():
    cfg = _small(context=None, context_range=(3, 60), num_seqs=3)
    inp = make_inputs(cfg)
    inp.q_latent[:] = 0
    inp.q_rope[:] = 0
    o, lse = _run(inp, "concat", out_rescale=1.0)
    for s in range(cfg.num_seqs):
        L = int(inp.seq_lens[s])
        rows = [inp.latent_cache[inp.block_table[s, t // 8], t % 8] for t in range(L)]
        np.testing.assert_allclose(o[s, 0, 0], np.mean(np.array(rows, dtype=np.float64), axis=0),
                                   rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(lse[s, 0], math.log(L), rtol=1e-14)


def test_closed_form_constant_latent_and_dominant_token():
    cfg = _small(context=29, n_branch=2)
    inp = make_inputs(cfg)
    inp.latent_cache[..., 0, :] = 1.25   # branch 0 constant: output is the constant
    o, _ = _run(inp, "concat", out_rescale=1.0)
    np.testing.assert_allclose(o[:, :, :, 0], 1.25, rtol=1e-14)
    # one token with a huge score takes all the weight
    inp2 = make_inputs(cfg)
    t_star = 17
    blk, slot = inp2.block_table[0, t_star // 8], t_star % 8
    inp2.rope_cache[blk, slot] = 0
    inp2.rope_cache[blk, slot, 0] = 1e4
    inp2.q_rope[0, 0, :, :] = 0
    inp2.q_rope[0, 0, :, 0] = 1.0
    o2, _ = _run(inp2, "concat", out_rescale=1.0)
    np.testing.assert_allclose(o2[0, 0, :, :], np.broadcast_to(
        inp2.latent_cache[blk, slot].astype(np.float64), o2[0, 0].shape), rtol=1e-12)


def test_closed_form_nothing_visible():
    cfg = _small(q_len=2, context=2, num_seqs=3, seed=1)
    inp = make_inputs(cfg)
    inp.seq_lens[:] = [0, 1, 2]
    o, lse = _run(inp, "sum")
    assert np.all(o[0] == 0) and np.all(np.isneginf(lse[0]))         # L = 0
    assert np.all(o[1, 0] == 0) and np.all(np.isneginf(lse[1, 0]))   # query 0 sees 0
    assert np.all(np.isfinite(lse[1, 1])) and np.all(np.isfinite(lse[2]))


# --------------------------------------------------------------------------- invariants

def test_causal_consistency_two_queries():
    cfg = _small(q_len=2, context=None, context_range=(2, 70), num_seqs=3)
    inp = make_inputs(cfg)
    o, lse = _run(inp, "concat")
    for j, shift in ((1, 0), (0, 1)):
        one = make_inputs(cfg)
        one.q_latent = inp.q_latent[:, j:j + 1].copy()
        one.q_rope = inp.q_rope[:, j:j + 1].copy()
        one.seq_lens = inp.seq_lens - shift
        o1, l1 = mlra_decode(one.q_latent, one.q_rope, inp.latent_cache, inp.rope_cache,
                             inp.block_table, one.seq_lens, cfg.scale, cfg.out_rescale,
                             "concat", True, cfg.block_size)
        np.testing.assert_allclose(o[:, j], o1[:, 0], rtol=1e-13, atol=1e-15)
        np.testing.assert_allclose(lse[:, j], l1[:, 0], rtol=1e-13)


def test_fused_equals_sum_of_single_branch_shares():
    cfg = _small(n_branch=4, context=None, context_range=(20, 90), num_seqs=3)
    inp = make_inputs(cfg)
    o, lse = _run(inp, "sum")
    acc = 0
    for b in range(4):
        ob, lb = mlra_decode(inp.q_latent[:, :, :, b:b + 1], inp.q_rope,
                             inp.latent_cache[:, :, b:b + 1], inp.rope_cache,
                             inp.block_table, inp.seq_lens, cfg.scale, cfg.out_rescale,
                             "sum", True, cfg.block_size)
        acc = acc + ob
        np.testing.assert_allclose(lse[..., b], lb[..., 0], rtol=1e-14)
    np.testing.assert_allclose(o, acc, rtol=1e-12, atol=1e-14)


def test_block_permutation_invariance_and_identity_table():
    cfg = _small(context=None, context_range=(10, 64), num_seqs=3, placement="identity")
    inp = make_inputs(cfg)
    o, lse = _run(inp, "concat")
    # contiguous: identity table means token t is row t of the flattened cache
    flat = inp.latent_cache.reshape(-1, *inp.latent_cache.shape[2:])
    start = 0
    for s in range(3):
        L = int(inp.seq_lens[s])
        got = paged_gather(inp.latent_cache, inp.block_table[s], L, 8)
        np.testing.assert_array_equal(got, flat[start:start + L])
        start += -(-L // 8) * 8
    # relabel physical blocks with a permutation; the result must not change
    rng = np.random.default_rng(3)
    perm = rng.permutation(inp.num_blocks)           # new position of old block i
    lat2 = np.empty_like(inp.latent_cache)
    rope2 = np.empty_like(inp.rope_cache)
    lat2[perm] = inp.latent_cache
    rope2[perm] = inp.rope_cache
    o2, lse2 = mlra_decode(inp.q_latent, inp.q_rope, lat2, rope2, perm[inp.block_table],
                           inp.seq_lens, cfg.scale, cfg.out_rescale, "concat", True, 8)
    np.testing.assert_array_equal(o, o2)
    np.testing.assert_array_equal(lse, lse2)


def test_unused_slots_are_never_read():
    """Rows past the end and the spare block are NaN; outputs stay finite."""
    cfg = _small(q_len=2, context=None, context_range=(1, 70), num_seqs=4)
    inp = make_inputs(cfg)
    assert np.isnan(inp.latent_cache[inp.poison_block]).all()
    o, lse = _run(inp, "sum")
    assert np.isfinite(o).all()
    assert not np.isnan(lse).any()


# --------------------------------------------------------------------------- statistics

def _tilting_check(inp, s_list):
    """Gaussian exponential tilting: for c ~ N(0, I), k ~ N(0, I) independent,
    with a = scale*q_b and a_r = scale*q_r, sigma^2 = |a|^2 + |a_r|^2:
        E[exp(z)] = exp(sigma^2/2)      -> lse ~ ln V + sigma^2/2,
        E[exp(z) c] / E[exp(z)] = a     -> o_b ~ a,
    with sampling sd sqrt((e^{sigma^2} - 1)/V) for lse and
    sqrt(e^{sigma^2} (1 + a_d^2)/V) per coordinate of o_b."""
    cfg = inp.cfg
    o, lse = mlra_decode(inp.q_latent[s_list], inp.q_rope[s_list], inp.latent_cache,
                         inp.rope_cache, inp.block_table[s_list], inp.seq_lens[s_list],
                         cfg.scale, 1.0, "concat", cfg.causal, cfg.block_size)
    a = cfg.scale * inp.q_latent[s_list].astype(np.float64)          # [S][Q][H][NB][DC]
    ar = cfg.scale * inp.q_rope[s_list].astype(np.float64)           # [S][Q][H][DR]
    sig2 = (a ** 2).sum(-1) + (ar ** 2).sum(-1)[..., None]           # [S][Q][H][NB]
    V = inp.seq_lens[s_list].astype(np.float64)[:, None, None, None]
    z_lse = (lse - np.log(V) - sig2 / 2) / np.sqrt(np.expm1(sig2) / V)
    z_o = (o - a) / np.sqrt(np.exp(sig2)[..., None] * (1 + a ** 2) / V[..., None])
    return z_lse, z_o


@pytest.mark.slow
def test_statistics_full_size_tp_share():
    inp = make_inputs(configs.MLRA4_TP_SHARE)
    z_lse, z_o = _tilting_check(inp, list(range(inp.cfg.num_seqs)))
    assert np.abs(z_lse).max() < 6.0
    assert np.abs(z_o).max() < 6.5
    assert abs(z_o.mean()) < 0.05 and 0.8 < z_o.std() < 1.2
    assert abs(z_lse.mean()) < 6.0 / math.sqrt(z_lse.size)
