"""GPU parity of chunked-prefill attention (mlra_prefill_attention through the
C ABI) against the float64 CPU oracle.

The oracle's mlra_decode defines the output for any chunk length Q. Small
workloads are compared element by element, at sizes that span several
256-row workgroups with a ragged last one and contexts that end inside a
cache block; full-size workloads are compared on sampled query tokens (all
heads and branches of each), for which the oracle is called with one query
token and the visible length as its sequence length (the causal rule of the
oracle, token j of Q sees L - (Q - 1 - j) tokens). Bar: as for decode
(max-abs 2e-2, L2-relative 1e-2, lse within 1e-3, -inf exactly where the
oracle has it).
"""
import numpy as np
import pytest
import torch

from latent_kv_cache_amd import api, configs
from latent_kv_cache_amd.inputs import make_inputs, to_device
from oracle import mlra_decode

pytestmark = pytest.mark.gpu

ATOL, RTOL_L2, LSE_ATOL = 2e-2, 1e-2, 1e-3


def _say(msg):
    print(f"[gpu-case] {msg}", flush=True)


def run_prefill(inp, reduce="sum", num_splits=0, dev=None, seq_lens=None, sum_seq_lens=0):
    cfg = inp.cfg
    d = dev if dev is not None else to_device(inp)
    sl = d["seq_lens"] if seq_lens is None else torch.from_numpy(seq_lens).cuda()
    out, lse = api.mlra_prefill_attention(
        d["q_latent"], d["q_rope"], d["latent_cache"], d["rope_cache"], d["block_table"], sl,
        cfg.n_branch, cfg.scale, cfg.out_rescale, max_seq_len=inp.max_seq_len, reduce=reduce,
        causal=cfg.causal, num_splits=num_splits, sum_seq_lens=sum_seq_lens)
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


def oracle(inp, reduce="sum", seq_lens=None):
    c = inp.cfg
    return mlra_decode(inp.q_latent, inp.q_rope, inp.latent_cache, inp.rope_cache,
                       inp.block_table, inp.seq_lens if seq_lens is None else seq_lens,
                       c.scale, c.out_rescale, reduce, c.causal, c.block_size)


def oracle_tokens(inp, s, js, reduce="sum"):
    """Oracle output of query tokens js of sequence s (every head and branch)."""
    c = inp.cfg
    L = int(inp.seq_lens[s])
    outs, lses = [], []
    for j in js:
        V = L - (c.q_len - 1 - j) if c.causal else L
        o, l = mlra_decode(inp.q_latent[s:s + 1, j:j + 1], inp.q_rope[s:s + 1, j:j + 1],
                           inp.latent_cache, inp.rope_cache, inp.block_table[s:s + 1],
                           np.array([V], dtype=np.int32), c.scale, c.out_rescale, reduce,
                           False, c.block_size)
        outs.append(o[0, 0])
        lses.append(l[0, 0])
    return np.stack(outs), np.stack(lses)


def assert_parity(out, lse, ref_out, ref_lse):
    assert out.shape == ref_out.shape and lse.shape == ref_lse.shape
    assert not np.isnan(out).any(), "NaN in GPU output"
    err = np.abs(out - ref_out)
    rel = np.linalg.norm(out - ref_out) / max(np.linalg.norm(ref_out), 1e-30)
    assert err.max() <= ATOL, f"max-abs {err.max():.3e}"
    assert rel <= RTOL_L2 or np.linalg.norm(ref_out) == 0, f"L2-rel {rel:.3e}"
    ninf = np.isneginf(ref_lse)
    assert np.array_equal(np.isneginf(lse), ninf), "-inf pattern of lse differs"
    if (~ninf).any():
        lerr = np.abs(lse[~ninf] - ref_lse[~ninf]).max()
        assert lerr <= LSE_ATOL, f"lse max-abs {lerr:.3e}"


def _cfg(**kw):
    base = dict(name="p", num_seqs=2, q_len=37, num_heads=8, n_branch=1, d_latent=128,
                d_rope=64, dtype="bf16", context=None, context_range=(40, 300), seed=31,
                scale=1 / np.sqrt(192), out_rescale=0.5)
    base.update(kw)
    return configs.DecodeConfig(**base)


# Every kernel instance (latent width x RoPE width) with 1, 2 and 4 branches;
# 37 tokens x 8 heads = 296 rows: a full 256-row group and a ragged one.
SHAPES = [(nb, dc, dr) for nb in (1, 2, 4) for dc in (64, 128) for dr in (32, 64)]


@pytest.mark.parametrize("nb,dc,dr", SHAPES)
def test_small_every_instance(nb, dc, dr):
    cfg = _cfg(n_branch=nb, d_latent=dc, d_rope=dr, seed=200 + 11 * nb + dc + dr,
               scale=1 / np.sqrt(dc + dr))
    inp = make_inputs(cfg)
    dev = to_device(inp)
    for reduce in ("sum", "concat"):
        _say(f"prefill small nb={nb} dc={dc} dr={dr} {reduce} lens={inp.seq_lens.tolist()}")
        out, lse = run_prefill(inp, reduce, dev=dev)
        assert_parity(out, lse, *oracle(inp, reduce))


@pytest.mark.parametrize("num_splits", [0, 1, 2, 3, 7])
def test_split_counts_and_wave_aligned_tokens(num_splits):
    # 32 heads: each wave's rows are one query token (a wave-uniform causal
    # edge); contexts up to 900 tokens split into up to 7 ranges
    cfg = _cfg(num_seqs=3, q_len=24, num_heads=32, n_branch=2, context_range=(24, 900),
               seed=41)
    inp = make_inputs(cfg)
    dev = to_device(inp)
    for reduce in ("sum", "concat"):
        _say(f"prefill splits={num_splits} {reduce} lens={inp.seq_lens.tolist()}")
        out, lse = run_prefill(inp, reduce, num_splits=num_splits, dev=dev)
        assert_parity(out, lse, *oracle(inp, reduce))


def test_rows_of_a_wave_span_several_tokens():
    # 5 heads: 32-row tiles cut across query tokens, each lane its own edge
    cfg = _cfg(num_seqs=2, q_len=61, num_heads=5, n_branch=1, context_range=(61, 200),
               seed=42)
    inp = make_inputs(cfg)
    for splits in (0, 2):
        _say(f"prefill h=5 q=61 splits={splits}")
        out, lse = run_prefill(inp, "sum", num_splits=splits)
        assert_parity(out, lse, *oracle(inp, "sum"))


def test_non_causal_chunk():
    cfg = _cfg(causal=False, num_heads=16, q_len=20, n_branch=4, seed=43)
    inp = make_inputs(cfg)
    for reduce in ("sum", "concat"):
        _say(f"prefill non-causal {reduce}")
        out, lse = run_prefill(inp, reduce, num_splits=2)
        assert_parity(out, lse, *oracle(inp, reduce))


def test_empty_and_short_sequences():
    # L = 0, L < Q (early query tokens see nothing), L = 1, L at a block edge
    cfg = _cfg(num_seqs=5, q_len=40, num_heads=8, n_branch=2, context=192, seed=44)
    inp = make_inputs(cfg)
    lens = np.array([0, 17, 1, 64, 192], dtype=np.int32)
    dev = to_device(inp)
    for reduce in ("sum", "concat"):
        for splits in (0, 1, 3):
            _say(f"prefill short lens={lens.tolist()} {reduce} splits={splits}")
            out, lse = run_prefill(inp, reduce, num_splits=splits, dev=dev, seq_lens=lens)
            ro, rl = oracle(inp, reduce, seq_lens=lens)
            assert_parity(out, lse, ro, rl)
            assert np.all(out[0] == 0) and np.all(np.isneginf(lse[0]))


def test_whole_sequence_prefill_small():
    # the chunk is the sequence: token 0 sees itself only
    cfg = _cfg(num_seqs=2, q_len=300, num_heads=4, n_branch=1, context=300, seed=45)
    inp = make_inputs(cfg)
    _say("prefill whole 300")
    out, lse = run_prefill(inp, "sum")
    ro, rl = oracle(inp, "sum")
    assert_parity(out, lse, ro, rl)


def test_repeat_calls_are_bitwise_identical():
    cfg = _cfg(num_seqs=2, q_len=33, num_heads=16, n_branch=4, context_range=(100, 700),
               seed=46)
    inp = make_inputs(cfg)
    dev = to_device(inp)
    _say("prefill determinism")
    a = run_prefill(inp, "sum", dev=dev, num_splits=3)
    b = run_prefill(inp, "sum", dev=dev, num_splits=3)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_dispatch_order_does_not_change_results():
    # Workgroups take their (sequence, row tile, split) item longest first
    # unless the length hint shows a uniform batch; each item's arithmetic is
    # the same either way, so both orders give bit-identical results, and
    # ragged lengths (ranked) match the oracle.
    cfg = _cfg(num_seqs=3, q_len=40, num_heads=16, n_branch=2, context=600, context_range=None,
               seed=52)
    inp = make_inputs(cfg)
    dev = to_device(inp)
    for splits in (0, 3):
        _say(f"prefill uniform batch, ranked and fixed order, splits={splits}")
        ranked = run_prefill(inp, "sum", dev=dev, num_splits=splits)
        fixed = run_prefill(inp, "sum", dev=dev, num_splits=splits,
                            sum_seq_lens=int(inp.seq_lens.sum()))
        assert np.array_equal(ranked[0], fixed[0]) and np.array_equal(ranked[1], fixed[1])
        assert_parity(*ranked, *oracle(inp, "sum"))
    rag = make_inputs(cfg.with_(name="pf_rag_order", context=None, context_range=(40, 900), seed=53))
    _say(f"prefill ragged batch ranked, lens={rag.seq_lens.tolist()}")
    assert_parity(*run_prefill(rag, "concat", sum_seq_lens=int(rag.seq_lens.sum())),
                  *oracle(rag, "concat"))


def test_branch_major_latent_and_padded_rope_strides():
    # latent stored branch-major [blocks][NB][64][DC] (viewed token-major), RoPE
    # keys in rows of twice their width: the loads follow the stride arguments
    cfg = _cfg(num_seqs=2, q_len=30, num_heads=16, n_branch=4, context_range=(30, 400), seed=48)
    inp = make_inputs(cfg)
    d = to_device(inp)
    d["latent_cache"] = d["latent_cache"].permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3)
    assert d["latent_cache"].stride(2) == 64 * cfg.d_latent
    wide = torch.zeros(d["rope_cache"].shape[:2] + (2 * cfg.d_rope,), dtype=d["rope_cache"].dtype,
                       device=d["rope_cache"].device)
    wide[..., :cfg.d_rope] = d["rope_cache"]
    d["rope_cache"] = wide[..., :cfg.d_rope]
    assert d["rope_cache"].stride(1) == 2 * cfg.d_rope
    for reduce in ("sum", "concat"):
        _say(f"prefill strided caches {reduce}")
        out, lse = run_prefill(inp, reduce, dev=d)
        assert_parity(out, lse, *oracle(inp, reduce))


def test_seq_len_above_max_is_clamped_not_read_out_of_bounds():
    # a length past max_seq_len is treated as max_seq_len (never a read past
    # the block table); the result equals the clamped call's
    cfg = _cfg(num_seqs=2, q_len=20, num_heads=8, context=256, context_range=None, seed=49)
    inp = make_inputs(cfg)
    big = np.array([256, 100_000], dtype=np.int32)
    _say("prefill clamped length")
    out, lse = run_prefill(inp, "sum", seq_lens=big)
    ref = run_prefill(inp, "sum", seq_lens=np.array([256, 256], dtype=np.int32))
    assert np.array_equal(out, ref[0]) and np.array_equal(lse, ref[1])
    assert_parity(out, lse, *oracle(inp, "sum"))


def _sampled(cfg, tokens, reduce="sum"):
    inp = make_inputs(cfg)
    _say(f"prefill full {cfg.name} {reduce}")
    out, lse = run_prefill(inp, reduce)
    assert not np.isnan(out).any()
    for s in range(cfg.num_seqs):
        js = [j for j in tokens if j < cfg.q_len]
        ro, rl = oracle_tokens(inp, s, js, reduce)
        assert_parity(out[s, js], lse[s, js], ro, rl)
    return inp, out, lse


def test_full_size_chunked_prefill_sampled_tokens():
    cfg = configs.MLRA4_TP_PREFILL
    _sampled(cfg, [0, 1, 7, 8, 255, 1024, 2046, 2047])


def test_full_size_whole_prefill_sampled_tokens():
    cfg = configs.MLRA4_TP_PREFILL_WHOLE
    inp, out, _ = _sampled(cfg, [0, 1, 31, 32, 63, 64, 4095, 16383])
    # token 0 sees only itself: its output is its own latent times the factor
    c0 = inp.latent_cache[inp.block_table[0, 0], 0, 0].astype(np.float64)
    np.testing.assert_allclose(out[0, 0], np.broadcast_to(cfg.out_rescale * c0, out[0, 0].shape),
                               rtol=0, atol=1e-2)


def test_full_size_fused_branches_sampled_tokens():
    cfg = configs.MLRA4_FUSED_PREFILL
    for reduce in ("sum", "concat"):
        _sampled(cfg, [0, 5, 256, 511], reduce)


def test_long_context_splits_past_the_staged_block_ids():
    # 70,000 cached tokens (1094 tiles) and rows enough that one split would
    # fill the GPU: a split's block ids are staged in LDS (at most 1024
    # tiles), so the context is cut in two and the halves merged
    cfg = _cfg(num_seqs=1, q_len=2048, num_heads=32, n_branch=1, context=70_000,
               context_range=None, seed=47)
    inp = make_inputs(cfg)
    d = to_device(inp)
    dims = api.make_dims(d["q_latent"], d["q_rope"], d["latent_cache"], d["rope_cache"],
                         d["block_table"], max_seq_len=inp.max_seq_len, causal=True)
    plan = api.make_prefill_plan(dims, 1)
    assert plan.splits_per_seq == 2 and plan.tiles_per_split <= 1024
    _say("prefill long context 70000, two splits")
    out, lse = run_prefill(inp, "sum", dev=d)
    js = [0, 1, 1023, 2047]
    ro, rl = oracle_tokens(inp, 0, js, "sum")
    assert_parity(out[0, js], lse[0, js], ro, rl)


def _random_case(rng, i):
    """One seeded random prefill case: branches, latent and RoPE widths, chunk
    length and heads (row counts that do and do not fill 256-row groups),
    ragged cached contexts behind the chunk, causal or not, and an explicit
    split count or the planner's."""
    nb = int(rng.choice([1, 2, 4]))
    dc = int(rng.choice([64, 128]))
    dr = int(rng.choice([32, 64]))
    q = int(rng.integers(1, 97))
    h = int(rng.integers(1, 25))
    s = int(rng.integers(1, 4))
    extra = int(rng.integers(0, 1001))
    cfg = _cfg(name=f"prand{i}", n_branch=nb, d_latent=dc, d_rope=dr, q_len=q, num_heads=h,
               num_seqs=s, context_range=(q, q + extra), causal=bool(rng.integers(4) > 0),
               seed=2000 + i, scale=1 / np.sqrt(dc + dr), out_rescale=float(rng.uniform(0.3, 1.0)))
    return make_inputs(cfg), int(rng.choice([0, 0, 1, 2, 5]))


@pytest.mark.parametrize("i", range(16))
def test_random_shapes_match_the_oracle(i):
    inp, splits = _random_case(np.random.default_rng(5151 + i), i)
    c = inp.cfg
    reduce = "concat" if i % 3 == 0 else "sum"
    _say(f"prefill random {i}: nb={c.n_branch} dc={c.d_latent} dr={c.d_rope} q={c.q_len} "
         f"h={c.num_heads} causal={c.causal} {reduce} splits={splits} lens={inp.seq_lens.tolist()}")
    out, lse = run_prefill(inp, reduce, num_splits=splits)
    assert_parity(out, lse, *oracle(inp, reduce))


@pytest.mark.parametrize("q,h,nb", [(1, 32, 4), (2, 32, 1), (2, 16, 2)])
def test_prefill_and_decode_calls_agree_on_short_chunks(q, h, nb):
    # the two entry points compute the same function: on chunks the decode
    # call accepts, their outputs agree to rounding (different kernels and
    # split orders)
    cfg = _cfg(q_len=q, num_heads=h, n_branch=nb, num_seqs=3, context_range=(q, 1500),
               seed=300 + 10 * q + nb)
    inp = make_inputs(cfg)
    d = to_device(inp)
    _say(f"prefill vs decode q={q} h={h} nb={nb} lens={inp.seq_lens.tolist()}")
    po, pl = run_prefill(inp, "concat", dev=d)
    do, dl = api.mlra_decode_attention(d["q_latent"], d["q_rope"], d["latent_cache"],
                                       d["rope_cache"], d["block_table"], d["seq_lens"], nb,
                                       cfg.scale, cfg.out_rescale, max_seq_len=inp.max_seq_len,
                                       reduce="concat")
    torch.cuda.synchronize()
    do = do.float().cpu().numpy().astype(np.float64)
    dl = dl.cpu().numpy().astype(np.float64)
    assert np.abs(po - do).max() <= 2e-2
    assert np.linalg.norm(po - do) / np.linalg.norm(do) <= 1e-2
    assert np.abs(pl - dl).max() <= 1e-3
