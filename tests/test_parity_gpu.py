"""GPU parity: the HIP path through the C ABI against the float64 CPU oracle.

Bar (per output tensor): max |out - ref| <= 2e-2 and ||out - ref||_2 / ||ref||_2
<= 1e-2; lse within 1e-3 absolute where finite, and -inf exactly where the
oracle has -inf. float32 workloads must also be within 1e-4 absolute.
"""
import numpy as np
import pytest
import torch

from latent_kv_cache_amd import _lib, api, configs
from latent_kv_cache_amd.inputs import make_inputs, to_device
from oracle import mlra_decode

pytestmark = pytest.mark.gpu

ATOL, RTOL_L2, LSE_ATOL = 2e-2, 1e-2, 1e-3


def _say(msg):
    print(f"[gpu-case] {msg}", flush=True)


def run_gpu(inp, reduce="sum", num_splits=0, dev=None, hint=True, entry="mlra"):
    cfg = inp.cfg
    d = dev if dev is not None else to_device(inp)
    kw = dict(max_seq_len=inp.max_seq_len, causal=cfg.causal, num_splits=num_splits,
              sum_seq_lens=int(inp.seq_lens.sum()) if hint else 0)
    if entry == "mla":
        out, lse = api.mla_decode_attention(d["q_latent"], d["q_rope"], d["latent_cache"],
                                            d["rope_cache"], d["block_table"], d["seq_lens"],
                                            cfg.scale, **kw)
        lse = lse[..., None]
    else:
        out, lse = api.mlra_decode_attention(d["q_latent"], d["q_rope"], d["latent_cache"],
                                             d["rope_cache"], d["block_table"], d["seq_lens"],
                                             cfg.n_branch, cfg.scale, cfg.out_rescale,
                                             reduce=reduce, **kw)
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


def oracle(inp, reduce="sum"):
    c = inp.cfg
    return mlra_decode(inp.q_latent, inp.q_rope, inp.latent_cache, inp.rope_cache,
                       inp.block_table, inp.seq_lens, c.scale, c.out_rescale, reduce, c.causal,
                       c.block_size)


def assert_parity(out, lse, ref_out, ref_lse, fp32=False):
    assert out.shape == ref_out.shape and lse.shape == ref_lse.shape
    assert not np.isnan(out).any(), "NaN in GPU output"
    err = np.abs(out - ref_out)
    rel = np.linalg.norm(out - ref_out) / max(np.linalg.norm(ref_out), 1e-30)
    assert err.max() <= ATOL, f"max-abs {err.max():.3e}"
    assert rel <= RTOL_L2, f"L2-rel {rel:.3e}"
    if fp32:
        assert err.max() <= 1e-4, f"fp32 max-abs {err.max():.3e}"
    ninf = np.isneginf(ref_lse)
    assert np.array_equal(np.isneginf(lse), ninf), "-inf pattern of lse differs"
    if (~ninf).any():
        lerr = np.abs(lse[~ninf] - ref_lse[~ninf]).max()
        assert lerr <= LSE_ATOL, f"lse max-abs {lerr:.3e}"


def _cfg(**kw):
    base = dict(name="t", num_seqs=3, q_len=1, num_heads=32, n_branch=4, d_latent=128,
                d_rope=64, dtype="bf16", context=None, context_range=(1, 700), seed=21,
                scale=1 / np.sqrt(192), out_rescale=0.5)
    base.update(kw)
    return configs.DecodeConfig(**base)


# Every kernel instance: branches x latent width x RoPE width x row tiles.
SHAPES = []
for nb in (1, 2, 4):
    for dc in (64, 128):
        for dr in (32, 64):
            for h, q in ((16, 1), (24, 2), (24, 4)):
                SHAPES.append((nb, dc, dr, h, q))
SHAPES += [(1, 512, 64, 32, 1), (1, 512, 64, 32, 2), (1, 512, 64, 24, 4), (1, 512, 64, 32, 4)]
SHAPES += [(1, 256, 64, 32, 1), (1, 256, 64, 24, 2), (2, 256, 64, 16, 1), (2, 256, 64, 24, 2),
           (1, 256, 64, 32, 4), (2, 256, 64, 32, 3)]


@pytest.mark.parametrize("nb,dc,dr,h,q", SHAPES)
def test_small_shapes_every_instance(nb, dc, dr, h, q):
    cfg = _cfg(n_branch=nb, d_latent=dc, d_rope=dr, num_heads=h, q_len=q,
               seed=100 + nb * 7 + dc + dr + h + q, scale=1 / np.sqrt(dc + dr))
    inp = make_inputs(cfg)
    for reduce in ("sum", "concat"):
        _say(f"small nb={nb} dc={dc} dr={dr} h={h} q={q} {reduce} lens={inp.seq_lens.tolist()}")
        out, lse = run_gpu(inp, reduce)
        ro, rl = oracle(inp, reduce)
        assert_parity(out, lse, ro, rl)


@pytest.mark.parametrize("cfg", configs.ALL + [configs.MLRA4_TP_SHARE_Q4], ids=lambda c: c.name)
def test_full_size_workloads(cfg):
    _say(f"full {cfg.name}")
    inp = make_inputs(cfg)
    out, lse = run_gpu(inp)
    ro, rl = oracle(inp)
    assert_parity(out, lse, ro, rl, fp32=cfg.dtype == "fp32")


def test_full_size_mla_comparison_call():
    cfg = configs.MLA_COMPARE
    _say(f"full {cfg.name} via mla_decode_attention")
    inp = make_inputs(cfg)
    out, lse = run_gpu(inp, entry="mla")
    ro, rl = oracle(inp)
    assert_parity(out, lse, ro, rl)


def test_full_size_mlra2():
    cfg = configs.MLRA2_FUSED
    _say(f"full {cfg.name}")
    inp = make_inputs(cfg)
    for reduce in ("sum", "concat"):
        out, lse = run_gpu(inp, reduce)
        assert_parity(out, lse, *oracle(inp, reduce))


def oracle_heads_by_branch(inp, heads):
    """Oracle outputs for a sample of heads, one branch at a time.

    Heads and branches are independent in the method, so branch b of heads
    `heads` is the oracle run on the one-branch problem made of branch b's
    latents and queries (host memory then holds one branch in float64).
    Returns (concat out [S][Q][len(heads)][NB][DC], lse [S][Q][len(heads)][NB]).
    """
    c = inp.cfg
    outs, lses = [], []
    for b in range(c.n_branch):
        o, l = mlra_decode(inp.q_latent[:, :, heads, b:b + 1], inp.q_rope[:, :, heads],
                           inp.latent_cache[:, :, b:b + 1], inp.rope_cache, inp.block_table,
                           inp.seq_lens, c.scale, c.out_rescale, "concat", c.causal,
                           c.block_size)
        outs.append(o[:, :, :, 0])
        lses.append(l[:, :, :, 0])
    return np.stack(outs, axis=3), np.stack(lses, axis=3)


@pytest.mark.parametrize("cfg", [configs.MLRA4_B1_T1M, configs.MLRA4_B1_T2M], ids=lambda c: c.name)
def test_single_sequence_million_token_context_sampled_heads(cfg):
    _say(f"{cfg.name}: inputs")
    inp = make_inputs(cfg)
    dev = to_device(inp)
    _say(f"{cfg.name}: GPU sum and concat")
    out_s, lse_s = run_gpu(inp, "sum", dev=dev)
    out_c, lse_c = run_gpu(inp, "concat", dev=dev)
    assert np.array_equal(lse_s, lse_c)
    heads = [0, 11, 31]
    _say(f"{cfg.name}: oracle on heads {heads}, branch by branch")
    ro, rl = oracle_heads_by_branch(inp, heads)
    assert_parity(out_c[:, :, heads], lse_c[:, :, heads], ro, rl)
    assert_parity(out_s[:, :, heads], lse_s[:, :, heads], ro.sum(axis=3), rl)


def test_fp32_path_small_shapes():
    for nb, dc, dr, q in ((1, 256, 64, 2), (2, 512, 32, 1), (4, 64, 32, 2), (2, 128, 64, 3),
                          (1, 64, 32, 4)):
        cfg = _cfg(dtype="fp32", n_branch=nb, d_latent=dc, d_rope=dr, q_len=q, num_heads=5,
                   context_range=(1, 300), seed=dc + nb)
        inp = make_inputs(cfg)
        _say(f"fp32 nb={nb} dc={dc} dr={dr} q={q}")
        for reduce in ("sum", "concat"):
            out, lse = run_gpu(inp, reduce)
            assert_parity(out, lse, *oracle(inp, reduce), fp32=True)


@pytest.mark.parametrize("nb,dc,q", [(1, 128, 1), (4, 128, 1), (1, 512, 1), (4, 128, 2),
                                    (2, 64, 2)])
def test_split_count_invariance(nb, dc, q):
    cfg = _cfg(n_branch=nb, d_latent=dc, num_seqs=2, context=None, context_range=(3000, 5000),
               q_len=q, seed=5 + nb + 10 * q)
    inp = make_inputs(cfg)
    ro, rl = oracle(inp)
    dev = to_device(inp)
    for ns in (1, 2, 7, 0, 79):
        _say(f"splits nb={nb} dc={dc} q={q} num_splits={ns}")
        out, lse = run_gpu(inp, num_splits=ns, dev=dev)
        assert_parity(out, lse, ro, rl)


@pytest.mark.parametrize("nb,dc,q", [(4, 128, 1), (2, 256, 1), (1, 512, 2)])
def test_block_relabelling_and_determinism_are_bitwise(nb, dc, q):
    # 256/512-wide latents also sum their slices' partial scores through LDS
    cfg = _cfg(num_seqs=4, context_range=(100, 2000), seed=77, n_branch=nb, d_latent=dc, q_len=q,
               scale=1 / np.sqrt(dc + 64))
    inp = make_inputs(cfg)
    _say(f"determinism nb={nb} dc={dc} q={q}")
    a = run_gpu(inp)
    b = run_gpu(inp)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    perm = np.random.default_rng(1).permutation(inp.num_blocks)
    inp2 = make_inputs(cfg)
    inp2.latent_cache[perm] = inp.latent_cache
    inp2.rope_cache[perm] = inp.rope_cache
    inp2.block_table = perm[inp.block_table].astype(np.int32)
    _say("relabelled blocks")
    c = run_gpu(inp2)
    assert np.array_equal(a[0], c[0]) and np.array_equal(a[1], c[1])


@pytest.mark.parametrize("q", [1, 2])
def test_fused_equals_sum_of_single_branch_shares(q):
    # with 64 query rows the fused call splits the branches over two
    # workgroups per split, a single-branch share holds both row tiles
    cfg = _cfg(num_seqs=2, context_range=(500, 1500), seed=9, q_len=q)
    inp = make_inputs(cfg)
    _say(f"fused vs single-branch shares q={q}")
    fused, lse_f = run_gpu(inp)
    d = to_device(inp)
    acc = 0
    for b in range(4):
        share = dict(d)
        share["q_latent"] = d["q_latent"][:, :, :, b:b + 1].contiguous()
        share["latent_cache"] = d["latent_cache"][:, :, b:b + 1]
        one = inp.cfg.with_(n_branch=1)
        inp_b = make_inputs(cfg)
        inp_b.cfg = one
        o, l = run_gpu(inp_b, dev=share)
        acc = acc + o
        np.testing.assert_allclose(l[..., 0], lse_f[..., b], atol=2e-5)
    assert np.abs(acc - fused).max() <= 2e-2
    assert np.linalg.norm(acc - fused) / np.linalg.norm(fused) <= 1e-2


@pytest.mark.parametrize("q,nb,dc", [(1, 4, 128), (2, 4, 128), (1, 2, 256), (2, 2, 256)])
def test_branch_major_cache_strides(q, nb, dc):
    cfg = _cfg(num_seqs=2, context_range=(64, 900), seed=13, q_len=q, n_branch=nb, d_latent=dc,
               scale=1 / np.sqrt(dc + 64))
    inp = make_inputs(cfg)
    d = to_device(inp)
    # same values stored branch-major [blocks][NB][64][DC], viewed as [blocks][64][NB][DC]
    bm = d["latent_cache"].permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3)
    assert bm.stride(2) == 64 * cfg.d_latent
    d["latent_cache"] = bm
    _say(f"branch-major strides q={q} nb={nb} dc={dc}")
    out, lse = run_gpu(inp, dev=d)
    assert_parity(out, lse, *oracle(inp))


def test_empty_and_degenerate_sequences():
    cfg = _cfg(q_len=2, num_seqs=5, context=130, context_range=None, seed=4)
    inp = make_inputs(cfg)
    inp.seq_lens[:] = [0, 1, 2, 64, 130]
    _say("degenerate lengths")
    out, lse = run_gpu(inp)
    ro, rl = oracle(inp)
    assert_parity(out, lse, ro, rl)
    assert np.all(out[0] == 0) and np.all(np.isneginf(lse[0]))
    assert np.all(out[1, 0] == 0) and np.all(np.isneginf(lse[1, 0]))
    inp.seq_lens[:] = 0
    out, lse = run_gpu(inp, hint=False)
    assert np.all(out == 0) and np.all(np.isneginf(lse))


def test_seq_len_above_max_is_clamped_not_read_out_of_bounds():
    cfg = _cfg(num_seqs=2, context=256, context_range=None, seed=3)
    inp = make_inputs(cfg)
    d = to_device(inp)
    d["seq_lens"] = torch.tensor([10_000, 256], dtype=torch.int32, device="cuda")
    _say("over-long seq_lens clamp")
    out, lse = api.mlra_decode_attention(d["q_latent"], d["q_rope"], d["latent_cache"],
                                         d["rope_cache"], d["block_table"], d["seq_lens"], 4,
                                         cfg.scale, cfg.out_rescale, max_seq_len=256)
    torch.cuda.synchronize()
    ro, rl = oracle(inp)
    assert_parity(out.float().cpu().numpy().astype(np.float64), lse.cpu().numpy(), ro, rl)


@pytest.mark.parametrize("num_splits", [0, 40, 200])
def test_workspace_contents_are_never_read_before_written(num_splits):
    # Ragged lengths leave split slots of short sequences unwritten. With many
    # splits over a few (sequence, row) pairs the column-sliced combine runs
    # (16- and 8-column slices); with the library's plan the per-row one.
    # Poisoned workspaces must not leak into the output.
    cfg = _cfg(num_seqs=2, context_range=(100, 30000), seed=41)
    inp = make_inputs(cfg)
    d = to_device(inp)
    args = (d["q_latent"], d["q_rope"], d["latent_cache"], d["rope_cache"], d["block_table"],
            d["seq_lens"], cfg.n_branch)
    kw = dict(max_seq_len=inp.max_seq_len, num_splits=num_splits)
    dims = api.make_dims(d["q_latent"], d["q_rope"], d["latent_cache"], d["rope_cache"],
                         d["block_table"], **kw)
    nbytes = api.make_plan(dims, cfg.n_branch).workspace_bytes
    ro, rl = oracle(inp)
    results = []
    for fill in (float("nan"), float("inf"), -float("inf")):
        # the header (status word, merge counters) starts at zero; everything
        # after it is poisoned
        ws = torch.full((nbytes // 4,), fill, dtype=torch.float32, device="cuda")
        ws[: _lib.MLRA_DECODE_WS_HEADER_BYTES // 4] = 0
        _say(f"poisoned workspace {fill} num_splits={num_splits}")
        o, l = api.mlra_decode_attention(*args, cfg.scale, cfg.out_rescale, workspace=ws, **kw)
        torch.cuda.synchronize()
        results.append((o.clone(), l.clone()))
        assert_parity(o.float().cpu().numpy().astype(np.float64),
                      l.cpu().numpy().astype(np.float64), ro, rl)
    for o, l in results[1:]:
        assert torch.equal(o, results[0][0]) and torch.equal(l, results[0][1])


def test_two_phase_and_prepared_calls_match_the_single_call_bitwise():
    cfg = _cfg(num_seqs=3, context_range=(100, 3000), seed=31)
    inp = make_inputs(cfg)
    d = to_device(inp)
    args = (d["q_latent"], d["q_rope"], d["latent_cache"], d["rope_cache"], d["block_table"],
            d["seq_lens"], cfg.n_branch)
    kw = dict(max_seq_len=inp.max_seq_len, sum_seq_lens=int(inp.seq_lens.sum()))
    _say("single call vs partials+combine vs prepared")
    o1, l1 = api.mlra_decode_attention(*args, cfg.scale, cfg.out_rescale, **kw)
    o1, l1 = o1.clone(), l1.clone()
    ws = api.mlra_decode_partials(*args, cfg.scale, **kw)
    o2, l2 = api.mlra_decode_combine(*args, cfg.out_rescale, workspace=ws, **kw)
    prep = api.PreparedDecode(*args, cfg.scale, cfg.out_rescale, **kw)
    prep.out.zero_()
    prep.partials()
    o3, l3 = (t.clone() for t in prep.combine())
    prep.out.zero_()
    o4, l4 = prep.run(d["block_table"].clone())
    torch.cuda.synchronize()
    for o, l in ((o2, l2), (o3, l3), (o4, l4)):
        assert torch.equal(o, o1) and torch.equal(l, l1)
    assert_parity(o1.float().cpu().numpy().astype(np.float64),
                  l1.cpu().numpy().astype(np.float64), *oracle(inp))


def _random_case(rng, i):
    """One seeded random decode case over the supported shape space: branches
    and latent width (with their RoPE widths), heads and up to 4 query tokens
    (up to 128 rows), ragged lengths including empty and single-token sequences, causal or
    not, and an explicit split count or the planner's."""
    nb, dc, dr = [(1, 64, 32), (1, 128, 64), (2, 64, 64), (2, 128, 32), (4, 64, 32),
                  (4, 128, 64), (1, 256, 64), (2, 256, 64), (1, 512, 64)][rng.integers(9)]
    q = int(rng.integers(1, 5))
    h = int(rng.integers(1, 128 // q + 1))
    s = int(rng.integers(1, 6))
    hi = int(rng.integers(1, 1500))
    cfg = _cfg(name=f"rand{i}", n_branch=nb, d_latent=dc, d_rope=dr, num_heads=h, q_len=q,
               num_seqs=s, context_range=(1, hi), causal=bool(rng.integers(2)),
               seed=1000 + i, scale=1 / np.sqrt(dc + dr), out_rescale=float(rng.uniform(0.3, 1.0)))
    inp = make_inputs(cfg)
    if s > 1 and rng.integers(3) == 0:
        inp.seq_lens[int(rng.integers(s))] = 0  # an empty sequence
    splits = int(rng.choice([0, 0, 1, 3, 17]))
    return inp, splits


@pytest.mark.parametrize("i", range(24))
def test_random_shapes_match_the_oracle(i):
    inp, splits = _random_case(np.random.default_rng(4242 + i), i)
    c = inp.cfg
    reduce = "concat" if i % 3 == 0 else "sum"
    _say(f"random {i}: nb={c.n_branch} dc={c.d_latent} dr={c.d_rope} h={c.num_heads} q={c.q_len} "
         f"causal={c.causal} {reduce} splits={splits} lens={inp.seq_lens.tolist()}")
    out, lse = run_gpu(inp, reduce, num_splits=splits)
    assert_parity(out, lse, *oracle(inp, reduce))


@pytest.mark.parametrize("nb", [1, 4])
def test_four_query_tokens_mid_size(nb):
    # speculative-style verification of four new tokens per sequence: 128
    # rows, four row tiles per workgroup (one branch) or four branch groups
    # per split (four branches)
    cfg = _cfg(num_seqs=4, q_len=4, num_heads=32, n_branch=nb, context_range=(1200, 3000),
               seed=60 + nb)
    inp = make_inputs(cfg)
    dev = to_device(inp)
    for reduce in ("sum", "concat"):
        _say(f"four tokens nb={nb} {reduce} lens={inp.seq_lens.tolist()}")
        out, lse = run_gpu(inp, reduce, dev=dev)
        assert_parity(out, lse, *oracle(inp, reduce))
