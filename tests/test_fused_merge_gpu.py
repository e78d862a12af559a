"""GPU tests of the split kernel's in-kernel merge (no combine launch).

The merge is asked for with MLRA_DECODE_FLAG_FUSED_MERGE and taken when the
batch is a multiple of 8 sequences, at most 64, and the whole call fits one
round of one workgroup per CU; each sequence's
workgroups then run on one XCD and merge their partial results through its
L2 (include/mlra.h, mlra_decode_attention). Checked here: parity with the
float64 oracle over the shapes the merge serves (branches, latent widths,
query tokens, SUM and CONCAT, causal), agreement with the two-kernel path,
bitwise repeatability, sequences shorter than the plan's bound (workgroups
with no tokens of their own), a clean status word, and recovery after calls
whose waits are made to expire from the host.
"""
import ctypes

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


def _oracle(inp, reduce):
    c = inp.cfg
    return mlra_decode(inp.q_latent, inp.q_rope, inp.latent_cache, inp.rope_cache,
                       inp.block_table, inp.seq_lens, c.scale, c.out_rescale, reduce, c.causal,
                       c.block_size)


def _parity(out, lse, ro, rl):
    out = out.float().cpu().numpy().astype(np.float64)
    lse = lse.cpu().numpy().astype(np.float64)
    assert not np.isnan(out).any(), "NaN in output"
    err = np.abs(out - ro)
    assert err.max() <= ATOL, f"max-abs {err.max():.3e}"
    assert np.linalg.norm(out - ro) / np.linalg.norm(ro) <= RTOL_L2
    fin = np.isfinite(rl)
    assert np.array_equal(np.isneginf(lse), np.isneginf(rl))
    assert np.abs(lse[fin] - rl[fin]).max() <= LSE_ATOL


def _call(inp, d, reduce, fused=True, ws=None, hint=True):
    c = inp.cfg
    return api.mlra_decode_attention(
        d["q_latent"], d["q_rope"], d["latent_cache"], d["rope_cache"], d["block_table"],
        d["seq_lens"], c.n_branch, c.scale, c.out_rescale, max_seq_len=inp.max_seq_len,
        reduce=reduce, causal=c.causal, sum_seq_lens=int(inp.seq_lens.sum()) if hint else 0,
        workspace=ws, fused_merge=fused)


def _plan(inp, d, reduce, hint=True):
    dims = api.make_dims(d["q_latent"], d["q_rope"], d["latent_cache"], d["rope_cache"],
                         d["block_table"], max_seq_len=inp.max_seq_len, reduce=reduce,
                         causal=inp.cfg.causal,
                         sum_seq_lens=int(inp.seq_lens.sum()) if hint else 0, fused_merge=True)
    return api.make_plan(dims, inp.cfg.n_branch)


SHARE = configs.MLRA4_TP_SHARE
CASES = [
    (SHARE.with_(name="fm_share_b8", num_seqs=8, context=3000, seed=51), "sum"),
    (SHARE.with_(name="fm_share_b16_q2", num_seqs=16, q_len=2, context=2100, seed=52), "sum"),
    (SHARE.with_(name="fm_share_b8_q4", num_seqs=8, q_len=4, context=1500, seed=53), "sum"),
    (SHARE.with_(name="fm_share_b8_h20", num_seqs=8, num_heads=20, context=1900, seed=54), "sum"),
    (configs.MLRA4_FUSED.with_(name="fm_fused_b8", num_seqs=8, context=2600, seed=55), "sum"),
    (configs.MLRA4_FUSED.with_(name="fm_fused_b8_cat", num_seqs=8, context=2600, seed=56), "concat"),
    (configs.MLRA4_FUSED.with_(name="fm_fused_b8_q2", num_seqs=8, q_len=2, context=1800, seed=57), "sum"),
    (configs.MLRA2_FUSED.with_(name="fm_mlra2_b8", num_seqs=8, context=2000, seed=58), "concat"),
    (configs.MLA_COMPARE.with_(name="fm_mla_b8", num_seqs=8, context=1700, seed=59), "sum"),
    (SHARE.with_(name="fm_share_b8_dc64", num_seqs=8, d_latent=64, d_rope=32, context=2500,
                 seed=60), "sum"),
]


@pytest.mark.parametrize("cfg,reduce", CASES, ids=lambda c: getattr(c, "name", c))
def test_fused_merge_matches_oracle_and_two_kernel_path(cfg, reduce):
    inp = make_inputs(cfg)
    d = to_device(inp)
    plan = _plan(inp, d, reduce)
    assert plan.fused_merge == 1, "shape should take the in-kernel merge"
    _say(f"fused merge {cfg.name} {reduce}")
    ws = api.new_workspace("cuda", plan.workspace_bytes)
    o1, l1 = _call(inp, d, reduce, ws=ws)
    o1, l1 = o1.clone(), l1.clone()
    o2, l2 = _call(inp, d, reduce, ws=ws)          # repeat: bit for bit
    o3, l3 = _call(inp, d, reduce, fused=False)    # the combine kernel
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2), "not repeatable"
    _parity(o1, l1, *_oracle(inp, reduce))
    assert (o1.float() - o3.float()).abs().max().item() <= 2e-2
    fin = torch.isfinite(l3)
    assert torch.equal(torch.isneginf(l1), torch.isneginf(l3))
    assert (l1[fin] - l3[fin]).abs().max().item() <= 1e-4
    assert api.read_status(ws) == 0


def test_sequences_shorter_than_the_bound():
    # No length hint: the plan splits max_seq_len, so the short sequences'
    # last splits have no tokens and their workgroups merge without a partial
    # of their own (one of them is the empty sequence).
    cfg = SHARE.with_(name="fm_ragged", num_seqs=8, context=None, context_range=(1, 6000), seed=61)
    inp = make_inputs(cfg)
    inp.seq_lens[3] = 0
    d = to_device(inp)
    plan = _plan(inp, d, "sum", hint=False)
    assert plan.fused_merge == 1 and plan.splits_per_seq > 1
    _say("fused merge, sequences shorter than the bound")
    ws = api.new_workspace("cuda", plan.workspace_bytes)
    out, lse = _call(inp, d, "sum", ws=ws, hint=False)
    torch.cuda.synchronize()
    ro, rl = _oracle(inp, "sum")
    _parity(out, lse, ro, rl)
    assert api.read_status(ws) == 0


def test_headline_shape_uses_the_merge_and_matches_oracle_rows():
    cfg = SHARE
    inp = make_inputs(cfg)
    d = to_device(inp)
    plan = _plan(inp, d, "sum")
    assert plan.fused_merge == 1
    _say("fused merge at B=16, T=8192")
    ws = api.new_workspace("cuda", plan.workspace_bytes)
    out, lse = _call(inp, d, "sum", ws=ws)
    o2, l2 = _call(inp, d, "sum", fused=False)
    torch.cuda.synchronize()
    assert (out.float() - o2.float()).abs().max().item() <= 2e-2
    assert (lse - l2).abs().max().item() <= 1e-4
    # oracle on three sequences
    sub = [0, 7, 15]
    ro, rl = mlra_decode(inp.q_latent[sub], inp.q_rope[sub], inp.latent_cache, inp.rope_cache,
                         inp.block_table[sub], inp.seq_lens[sub], cfg.scale, cfg.out_rescale,
                         "sum", cfg.causal, cfg.block_size)
    _parity(out[sub], lse[sub], ro, rl)
    assert api.read_status(ws) == 0


def test_expired_waits_are_reported_and_the_next_call_recovers():
    # Waits made to expire from the host (a bound of 0 polls and 0 ticks):
    # the kernel still ends, the status word reports it, and because every
    # workgroup still publishes its counter once, the next normal call on the
    # same workspace is correct.
    cfg = SHARE.with_(name="fm_expire", num_seqs=8, context=2000, seed=62)
    inp = make_inputs(cfg)
    d = to_device(inp)
    plan = _plan(inp, d, "sum")
    assert plan.fused_merge == 1
    lib = _lib.load()
    ws = api.new_workspace("cuda", plan.workspace_bytes)
    try:
        lib.mlra_testing_set_wait_limit(0)
        _say("fused merge with expiring waits")
        _call(inp, d, "sum", ws=ws)
        torch.cuda.synchronize()
    finally:
        lib.mlra_testing_set_wait_limit(-1)
    bits = api.read_status(ws, clear=True)
    assert bits & (_lib.MLRA_DEVSTATUS_WAIT_EXPIRED | _lib.MLRA_DEVSTATUS_MERGE_FAILED), bits
    assert api.read_status(ws) == 0
    _say("fused merge after the expired call")
    out, lse = _call(inp, d, "sum", ws=ws)
    torch.cuda.synchronize()
    _parity(out, lse, *_oracle(inp, "sum"))
    assert api.read_status(ws) == 0


def test_workspace_init_zeroes_the_header():
    cfg = SHARE.with_(name="fm_init", num_seqs=8, context=1000, seed=63)
    inp = make_inputs(cfg)
    d = to_device(inp)
    plan = _plan(inp, d, "sum")
    ws = torch.full((plan.workspace_bytes,), 0x5A, dtype=torch.uint8, device="cuda")
    lib = _lib.load()
    _lib.check(lib.mlra_decode_workspace_init(ws.data_ptr(), ws.numel(),
                                              torch.cuda.current_stream().cuda_stream),
               "mlra_decode_workspace_init")
    torch.cuda.synchronize()
    assert int(ws[: _lib.MLRA_DECODE_WS_HEADER_BYTES].max().item()) == 0
    assert int(ws[_lib.MLRA_DECODE_WS_HEADER_BYTES:].min().item()) == 0x5A
    _say("fused merge on an initialised workspace")
    out, lse = _call(inp, d, "sum", ws=ws)
    torch.cuda.synchronize()
    _parity(out, lse, *_oracle(inp, "sum"))


def test_fused_call_in_a_graph_replays_bitwise():
    cfg = configs.MLRA4_FUSED.with_(name="fm_graph", num_seqs=8, context=2000, seed=64)
    inp = make_inputs(cfg)
    d = to_device(inp)
    S, Q, H, NB, DC = inp.q_latent.shape
    out = torch.empty((S, Q, H, DC), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((S, Q, H, NB), dtype=torch.float32, device="cuda")
    prep = api.PreparedDecode(d["q_latent"], d["q_rope"], d["latent_cache"], d["rope_cache"],
                              d["block_table"], d["seq_lens"], NB, cfg.scale, cfg.out_rescale,
                              max_seq_len=inp.max_seq_len, out=out, lse=lse, fused_merge=True)
    assert prep.plan.fused_merge == 1
    _say("fused merge in a HIP graph")
    prep.run()
    torch.cuda.synchronize()
    _parity(out, lse, *_oracle(inp, "sum"))
    ref_out, ref_lse = out.clone(), lse.clone()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        prep.run(stream=torch.cuda.current_stream().cuda_stream)
    for r in range(4):
        out.fill_(float("nan"))
        lse.fill_(0.0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref_out) and torch.equal(lse, ref_lse), f"replay {r}"
    assert api.read_status(prep.workspace) == 0


def test_many_calls_keep_the_counters_level():
    # Every call advances each of a sequence's counter slots by one: after n
    # calls on a fresh workspace every slot holds count n and this XCD's id,
    # and no call waited out its bound (each stays far below the bound).
    cfg = SHARE.with_(name="fm_many", num_seqs=8, context=1200, seed=65)
    inp = make_inputs(cfg)
    d = to_device(inp)
    plan = _plan(inp, d, "sum")
    assert plan.fused_merge == 1
    ws = api.new_workspace("cuda", plan.workspace_bytes)
    n = 80
    _say(f"fused merge, {n} calls on one workspace")
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(n):
        out, lse = _call(inp, d, "sum", ws=ws)
    stop.record()
    torch.cuda.synchronize()
    assert start.elapsed_time(stop) / n < 5.0, "calls ran into the merge's wait bound"
    _parity(out, lse, *_oracle(inp, "sum"))
    assert api.read_status(ws) == 0
    hdr = ws[256: 256 + cfg.num_seqs * 1024].view(torch.int64).view(cfg.num_seqs, 128).cpu()
    per = plan.splits_per_seq * plan.row_groups
    for s in range(cfg.num_seqs):
        flags, verd = hdr[s, :32], hdr[s, 32:64]
        assert ((flags >> 8) == n).all(), (s, flags >> 8)
        assert ((verd >> 2) == n).all() and ((verd[:per] & 3) == 1).all()
        assert len(set((flags[:per] & 255).tolist())) == 1   # one XCD per sequence
