"""HIP-graph capture of the decode and prefill calls (GPU).

A captured call is replayed several times, with the program's own eager work
(overwriting the outputs) and synchronisations between replays; every replay
must reproduce the eager call's outputs bit for bit, and the eager call must
match the float64 oracle. The calls enqueue no memset and allocate nothing,
so they are safe to capture.
"""
import numpy as np
import pytest
import torch

from latent_kv_cache_amd import api, configs
from latent_kv_cache_amd.inputs import make_inputs, to_device
from oracle import mlra_decode

pytestmark = pytest.mark.gpu


def _say(msg):
    print(f"[gpu-case] {msg}", flush=True)


def _check_oracle(inp, out, lse, reduce="sum"):
    c = inp.cfg
    ro, rl = mlra_decode(inp.q_latent, inp.q_rope, inp.latent_cache, inp.rope_cache,
                         inp.block_table, inp.seq_lens, c.scale, c.out_rescale, reduce, c.causal,
                         c.block_size)
    got = out.float().cpu().numpy().astype(np.float64)
    assert np.abs(got - ro).max() <= 2e-2
    assert np.linalg.norm(got - ro) / np.linalg.norm(ro) <= 1e-2
    fin = np.isfinite(rl)
    assert np.abs(lse.cpu().numpy()[fin] - rl[fin]).max() <= 1e-3


def _replay_matches(graph, out, lse, ref_out, ref_lse, times=4):
    for r in range(times):
        out.fill_(float("nan"))  # eager work between replays
        lse.fill_(0.0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref_out) and torch.equal(lse, ref_lse), f"replay {r} differs"


@pytest.mark.parametrize("cfg", [configs.MLRA4_TP_SHARE.with_(name="g_share", num_seqs=4, context=3000),
                                 configs.MLRA4_FUSED.with_(name="g_fused", num_seqs=2, context=2500),
                                 configs.MLRA2_FUSED.with_(name="g_mlra2", num_seqs=2, context=2000),
                                 configs.MLA_COMPARE.with_(name="g_mla", num_seqs=2, context=1800)],
                         ids=lambda c: c.name)
def test_decode_graph_replays_match_eager(cfg):
    inp = make_inputs(cfg)
    d = to_device(inp)
    S, Q, H, NB, DC = inp.q_latent.shape
    out = torch.empty((S, Q, H, DC), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((S, Q, H, NB), dtype=torch.float32, device="cuda")
    prep = api.PreparedDecode(d["q_latent"], d["q_rope"], d["latent_cache"], d["rope_cache"],
                              d["block_table"], d["seq_lens"], NB, cfg.scale, cfg.out_rescale,
                              max_seq_len=inp.max_seq_len, out=out, lse=lse)
    _say(f"graph decode {cfg.name}")
    prep.run()
    torch.cuda.synchronize()
    _check_oracle(inp, out, lse)
    ref_out, ref_lse = out.clone(), lse.clone()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        prep.run(stream=torch.cuda.current_stream().cuda_stream)
    _replay_matches(graph, out, lse, ref_out, ref_lse)


@pytest.mark.parametrize("n_branch,reduce", [(1, "sum"), (2, "sum")])
def test_prefill_graph_replays_match_eager(n_branch, reduce):
    cfg = configs.MLRA4_TP_PREFILL.with_(name="g_prefill", num_seqs=2, q_len=48, num_heads=16,
                                         n_branch=n_branch, context=700)
    inp = make_inputs(cfg)
    d = to_device(inp)
    S, Q, H, NB, DC = inp.q_latent.shape
    out = torch.empty((S, Q, H, DC), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((S, Q, H, NB), dtype=torch.float32, device="cuda")
    dims = api.make_dims(d["q_latent"], d["q_rope"], d["latent_cache"], d["rope_cache"],
                         d["block_table"], max_seq_len=inp.max_seq_len, reduce=reduce)
    plan = api.make_prefill_plan(dims, NB)
    ws = torch.empty(max(plan.workspace_bytes, 256), dtype=torch.uint8, device="cuda")

    def call(stream=None):
        api.mlra_prefill_attention(d["q_latent"], d["q_rope"], d["latent_cache"], d["rope_cache"],
                                   d["block_table"], d["seq_lens"], NB, cfg.scale, cfg.out_rescale,
                                   max_seq_len=inp.max_seq_len, reduce=reduce, out=out, lse=lse,
                                   workspace=ws, stream=stream)

    _say(f"graph prefill nb={n_branch} {reduce} splits={plan.splits_per_seq}")
    call()
    torch.cuda.synchronize()
    _check_oracle(inp, out, lse, reduce)
    ref_out, ref_lse = out.clone(), lse.clone()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call(stream=torch.cuda.current_stream().cuda_stream)
    _replay_matches(graph, out, lse, ref_out, ref_lse)
