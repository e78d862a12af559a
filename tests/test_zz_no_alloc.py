"""The allocation-free decode entry point, through the C ABI (GPU).

mlra_decode_attention_static is mlra_decode_attention with the library's own
device scratch (a fixed array in its code object, looked up per device) in
place of a workspace. Two calls in a row on the same scratch, the second with
a smaller input, must give exactly what the workspace entry point gives for
the same inputs (same kernels and plan), and meet the oracle's bar; a plan
larger than the scratch is refused on the host.
"""
import ctypes

import numpy as np
import pytest
import torch

from latent_kv_cache_amd import _lib, api, configs
from latent_kv_cache_amd.inputs import make_inputs, to_device
from oracle import mlra_decode

pytestmark = pytest.mark.gpu


def _say(msg):
    print(f"[gpu-case] {msg}", flush=True)


def _both_entries(cfg, flags=0):
    inp = make_inputs(cfg)
    d = to_device(inp)
    S, Q, H, NB, DC = inp.q_latent.shape
    dims = api.make_dims(d["q_latent"], d["q_rope"], d["latent_cache"], d["rope_cache"],
                         d["block_table"], max_seq_len=inp.max_seq_len, causal=cfg.causal,
                         sum_seq_lens=int(inp.seq_lens.sum()))
    dims.flags = flags
    lib = _lib.load()
    stream = torch.cuda.current_stream().cuda_stream
    ptrs = [d[k].data_ptr() for k in ("q_latent", "q_rope", "latent_cache", "rope_cache",
                                      "block_table", "seq_lens")]
    outs = []
    for entry in ("mlra_decode_attention", "mlra_decode_attention_static"):
        out = torch.full((S, Q, H, DC), float("nan"), dtype=torch.bfloat16, device="cuda")
        lse = torch.full((S, Q, H, NB), float("nan"), dtype=torch.float32, device="cuda")
        if entry == "mlra_decode_attention":
            size = ctypes.c_size_t(0)
            _lib.check(lib.mlra_decode_workspace_size(dims, NB, ctypes.byref(size)), "size")
            ws = api.new_workspace("cuda", size.value)
            st = lib.mlra_decode_attention(*ptrs, NB, cfg.scale, cfg.out_rescale, out.data_ptr(),
                                           lse.data_ptr(), dims, ws.data_ptr(), ws.numel(), stream)
        else:
            st = lib.mlra_decode_attention_static(*ptrs, NB, cfg.scale, cfg.out_rescale,
                                                  out.data_ptr(), lse.data_ptr(), dims, stream)
        _lib.check(st, entry)
        torch.cuda.synchronize()
        outs.append((out, lse))
    return inp, outs


def _oracle_bar(inp, out, lse):
    c = inp.cfg
    ro, rl = mlra_decode(inp.q_latent, inp.q_rope, inp.latent_cache, inp.rope_cache,
                         inp.block_table, inp.seq_lens, c.scale, c.out_rescale, "sum", c.causal,
                         c.block_size)
    got = out.float().cpu().numpy().astype(np.float64)
    assert not np.isnan(got).any()
    assert np.abs(got - ro).max() <= 2e-2
    assert np.linalg.norm(got - ro) / np.linalg.norm(ro) <= 1e-2
    fin = np.isfinite(rl)
    assert np.abs(lse.cpu().numpy()[fin] - rl[fin]).max() <= 1e-3


def test_static_entry_matches_the_workspace_entry_on_two_calls():
    first = configs.MLRA4_FUSED.with_(name="noalloc_b8", num_seqs=8, context=5000, seed=71)
    second = configs.MLRA4_FUSED.with_(name="noalloc_b3", num_seqs=3, context=1300, seed=72)
    for cfg in (first, second):       # the second call is smaller, on the same scratch
        _say(f"static entry {cfg.name}")
        inp, ((o1, l1), (o2, l2)) = _both_entries(cfg)
        assert torch.equal(o1, o2) and torch.equal(l1, l2), cfg.name
        _oracle_bar(inp, o2, l2)


def test_static_entry_with_the_in_kernel_merge():
    # the merge's counters live in the scratch's header, which starts at zero
    # and is left ready by every call
    for i, cfg in enumerate((configs.MLRA4_TP_SHARE.with_(name="noalloc_fm16", num_seqs=16,
                                                          context=2000, seed=73),
                             configs.MLRA4_TP_SHARE.with_(name="noalloc_fm8", num_seqs=8,
                                                          context=900, seed=74))):
        _say(f"static entry, in-kernel merge {cfg.name}")
        inp, ((o1, l1), (o2, l2)) = _both_entries(cfg, flags=_lib.MLRA_DECODE_FLAG_FUSED_MERGE)
        assert torch.equal(o1, o2) and torch.equal(l1, l2), cfg.name
        _oracle_bar(inp, o2, l2)


def test_static_entry_refuses_a_plan_larger_than_the_scratch():
    # 8 sequences of 65536 tokens, 4 query tokens, four branches, 64 forced
    # splits: the plan needs 135 MB of partials, more than the scratch. Valid
    # (zero-filled) device tensors of the stated shapes, so that nothing could
    # be read out of bounds even if a launch happened.
    S, Q, H, NB, DC, DR, L = 8, 4, 32, 4, 128, 64, 65536
    nblk = L // 64
    dev = "cuda"
    q = torch.zeros((S, Q, H, NB, DC), dtype=torch.bfloat16, device=dev)
    qr = torch.zeros((S, Q, H, DR), dtype=torch.bfloat16, device=dev)
    lat = torch.zeros((S * nblk, 64, NB, DC), dtype=torch.bfloat16, device=dev)
    rope = torch.zeros((S * nblk, 64, DR), dtype=torch.bfloat16, device=dev)
    table = torch.arange(S * nblk, dtype=torch.int32, device=dev).view(S, nblk)
    lens = torch.full((S,), L, dtype=torch.int32, device=dev)
    dims = api.make_dims(q, qr, lat, rope, table, max_seq_len=L, num_splits=64)
    plan = api.make_plan(dims, NB)
    assert plan.workspace_bytes > _lib.MLRA_STATIC_SCRATCH_BYTES
    out = torch.empty((S, Q, H, DC), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((S, Q, H, NB), dtype=torch.float32, device=dev)
    lib = _lib.load()
    _say("static entry, plan larger than the scratch")
    st = lib.mlra_decode_attention_static(q.data_ptr(), qr.data_ptr(), lat.data_ptr(),
                                          rope.data_ptr(), table.data_ptr(), lens.data_ptr(), NB,
                                          0.07, 0.5, out.data_ptr(), lse.data_ptr(), dims,
                                          torch.cuda.current_stream().cuda_stream)
    assert st == 4  # MLRA_ERR_WORKSPACE, nothing enqueued
