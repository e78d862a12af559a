"""GPU parity of the cache append (mlra_cache_append) against the float64 oracle.

Bar: the latent rows written equal the oracle's exactly (the product of two
floats is exact in double and both sides round it once); rotated key values
equal the oracle's or differ by one unit in the last place of the cache dtype
(the sine and cosine come from different libraries); every cache element the
append does not write is bit-identical to what it held, NaN poison included.
"""
import numpy as np
import pytest
import torch

from latent_kv_cache_amd import api, configs
from latent_kv_cache_amd.inputs import make_append_inputs, make_inputs, to_device
from oracle import cache_append, mlra_decode, round_to_bf16_f64

pytestmark = pytest.mark.gpu


def _say(msg):
    print(f"[gpu-case] {msg}", flush=True)


def _ulp(x, dtype):
    mant = 8 if dtype == "bf16" else 24
    _, e = np.frexp(np.where(x == 0, 1.0, x))
    return np.ldexp(1.0, e - mant)


def _check(cfg, got_lat, got_rope, ref_lat, ref_rope, old_lat, old_rope):
    # untouched elements: bit-identical (NaN where NaN)
    touched = ~((ref_lat == old_lat) | (np.isnan(ref_lat) & np.isnan(old_lat)))
    assert np.array_equal(got_lat[~touched], old_lat[~touched], equal_nan=True)
    assert np.array_equal(got_lat, ref_lat, equal_nan=True), "latent rows differ"
    diff = np.abs(got_rope - ref_rope)
    both_nan = np.isnan(got_rope) & np.isnan(ref_rope)
    diff[both_nan] = 0.0
    assert not np.isnan(diff).any(), "NaN mismatch in the rope cache"
    bad = diff > _ulp(np.abs(ref_rope), cfg.dtype)
    assert not bad.any(), f"{bad.sum()} rope values beyond one ulp"
    changed_rows = touched.any(axis=(2, 3))
    return int(changed_rows.sum()), int((diff > 0).sum())


def _run(cfg, latent_scale=0.75, rope_base=10000.0, seq_lens=None, table=None):
    inp = make_inputs(cfg)
    lat_new, rope_new = make_append_inputs(cfg)
    d = to_device(inp)
    if seq_lens is not None:
        inp.seq_lens = np.asarray(seq_lens, dtype=np.int32)
        d["seq_lens"] = torch.from_numpy(inp.seq_lens).cuda()
    if table is not None:
        inp.block_table = np.asarray(table, dtype=np.int32)
        d["block_table"] = torch.from_numpy(inp.block_table).cuda()
    api.mlra_cache_append(torch.from_numpy(lat_new).cuda(), torch.from_numpy(rope_new).cuda(),
                          d["latent_cache"], d["rope_cache"], d["block_table"], d["seq_lens"],
                          np.float32(latent_scale), rope_base)
    torch.cuda.synchronize()
    got_lat = d["latent_cache"].float().cpu().numpy().astype(np.float64)
    got_rope = d["rope_cache"].float().cpu().numpy().astype(np.float64)
    ref_lat, ref_rope = cache_append(lat_new, rope_new, inp.latent_cache, inp.rope_cache,
                                     inp.block_table, inp.seq_lens, float(np.float32(latent_scale)),
                                     float(np.float32(rope_base)), cfg.block_size,
                                     to_bf16=cfg.dtype == "bf16")
    if cfg.dtype == "fp32":   # the float32 cache holds the nearest float
        ref_lat = ref_lat.astype(np.float32).astype(np.float64)
        ref_rope = ref_rope.astype(np.float32).astype(np.float64)
    return _check(cfg, got_lat, got_rope, ref_lat, ref_rope,
                  inp.latent_cache.astype(np.float64), inp.rope_cache.astype(np.float64)), inp


def _cfg(**kw):
    base = dict(name="a", num_seqs=5, q_len=2, num_heads=1, n_branch=4, d_latent=128,
                d_rope=64, dtype="bf16", context=None, context_range=(1, 700), seed=61)
    base.update(kw)
    return configs.DecodeConfig(**base)


CASES = [(nb, dc, dr, q, dt) for dt in ("bf16", "fp32") for nb in (1, 2, 4)
         for dc in (64, 128) for dr in (32, 64) for q in (1, 2)]
CASES += [(1, 512, 64, 1, "bf16"), (2, 256, 64, 2, "bf16"), (1, 256, 32, 1, "fp32")]


@pytest.mark.parametrize("nb,dc,dr,q,dt", CASES)
def test_append_small_shapes(nb, dc, dr, q, dt):
    cfg = _cfg(n_branch=nb, d_latent=dc, d_rope=dr, q_len=q, dtype=dt,
               seed=200 + nb + dc + dr + q + (dt == "fp32"))
    _say(f"append nb={nb} dc={dc} dr={dr} q={q} {dt}")
    (rows, _), inp = _run(cfg)
    assert rows == int(np.minimum(inp.seq_lens, cfg.q_len).sum())


def test_append_edge_positions_and_block_ids():
    cfg = _cfg(num_seqs=6, q_len=2, context=200, context_range=None, seed=71)
    inp = make_inputs(cfg)
    mb = inp.block_table.shape[1]
    # L < Q; L = 0; L one and two past the table's capacity; L far past it
    lens = [1, 0, mb * 64 + 1, mb * 64 + 2, 10 ** 6, 200]
    table = inp.block_table.copy()
    table[5, :] = inp.num_blocks + 7          # sequence 5: every block id outside the cache
    _say("append edge positions")
    (rows, _), _ = _run(cfg, seq_lens=lens, table=table)
    assert rows == 1 + 0 + 1 + 0 + 0 + 0


def test_append_full_size_headline_layout():
    cfg = configs.MLRA4_TP_SHARE
    _say(f"append {cfg.name}")
    (rows, _), _ = _run(cfg, latent_scale=1.0 / np.sqrt(2.0))
    assert rows == cfg.num_seqs * cfg.q_len


@pytest.mark.parametrize("name", ["mlra4_fused_b32_t16384", "mlra4_ragged_b64_q2",
                                  "mlra2_fused_b32_t16384"])
def test_append_full_size_layouts(name):
    # Untouched rows are compared on the device, bit for bit; the oracle runs
    # on a compact cache made of the touched blocks only (host memory stays
    # small at these sizes).
    cfg = configs.BY_NAME[name]
    inp = make_inputs(cfg)
    lat_new, rope_new = make_append_inputs(cfg)
    d = to_device(inp)
    before_lat, before_rope = d["latent_cache"].clone(), d["rope_cache"].clone()
    scale = float(np.float32(1.0 / np.sqrt(2.0)))
    _say(f"append {name}")
    api.mlra_cache_append(torch.from_numpy(lat_new).cuda(), torch.from_numpy(rope_new).cuda(),
                          d["latent_cache"], d["rope_cache"], d["block_table"], d["seq_lens"],
                          scale)
    torch.cuda.synchronize()
    BS, Q = cfg.block_size, cfg.q_len
    cols = {(s, (int(L) - Q + j) // BS) for s, L in enumerate(inp.seq_lens) for j in range(Q)}
    written = {(int(inp.block_table[s, (int(L) - Q + j) // BS]), (int(L) - Q + j) % BS)
               for s, L in enumerate(inp.seq_lens) for j in range(Q)}
    mask = torch.zeros(d["latent_cache"].shape[:2], dtype=torch.bool)
    for b, t in written:
        mask[b, t] = True
    mask = mask.cuda()
    iv = lambda x: x.view(torch.int16) if x.dtype == torch.bfloat16 else x.view(torch.int32)
    assert torch.equal(iv(d["latent_cache"])[~mask], iv(before_lat)[~mask])
    assert torch.equal(iv(d["rope_cache"])[~mask], iv(before_rope)[~mask])
    blocks = sorted({int(inp.block_table[s, c]) for s, c in cols})
    remap = {b: i for i, b in enumerate(blocks)}
    mini_table = np.full_like(inp.block_table, len(blocks))   # outside the compact cache
    for s, c in cols:
        mini_table[s, c] = remap[int(inp.block_table[s, c])]
    ref_lat, ref_rope = cache_append(lat_new, rope_new, inp.latent_cache[blocks],
                                     inp.rope_cache[blocks], mini_table, inp.seq_lens, scale,
                                     10000.0, BS, to_bf16=True)
    idx = torch.tensor(blocks, device="cuda")
    got_lat = d["latent_cache"][idx].float().cpu().numpy().astype(np.float64)
    got_rope = d["rope_cache"][idx].float().cpu().numpy().astype(np.float64)
    rows, _ = _check(cfg, got_lat, got_rope, ref_lat, ref_rope,
                     inp.latent_cache[blocks].astype(np.float64),
                     inp.rope_cache[blocks].astype(np.float64))
    assert rows == len(written) == cfg.num_seqs * Q


def test_append_positions_in_the_millions():
    cfg = _cfg(num_seqs=2, q_len=2, n_branch=1, context=40_000, context_range=None, seed=81)
    inp = make_inputs(cfg)
    # the table is long enough: move the new tokens to positions near 2^21
    mb = inp.block_table.shape[1]
    big = np.tile(inp.block_table, (1, (2_100_000 // 64) // mb + 1))
    _say("append at positions ~2.1M")
    (rows, ndiff), _ = _run(cfg, seq_lens=[2_097_152, 2_000_001], table=big)
    assert rows == 4


def test_append_then_decode_matches_the_oracle():
    cfg = _cfg(num_seqs=3, q_len=2, num_heads=16, n_branch=4, context_range=(64, 900), seed=91)
    inp = make_inputs(cfg)
    lat_new, rope_new = make_append_inputs(cfg)
    d = to_device(inp)
    api.mlra_cache_append(torch.from_numpy(lat_new).cuda(), torch.from_numpy(rope_new).cuda(),
                          d["latent_cache"], d["rope_cache"], d["block_table"], d["seq_lens"],
                          0.5)
    scale = 1 / np.sqrt(192)
    _say("append then decode")
    out, lse = api.mlra_decode_attention(d["q_latent"], d["q_rope"], d["latent_cache"],
                                         d["rope_cache"], d["block_table"], d["seq_lens"], 4,
                                         scale, 0.5, max_seq_len=inp.max_seq_len)
    torch.cuda.synchronize()
    ref_lat, ref_rope = cache_append(lat_new, rope_new, inp.latent_cache, inp.rope_cache,
                                     inp.block_table, inp.seq_lens, 0.5)
    ro, rl = mlra_decode(inp.q_latent, inp.q_rope, ref_lat, ref_rope, inp.block_table,
                         inp.seq_lens, scale, 0.5)
    o = out.float().cpu().numpy()
    assert np.abs(o - ro).max() <= 2e-2
    assert np.linalg.norm(o - ro) / np.linalg.norm(ro) <= 1e-2
    assert np.abs(lse.cpu().numpy() - rl).max() <= 1e-3
