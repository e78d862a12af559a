"""Pins of the oracle in the prefill regime: many causal query tokens (CPU only).

mlra_decode defines the output for any number Q of new query tokens: token j
of a chunk sees the cached context and the chunk's tokens up to itself,
t < L - (Q - 1 - j). These checks hold it to things other than itself:
torch's scaled_dot_product_attention with its own causal flag (a whole
sequence prefilled at once, where torch's top-left-aligned mask and the
chunk rule coincide) and with an explicit mask built from token positions;
the invariant that prefilling a sequence in chunks gives every token the
output of prefilling it whole; and planted mistakes in the visibility rule,
which must fail at least one of them.
"""
import inspect

import numpy as np
import pytest
import torch

import oracle.mlra_oracle as mo
from latent_kv_cache_amd import configs
from latent_kv_cache_amd.inputs import make_inputs


def _cfg(**kw):
    base = dict(name="prefill_small", num_seqs=2, q_len=12, num_heads=3, n_branch=2,
                d_latent=6, d_rope=4, dtype="fp32", context=30, block_size=8, seed=21,
                scale=0.45, out_rescale=0.5)
    base.update(kw)
    return configs.DecodeConfig(**base)


def _gather(cache, table_row, L, bs):
    # block-table walk written out per token, independent of paged_gather
    return np.stack([cache[table_row[t // bs], t % bs] for t in range(L)]).astype(np.float64)


def _sdpa_branch(q, k, v, scale, mask=None, is_causal=False):
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float64))
    return torch.nn.functional.scaled_dot_product_attention(
        t(q), t(k), t(v), attn_mask=None if mask is None else torch.from_numpy(mask),
        is_causal=is_causal, scale=scale).numpy()


def _reference(inp, mask_fn):
    """Per (sequence, head, branch): SDPA over keys [c_b ; k_r] and values c_b,
    with the boolean mask mask_fn(L, Q) (or torch's own causal flag)."""
    c = inp.cfg
    S, Q, H, NB, DC = inp.q_latent.shape
    out = np.zeros((S, Q, H, NB, DC))
    for s in range(S):
        L = int(inp.seq_lens[s])
        C = _gather(inp.latent_cache, inp.block_table[s], L, c.block_size)
        KR = _gather(inp.rope_cache, inp.block_table[s], L, c.block_size)
        for h in range(H):
            for b in range(NB):
                q = np.concatenate([inp.q_latent[s, :, h, b], inp.q_rope[s, :, h]], axis=1)
                k = np.concatenate([C[:, b], KR], axis=1)
                m = mask_fn(L, Q)
                if m is None:
                    out[s, :, h, b] = _sdpa_branch(q, k, C[:, b], c.scale, is_causal=True)
                else:
                    out[s, :, h, b] = _sdpa_branch(q, k, C[:, b], c.scale, mask=m)
    return out


def _oracle(mod, inp, **kw):
    c = inp.cfg
    args = dict(scale=c.scale, out_rescale=1.0, reduce="concat", causal=True,
                block_size=c.block_size)
    args.update(kw)
    return mod.mlra_decode(inp.q_latent, inp.q_rope, inp.latent_cache, inp.rope_cache,
                           inp.block_table, inp.seq_lens, **args)


def _whole_prefill_ok(mod):
    # Q = L: the chunk is the whole sequence, torch's is_causal applies as is
    inp = make_inputs(_cfg(q_len=23, context=23, seed=22))
    try:
        o, _ = _oracle(mod, inp)
    except Exception:
        return False
    return np.allclose(o, _reference(inp, lambda L, Q: None), rtol=1e-10, atol=1e-12)


def _chunk_mask_ok(mod):
    # a chunk of 12 new tokens after 18 cached ones: query j at position
    # L - Q + j sees every token at a position up to its own
    inp = make_inputs(_cfg())
    mask = lambda L, Q: (np.arange(L)[None, :] <= (L - Q + np.arange(Q))[:, None])
    try:
        o, _ = _oracle(mod, inp)
    except Exception:
        return False
    return np.allclose(o, _reference(inp, mask), rtol=1e-10, atol=1e-12)


def _chunking_invariant_ok(mod):
    # one 40-token sequence prefilled whole, then as chunks of 17, 1 and 22
    # tokens, each chunk call seeing the cache filled up to its own end
    cfg = _cfg(num_seqs=1, q_len=40, context=40, seed=23)
    inp = make_inputs(cfg)
    try:
        whole, lw = _oracle(mod, inp)
        start = 0
        for n in (17, 1, 22):
            part, lp = mod.mlra_decode(
                inp.q_latent[:, start:start + n], inp.q_rope[:, start:start + n],
                inp.latent_cache, inp.rope_cache, inp.block_table,
                np.array([start + n], dtype=np.int32), cfg.scale, 1.0, "concat", True,
                cfg.block_size)
            if not (np.allclose(part, whole[:, start:start + n], rtol=1e-13, atol=1e-15)
                    and np.allclose(lp, lw[:, start:start + n], rtol=1e-13)):
                return False
            start += n
    except Exception:
        return False
    return True


def _first_token_sees_one_ok(mod):
    # whole-sequence prefill: token 0 sees only itself, so its output is its
    # own latent and its lse is its own scaled score
    inp = make_inputs(_cfg(q_len=9, context=9, seed=24))
    try:
        o, lse = _oracle(mod, inp)
    except Exception:
        return False
    c = inp.cfg
    for s in range(c.num_seqs):
        c0 = inp.latent_cache[inp.block_table[s, 0], 0].astype(np.float64)   # [NB][DC]
        k0 = inp.rope_cache[inp.block_table[s, 0], 0].astype(np.float64)
        for h in range(c.num_heads):
            for b in range(c.n_branch):
                z = c.scale * (inp.q_latent[s, 0, h, b] @ c0[b] + inp.q_rope[s, 0, h] @ k0)
                if not (np.allclose(o[s, 0, h, b], c0[b], rtol=1e-13, atol=1e-15)
                        and np.isclose(lse[s, 0, h, b], z, rtol=1e-12, atol=1e-13)):
                    return False
    return True


def _all_ok(mod):
    return (_whole_prefill_ok(mod) and _chunk_mask_ok(mod) and _chunking_invariant_ok(mod)
            and _first_token_sees_one_ok(mod))


def test_whole_sequence_prefill_equals_torch_causal_sdpa():
    assert _whole_prefill_ok(mo)


def test_chunk_after_context_equals_sdpa_with_position_mask():
    assert _chunk_mask_ok(mo)


def test_chunked_prefill_equals_whole_prefill():
    assert _chunking_invariant_ok(mo)


def test_first_token_of_a_whole_prefill_sees_only_itself():
    assert _first_token_sees_one_ok(mo)


def test_non_causal_chunk_sees_everything():
    inp = make_inputs(_cfg(seed=25))
    o, _ = _oracle(mo, inp, causal=False)
    ref = _reference(inp, lambda L, Q: np.ones((Q, L), dtype=bool))
    np.testing.assert_allclose(o, ref, rtol=1e-10, atol=1e-12)


SRC = inspect.getsource(mo)
VIS = "    return int(seq_len) - (q_len - 1 - j) if causal else int(seq_len)\n"
MUTANTS = {
    "excludes_itself": (VIS, "    return int(seq_len) - (q_len - j) if causal else int(seq_len)\n"),
    "sees_one_ahead": (VIS, "    return int(seq_len) - (q_len - 2 - j) if causal else int(seq_len)\n"),
    "top_left_aligned": (VIS, "    return j + 1 if causal else int(seq_len)\n"),
    "chunk_reversed": (VIS, "    return int(seq_len) - j if causal else int(seq_len)\n"),
    "causal_ignored": (VIS, "    return int(seq_len)\n"),
}


def _mutant(name):
    old, new = MUTANTS[name]
    assert SRC.count(old) == 1, name
    ns = {"__name__": f"mutant_{name}"}
    exec(compile(SRC.replace(old, new), f"<mutant {name}>", "exec"), ns)

    class M:
        pass
    m = M()
    m.mlra_decode = ns["mlra_decode"]
    return m


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    assert not _all_ok(_mutant(name)), name


def test_unmutated_source_passes_the_same_pins():
    ns = {"__name__": "unmutated"}
    exec(compile(SRC, "<oracle>", "exec"), ns)

    class M:
        pass
    m = M()
    m.mlra_decode = ns["mlra_decode"]
    assert _all_ok(m)
