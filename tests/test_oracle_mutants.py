"""Planted mistakes in the oracle must be caught by its pins (CPU only).

Each mutant is the oracle's source with one plausible mistake substituted
(a dropped term, a wrong sign, base, index or operand); it is executed in a
private namespace and run through the pins that compare against independent
references (the hand-derived golden example, the brute-force loops and the
expanded form). A mutant that passes all of them means the pins are too weak.
"""
import inspect
import json
import math
import os

import numpy as np
import pytest

import oracle.mlra_oracle as om
from latent_kv_cache_amd import configs
from latent_kv_cache_amd.inputs import make_inputs

SRC = inspect.getsource(om)

MUTANTS = {
    "rope_sign": ("qb @ Cb.T + rope_dot", "qb @ Cb.T - rope_dot"),
    "rope_dropped": ("qb @ Cb.T + rope_dot", "qb @ Cb.T"),
    "scale_on_latent_only": ("scale * (qb @ Cb.T + rope_dot)", "scale * (qb @ Cb.T) + rope_dot"),
    "log2_lse": ("m + np.log(tot)", "m + np.log2(tot)"),
    "rescale_dropped": ("out[s, j] += out_rescale * ob", "out[s, j] += ob"),
    "sum_before_branch_softmax": ("z = scale * (qb @ Cb.T + rope_dot)",
                                  "z = scale * (np.asarray(q_latent[s, j], dtype=np.float64)"
                                  ".reshape(H, -1) @ C[:V].reshape(V, -1).T + rope_dot)"),
    "causal_off_by_one": ("int(seq_len) - (q_len - 1 - j)", "int(seq_len) - (q_len - j)"),
    "causal_reversed": ("int(seq_len) - (q_len - 1 - j)", "int(seq_len) - j"),
    "block_index_mod": ("phys = np.asarray(table_row)[t // block_size]",
                        "phys = np.asarray(table_row)[t % max(1, len(table_row))]"),
    "slot_reversed": ("cache[phys, t % block_size]", "cache[phys, block_size - 1 - t % block_size]"),
    "value_from_rope_weights": ("ob = (e / tot) @ Cb", "ob = (e / e.max(axis=1, keepdims=True)) @ Cb"),
    "max_not_subtracted_in_lse": ("m + np.log(tot)", "np.log(tot)"),
}


def _mutant(name):
    old, new = MUTANTS[name]
    assert SRC.count(old) >= 1, name
    ns = {"__name__": f"mutant_{name}"}
    exec(compile(SRC.replace(old, new), f"<mutant {name}>", "exec"), ns)
    return ns


def _golden_ok(ns):
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden",
                                    "hand_example.json")))
    env = {"ln2": math.log(2), "ln3": math.log(3), "ln9": math.log(9), "ln4": math.log(4),
           "nan": float("nan")}

    def ev(x):
        if isinstance(x, list):
            return [ev(v) for v in x]
        return float(eval(x, {"__builtins__": {}}, env)) if isinstance(x, str) else float(x)

    a = {k: np.array(ev(g[k])) for k in ("q_latent", "q_rope", "latent_cache", "rope_cache")}
    try:
        for reduce, key in (("sum", "expected_out_sum"), ("concat", "expected_out_concat")):
            out, lse = ns["mlra_decode"](a["q_latent"], a["q_rope"], a["latent_cache"],
                                         a["rope_cache"], np.array(g["block_table"]),
                                         np.array(g["seq_lens"]), g["scale"], g["out_rescale"],
                                         reduce, True, g["block_size"])
            if not (np.allclose(out, ev(g[key]), rtol=1e-12, atol=1e-12)
                    and np.allclose(lse, ev(g["expected_lse"]), rtol=1e-12)):
                return False
    except Exception:
        return False
    return True


def _bruteforce_ok(ns):
    cfg = configs.DecodeConfig(name="m", num_seqs=2, q_len=2, num_heads=2, n_branch=2,
                               d_latent=3, d_rope=2, dtype="fp32", context=None,
                               context_range=(3, 20), block_size=4, seed=9, scale=0.6,
                               out_rescale=0.5)
    inp = make_inputs(cfg)
    args = (inp.q_latent, inp.q_rope, inp.latent_cache, inp.rope_cache, inp.block_table,
            inp.seq_lens, cfg.scale, cfg.out_rescale)
    try:
        for reduce in ("sum", "concat"):
            o1, l1 = ns["mlra_decode"](*args, reduce, True, 4)
            o2, l2 = om.mlra_decode_bruteforce(*args, reduce, True, 4)
            if not (np.allclose(o1, o2, rtol=1e-10, atol=1e-12)
                    and np.allclose(l1, l2, rtol=1e-10)):
                return False
    except Exception:
        return False
    return True


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    ns = _mutant(name)
    assert not (_golden_ok(ns) and _bruteforce_ok(ns)), f"mutant {name} passed every pin"


def test_unmutated_source_passes_the_same_pins():
    ns = {"__name__": "unmutated"}
    exec(compile(SRC, "<oracle>", "exec"), ns)
    assert _golden_ok(ns) and _bruteforce_ok(ns)
