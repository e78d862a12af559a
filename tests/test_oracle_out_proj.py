"""Pins of the output-projection oracle (CPU only): a hand-derived example,
the two-stage definition with independent random factors, brute-force loops
and linearity; planted mistakes in the oracle's source must fail one of them.
"""
import inspect
import json
import os

import numpy as np
import pytest

import oracle.out_proj_oracle as po

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "out_proj_example.json")


def _golden_ok(mod):
    g = json.load(open(GOLDEN))
    try:
        w = mod.absorb_weights(np.array(g["w_uv"]), np.array(g["w_o"]))
        y = mod.out_projection(np.array(g["o_concat"]), w)
    except Exception:
        return False
    return (np.array_equal(w, np.array(g["expected_absorbed"], dtype=np.float64))
            and np.array_equal(y, np.array(g["expected_y"], dtype=np.float64)))


def _two_stage_ok(mod, seed=3):
    rng = np.random.default_rng(seed)
    S, Q, H, NB, DC, dv, D = 2, 2, 3, 2, 5, 4, 7
    w_uv = rng.standard_normal((H, NB, dv, DC))
    w_o = rng.standard_normal((D, H * dv))
    o = rng.standard_normal((S, Q, H, NB, DC))
    # per head: sum of the branches' value up-projections; then the output projection
    v = np.zeros((S, Q, H, dv))
    for h in range(H):
        for b in range(NB):
            v[:, :, h] += o[:, :, h, b] @ w_uv[h, b].T
    ref = v.reshape(S, Q, H * dv) @ w_o.T
    try:
        y = mod.out_projection(o, mod.absorb_weights(w_uv, w_o))
    except Exception:
        return False
    return y.shape == ref.shape and np.allclose(y, ref, rtol=1e-12, atol=1e-12)


def _bruteforce_ok(mod, seed=4):
    rng = np.random.default_rng(seed)
    S, Q, H, NB, DC, dv, D = 1, 2, 2, 2, 3, 2, 3
    w_uv = rng.standard_normal((H, NB, dv, DC))
    w_o = rng.standard_normal((D, H * dv))
    o = rng.standard_normal((S, Q, H, NB, DC))
    try:
        w = mod.absorb_weights(w_uv, w_o)
        y = mod.out_projection(o, w)
    except Exception:
        return False
    for n in range(D):
        for h in range(H):
            for b in range(NB):
                for c in range(DC):
                    t = sum(w_o[n, h * dv + d] * w_uv[h, b, d, c] for d in range(dv))
                    if not np.isclose(w[n, (h * NB + b) * DC + c], t, rtol=1e-13, atol=1e-13):
                        return False
    for s in range(S):
        for j in range(Q):
            for n in range(D):
                t = sum(o[s, j, h, b, c] * w[n, (h * NB + b) * DC + c]
                        for h in range(H) for b in range(NB) for c in range(DC))
                if not np.isclose(y[s, j, n], t, rtol=1e-13, atol=1e-13):
                    return False
    return True


def test_golden_example():
    assert _golden_ok(po)


def test_two_stage_definition():
    assert _two_stage_ok(po)


def test_brute_force_loops():
    assert _bruteforce_ok(po)


def test_linearity():
    rng = np.random.default_rng(6)
    w = rng.standard_normal((5, 2 * 2 * 3))
    o1, o2 = rng.standard_normal((2, 2, 2, 2, 3)), rng.standard_normal((2, 2, 2, 2, 3))
    a = 0.37
    lhs = po.out_projection(a * o1 + o2, w)
    rhs = a * po.out_projection(o1, w) + po.out_projection(o2, w)
    assert np.allclose(lhs, rhs, rtol=1e-12, atol=1e-12)


SRC = inspect.getsource(po)
MUTANTS = {
    "head_slice_without_dv": ("wo_h = w_o[:, h * dv:(h + 1) * dv]", "wo_h = w_o[:, h:h + dv]"),
    "branch_up_projection_transposed": ("w[:, h, b, :] = wo_h @ w_uv[h, b]",
                                        "w[:, h, b, :] = (wo_h @ w_uv[h, b].reshape(DC, dv).T)"),
    "branch_and_column_swapped": ("w = np.empty((D, H, NB, DC))", "w = np.empty((D, H, DC, NB))"),
    "columns_reversed": ("return (x @ np.asarray(w, dtype=np.float64).T)",
                         "return (x @ np.asarray(w, dtype=np.float64)[:, ::-1].T)"),
    "features_reversed": ("return (x @ np.asarray(w, dtype=np.float64).T)",
                          "return (x @ np.asarray(w, dtype=np.float64)[::-1].T)"),
    "first_branch_only": ("for b in range(NB):\n            w[:, h, b, :] = wo_h @ w_uv[h, b]",
                          "for b in range(NB):\n            w[:, h, b, :] = wo_h @ w_uv[h, 0]"),
}


def _mutant(name):
    old, new = MUTANTS[name]
    assert SRC.count(old) == 1, name
    ns = {"__name__": f"mutant_{name}"}
    exec(compile(SRC.replace(old, new), f"<mutant {name}>", "exec"), ns)

    class M:
        pass
    m = M()
    m.absorb_weights, m.out_projection = ns["absorb_weights"], ns["out_projection"]
    return m


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    m = _mutant(name)
    assert not (_golden_ok(m) and _two_stage_ok(m) and _bruteforce_ok(m)), name
