"""Pins of the cache-append oracle (CPU only).

Each check compares the oracle with something other than itself: a
hand-derived example, properties that every rotary embedding of this form
has (identity at position 0, kept pair norms, composition, scores that depend
only on the position difference), the seeded generator's independent float32
rounding, and brute-force gathers of the appended caches. Planted mistakes in
the oracle's source must fail at least one of them.
"""
import inspect
import json
import math
import os

import numpy as np
import pytest

import oracle.append_oracle as ao
from oracle import paged_gather
from latent_kv_cache_amd.inputs import round_to_bf16

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "append_example.json")


def _ev(x):
    env = {"cos": math.cos, "sin": math.sin}
    if isinstance(x, list):
        return [_ev(v) for v in x]
    return float(eval(x, {"__builtins__": {}}, env)) if isinstance(x, str) else float(x)


def _golden_ok(mod):
    g = json.load(open(GOLDEN))
    bs, nb = g["block_size"], g["num_blocks"]
    lat_new = np.array(g["latent_new"], dtype=np.float64)
    rope_new = np.array(g["rope_new"], dtype=np.float64)
    lat0 = np.full((nb, bs) + lat_new.shape[2:], g["initial_latent"])
    rope0 = np.full((nb, bs, rope_new.shape[-1]), g["initial_rope"])
    exp_lat, exp_rope = lat0.copy(), rope0.copy()
    for w in g["expected_latent_writes"]:
        exp_lat[w["block"], w["slot"]] = np.array(_ev(w["value"])).reshape(exp_lat.shape[2:])
    for w in g["expected_rope_writes"]:
        exp_rope[w["block"], w["slot"]] = _ev(w["value"])
    try:
        lat, rope = mod.cache_append(lat_new, rope_new, lat0, rope0,
                                     np.array(g["block_table"]), np.array(g["seq_lens"]),
                                     g["latent_scale"], g["rope_base"], bs, to_bf16=False)
    except Exception:
        return False
    return (np.allclose(lat, exp_lat, rtol=0, atol=1e-15)
            and np.allclose(rope, exp_rope, rtol=0, atol=1e-15))


def _rope_properties_ok(mod):
    rng = np.random.default_rng(3)
    try:
        for DR in (2, 8, 64):
            x = rng.standard_normal((5, DR))
            if not np.allclose(mod.rope_rotate(x, 0), x, rtol=0, atol=0):
                return False
            pos = rng.integers(0, 3_000_000, size=5)
            y = mod.rope_rotate(x, pos)
            pn = lambda v: np.hypot(v[..., 0::2], v[..., 1::2])
            if not np.allclose(pn(y), pn(x), rtol=1e-12):
                return False
            a, b = 1234, 98765
            if not np.allclose(mod.rope_rotate(mod.rope_rotate(x, a), b),
                               mod.rope_rotate(x, a + b), rtol=1e-9, atol=1e-9):
                return False
            q, k = rng.standard_normal(DR), rng.standard_normal(DR)
            m, n, d = 70_001, 12_345, 4_567
            s1 = mod.rope_rotate(q, m) @ mod.rope_rotate(k, n)
            s2 = mod.rope_rotate(q, m + d) @ mod.rope_rotate(k, n + d)
            if not math.isclose(s1, s2, rel_tol=1e-8, abs_tol=1e-9):
                return False
    except Exception:
        return False
    return True


def test_golden_example():
    assert _golden_ok(ao)


def test_rope_properties():
    assert _rope_properties_ok(ao)


def test_rope_angles_grow_with_the_pair_index_as_the_base_power():
    # pair i of a unit vector at position 1 turns by base**(-2i/DR): its cosine
    DR, base = 8, 10000.0
    x = np.zeros(DR)
    x[0::2] = 1.0
    y = ao.rope_rotate(x, 1, base)
    for i in range(DR // 2):
        assert math.isclose(y[2 * i], math.cos(base ** (-2.0 * i / DR)), rel_tol=1e-15)


def test_bf16_rounding():
    f = ao.round_to_bf16_f64
    assert f(1.0 + 2.0 ** -8) == 1.0                   # tie, to even
    assert f(1.0 + 3 * 2.0 ** -8) == 1.0 + 2.0 ** -6   # tie, to even (up)
    assert f(-(1.0 + 2.0 ** -8)) == -1.0
    assert f(1.0 + 2.0 ** -8 + 2.0 ** -30) == 1.0 + 2.0 ** -7   # past the tie
    assert f(0.0) == 0.0
    rng = np.random.default_rng(5)
    x = (rng.standard_normal(100_000) * np.exp(rng.uniform(-20, 20, 100_000))).astype(np.float32)
    ref = round_to_bf16(x.copy()).astype(np.float64)   # the generator's own float32 rounding
    assert np.array_equal(f(x.astype(np.float64)), ref)
    assert np.array_equal(f(ref), ref)                  # bf16-exact values stay put


def _random_case(seed, S=5, Q=2, NB=2, DC=4, DR=6, BS=4, max_blocks=6):
    rng = np.random.default_rng(seed)
    nblocks = S * max_blocks + 1
    table = rng.permutation(nblocks - 1)[:S * max_blocks].reshape(S, max_blocks).astype(np.int32)
    seq_lens = rng.integers(0, BS * max_blocks + 1, size=S).astype(np.int32)
    lat = rng.standard_normal((nblocks, BS, NB, DC))
    rope = rng.standard_normal((nblocks, BS, DR))
    lat_new = rng.standard_normal((S, Q, NB, DC))
    rope_new = rng.standard_normal((S, Q, DR))
    return table, seq_lens, lat, rope, lat_new, rope_new


def test_brute_force_gather_after_append():
    table, seq_lens, lat, rope, lat_new, rope_new = _random_case(11)
    BS, Q = lat.shape[1], lat_new.shape[1]
    scale, base = 0.75, 500.0
    lat2, rope2 = ao.cache_append(lat_new, rope_new, lat, rope, table, seq_lens, scale, base,
                                  BS, to_bf16=False)
    written = np.zeros(lat.shape[:2], dtype=bool)
    for s, L in enumerate(seq_lens):
        L = int(L)
        C = paged_gather(lat2, table[s], L, BS)
        K = paged_gather(rope2, table[s], L, BS)
        C0 = paged_gather(lat, table[s], L, BS)
        K0 = paged_gather(rope, table[s], L, BS)
        for t in range(L):
            j = t - (L - Q)
            if j < 0:
                assert np.array_equal(C[t], C0[t]) and np.array_equal(K[t], K0[t])
                continue
            written[table[s, t // BS], t % BS] = True
            assert np.allclose(C[t], scale * lat_new[s, j], rtol=1e-15)
            # the key: a plain per-pair rotation matrix at angle t * base**(-2i/DR)
            DR = K.shape[-1]
            for i in range(DR // 2):
                a = t * base ** (-2.0 * i / DR)
                R = np.array([[math.cos(a), -math.sin(a)], [math.sin(a), math.cos(a)]])
                assert np.allclose(K[t, 2 * i:2 * i + 2], R @ rope_new[s, j, 2 * i:2 * i + 2],
                                   rtol=1e-12, atol=1e-12)
    # nothing else changed
    assert np.array_equal(lat2[~written], lat[~written])
    assert np.array_equal(rope2[~written], rope[~written])


def test_block_permutation_invariance_and_skipped_writes():
    table, seq_lens, lat, rope, lat_new, rope_new = _random_case(12)
    BS = lat.shape[1]
    a_lat, a_rope = ao.cache_append(lat_new, rope_new, lat, rope, table, seq_lens, 1.5,
                                    block_size=BS)
    perm = np.random.default_rng(2).permutation(lat.shape[0])
    lat_p, rope_p = np.empty_like(lat), np.empty_like(rope)
    lat_p[perm], rope_p[perm] = lat, rope
    b_lat, b_rope = ao.cache_append(lat_new, rope_new, lat_p, rope_p, perm[table], seq_lens, 1.5,
                                    block_size=BS)
    assert np.array_equal(b_lat[perm], a_lat) and np.array_equal(b_rope[perm], a_rope)
    # a block id outside the cache, or a position past the table, writes nothing
    bad = table.copy()
    bad[:, :] = lat.shape[0] + 3
    c_lat, c_rope = ao.cache_append(lat_new, rope_new, lat, rope, bad, seq_lens, 1.5,
                                    block_size=BS)
    assert np.array_equal(c_lat, lat) and np.array_equal(c_rope, rope)
    # L one past the table's capacity: token 0 of 2 fills the last slot, token 1 is dropped
    long = np.full_like(seq_lens, table.shape[1] * BS + 1)
    d_lat, _ = ao.cache_append(lat_new, rope_new, lat, rope, table, long, 1.5, block_size=BS)
    changed = (d_lat != lat).any(axis=(2, 3))
    assert changed.sum() == len(seq_lens)
    assert all(changed[table[s, -1], BS - 1] for s in range(len(seq_lens)))


SRC = inspect.getsource(ao)
MUTANTS = {
    "rotation_sign": ("y[..., 0::2] = xe * c - xo * s", "y[..., 0::2] = xe * c + xo * s"),
    "half_split_pairs": ("xe, xo = x[..., 0::2], x[..., 1::2]",
                         "xe, xo = x[..., :DR // 2], x[..., DR // 2:]"),
    "exponent_without_two": ("theta = float(base) ** (-2.0 * i / DR)",
                             "theta = float(base) ** (-1.0 * i / DR)"),
    "position_off_by_one": ("            p = L - Q + j\n", "            p = L - Q + j + 1\n"),
    "position_from_start": ("            p = L - Q + j\n", "            p = j\n"),
    "scale_dropped": ("c = float(latent_scale) * np.asarray", "c = np.asarray"),
    "scale_on_key": ("k = rope_rotate(rope_new[s, j], p, rope_base)",
                     "k = float(latent_scale) * rope_rotate(rope_new[s, j], p, rope_base)"),
    "slot_from_block": ("lat[blk, p % block_size] = c", "lat[blk, p // block_size] = c"),
    "round_half_away": ("np.rint(m * 256.0)", "np.trunc(m * 256.0 + np.copysign(0.5, m))"),
    "round_seven_bits": ("np.rint(m * 256.0), e - 8", "np.rint(m * 128.0), e - 7"),
}


def _mutant(name):
    old, new = MUTANTS[name]
    assert SRC.count(old) == 1, name
    ns = {"__name__": f"mutant_{name}"}
    exec(compile(SRC.replace(old, new), f"<mutant {name}>", "exec"), ns)

    class M:
        pass
    m = M()
    for k in ("rope_rotate", "round_to_bf16_f64", "cache_append"):
        setattr(m, k, ns[k])
    return m


def _rounding_ok(mod):
    try:
        f = mod.round_to_bf16_f64
        return (f(1.0 + 2.0 ** -8) == 1.0 and f(1.0 + 3 * 2.0 ** -8) == 1.0 + 2.0 ** -6
                and f(1.0 + 2.0 ** -7) == 1.0 + 2.0 ** -7)
    except Exception:
        return False


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    m = _mutant(name)
    assert not (_golden_ok(m) and _rope_properties_ok(m) and _rounding_ok(m)), name


def test_unmutated_source_passes_the_same_pins():
    ns = {"__name__": "unmutated"}
    exec(compile(SRC, "<oracle>", "exec"), ns)

    class M:
        pass
    m = M()
    for k in ("rope_rotate", "round_to_bf16_f64", "cache_append"):
        setattr(m, k, ns[k])
    assert _golden_ok(m) and _rope_properties_ok(m) and _rounding_ok(m)
