"""Pins of the normalised linear-attention oracle (oracle/norm_la.py).

Page "Linear attention e fast weights", section "Conceito": the output for
token t is the average of the values v_i, i <= t, weighted by
phi(q_t)^T phi(k_i); the matrix state and the normaliser keep the two sums
incrementally. Each pin reaches the oracle's result by another route: the
weighted average written out (brute force), closed forms (constant values,
one token, identical keys), the unnormalised check-oracle of the additive
rule, and invariances a plausible mistake breaks (scaling of the features,
order of earlier tokens, splitting the sequence). Planted mistakes in a copy
of the oracle show that the pins catch them.
"""
import inspect
import os

import numpy as np
import pytest

import gdr_synth as gs
from oracle import forms
from oracle import norm_la

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "capital_city.txt")


def _pos(rng, shape):
    return np.abs(rng.standard_normal(shape)) + 0.05


def _one_head(rng, T, D, Dv=None):
    Dv = Dv or D
    return _pos(rng, (T, D)), _pos(rng, (T, D)), rng.standard_normal((T, Dv))


def _run1(q, k, v, S0=None, z0=None, fn=None):
    """One head through a recurrence function with the prefill layout."""
    fn = fn or norm_la.recurrent
    o, S, z = fn(q[None, :, None], k[None, :, None], v[None, :, None],
                 None if S0 is None else S0[None, None], None if z0 is None else z0[None, None])
    return o[0, :, 0], S[0, 0], z[0, 0]


def test_brute_force_weighted_average():
    rng = np.random.default_rng(0)
    q, k, v = _one_head(rng, 23, 8, 5)
    o, _, _ = _run1(q, k, v)
    assert np.max(np.abs(o - norm_la.weighted_average(q, k, v))) < 1e-13


def test_constant_values_are_returned():
    rng = np.random.default_rng(1)
    q, k, _ = _one_head(rng, 17, 6)
    c = np.array([0.5, -1.25, 2.0, 0.75, 3.0, -0.125])
    o, _, _ = _run1(q, k, np.tile(c, (17, 1)))
    assert np.max(np.abs(o - c)) < 1e-14


def test_single_token_returns_its_value():
    rng = np.random.default_rng(2)
    q, k, v = _one_head(rng, 1, 8)
    o, S, z = _run1(q, k, v)
    assert np.max(np.abs(o[0] - v[0])) < 1e-15
    assert np.array_equal(S, np.outer(k[0], v[0])) and np.array_equal(z, k[0])


def _golden():
    vals = {}
    for line in open(GOLDEN):
        if line.strip() and not line.startswith("#"):
            name, *rest = line.split()
            vals[name] = np.array([float(x) for x in rest])
    return vals


def test_capital_city_identical_keys_give_the_mean():
    """Writing v_paris then v_brasilia under the same key and reading with it:
    the additive memory returns their sum, the normalised read their mixture
    with equal weights, the mean (the page: the old association is never
    removed, the read returns a mixture of the two)."""
    g = _golden()
    k = np.abs(g["k"])[None].repeat(2, axis=0)
    v = np.stack([g["v_paris"], g["v_brasilia"]])
    o, _, _ = _run1(k, k, v)
    assert np.array_equal(o[1], g["expect_normalised_mean"])
    assert np.array_equal(o[1] * 2.0, g["expect_additive"])


def test_numerator_is_the_additive_rule():
    """S_t^T phi(q_t) is the unnormalised (additive) linear attention read of
    the family analysis's check-oracle, in that page's d_v x d_k layout; the
    oracle's output times its normaliser must equal it."""
    rng = np.random.default_rng(3)
    q, k, v = _one_head(rng, 19, 7, 4)
    o, S, z = _run1(q, k, v)
    o_add, Sp = forms.additive_la(q, k, v)
    den = np.array([np.cumsum(k, axis=0)[t] @ q[t] for t in range(19)])
    assert np.max(np.abs(o * den[:, None] - o_add)) < 1e-12
    assert np.max(np.abs(S - Sp.T)) < 1e-13


def test_feature_scaling_invariance():
    rng = np.random.default_rng(4)
    q, k, v = _one_head(rng, 15, 8)
    o, _, _ = _run1(q, k, v)
    o2, _, _ = _run1(3.0 * q, 0.25 * k, v)
    assert np.max(np.abs(o - o2)) < 1e-13


def test_order_of_earlier_tokens_does_not_matter():
    rng = np.random.default_rng(5)
    q, k, v = _one_head(rng, 12, 8)
    perm = np.concatenate([rng.permutation(11), [11]])
    o, S, z = _run1(q, k, v)
    o2, S2, z2 = _run1(q[perm], k[perm], v[perm])
    assert np.max(np.abs(o[-1] - o2[-1])) < 1e-13
    assert np.max(np.abs(S - S2)) < 1e-13 and np.max(np.abs(z - z2)) < 1e-13


def test_split_and_resume():
    rng = np.random.default_rng(6)
    q, k, v = _one_head(rng, 30, 8)
    o, S, z = _run1(q, k, v)
    o1, S1, z1 = _run1(q[:11], k[:11], v[:11])
    o2, S2, z2 = _run1(q[11:], k[11:], v[11:], S0=S1, z0=z1)
    assert np.max(np.abs(np.concatenate([o1, o2]) - o)) < 1e-13
    assert np.max(np.abs(S2 - S)) < 1e-13 and np.max(np.abs(z2 - z)) < 1e-13


def test_grouped_heads_and_stored_inputs():
    """V head h reads QK head h / (H_v / H_qk); bfloat16 inputs are widened
    exactly. Each V head equals the one-head run of its own slices."""
    inp = gs.make_norm_la_inputs(2, 9, 2, 6, 8, io="bf16", seed=7, state=True)
    o, S, z = norm_la.recurrent(inp["phq"], inp["phk"], inp["v"], inp["S0"], inp["z0"])
    from oracle import upcast
    q, k, v = upcast(inp["phq"]), upcast(inp["phk"]), upcast(inp["v"])
    for b in range(2):
        for h in range(6):
            hq = h // 3
            o1, S1, z1 = _run1(q[b, :, hq], k[b, :, hq], v[b, :, h], S0=inp["S0"][b, h].astype(np.float64),
                               z0=inp["z0"][b, h].astype(np.float64))
            assert np.array_equal(o1, o[b, :, h]) and np.array_equal(S1, S[b, h]) and np.array_equal(z1, z[b, h])


def test_zero_normaliser_is_rejected():
    q = np.zeros((1, 1, 1, 4))
    k = np.ones((1, 1, 1, 4))
    with pytest.raises(ValueError):
        norm_la.recurrent(q, k, np.ones((1, 1, 1, 4)))


# Planted mistakes: each must fail at least one pin above.
BODY = ("                S[b, h] += np.outer(kt, v[b, t, h])          # write phi(k) v^T\n"
        "                z[b, h] += kt                                 # normaliser\n"
        "                den = z[b, h] @ qt\n"
        "                if den == 0.0:\n"
        "                    raise ValueError(\"zero normaliser z^T phi(q)\")\n"
        "                o[b, t, h] = (S[b, h].T @ qt) / den           # read after the write\n")
MUTANTS = {
    # the read before the token's own write (sum over i < t; an epsilon keeps t = 0 finite)
    "read_before_write": (BODY, "                den = z[b, h] @ qt + 1e-300\n"
                                "                o[b, t, h] = (S[b, h].T @ qt) / den\n"
                                "                S[b, h] += np.outer(kt, v[b, t, h])\n"
                                "                z[b, h] += kt\n"),
    "normaliser_not_updated": ("z[b, h] += kt                                 # normaliser",
                               "z[b, h] = kt"),
    "normaliser_with_key": ("den = z[b, h] @ qt", "den = z[b, h] @ kt"),
    "state_transposed_write": ("S[b, h] += np.outer(kt, v[b, t, h])", "S[b, h] += np.outer(v[b, t, h], kt)"),
    "read_with_key": ("o[b, t, h] = (S[b, h].T @ qt) / den", "o[b, t, h] = (S[b, h].T @ kt) / den"),
    "no_normalisation": ("o[b, t, h] = (S[b, h].T @ qt) / den", "o[b, t, h] = (S[b, h].T @ qt)"),
    "wrong_qk_head": ("hq = h // grp", "hq = h % Hqk"),
}


def _mutant(name):
    old, new = MUTANTS[name]
    src = inspect.getsource(norm_la.recurrent)
    assert old in src, name
    ns = dict(norm_la.__dict__)
    exec(src.replace(old, new, 1), ns)
    return ns["recurrent"]


def _pins_pass(fn):
    checks = []
    rng = np.random.default_rng(10)
    q, k, v = _one_head(rng, 13, 6)
    try:
        o, _, _ = _run1(q, k, v, fn=fn)
        checks.append(np.max(np.abs(o - norm_la.weighted_average(q, k, v))) < 1e-13)
        c = np.linspace(-1, 1, 6)
        o, _, _ = _run1(q, k, np.tile(c, (13, 1)), fn=fn)
        checks.append(np.max(np.abs(o - c)) < 1e-14)
        # grouped heads against one-head runs of each V head's own slices
        inp = gs.make_norm_la_inputs(1, 5, 2, 4, 6, io="f32", seed=3)
        o_m, _, _ = fn(inp["phq"], inp["phk"], inp["v"])
        q2, k2, v2 = (inp[n].astype(np.float64) for n in ("phq", "phk", "v"))
        for h in range(4):
            o1, _, _ = _run1(q2[0, :, h // 2], k2[0, :, h // 2], v2[0, :, h], fn=fn)
            checks.append(np.array_equal(o1, o_m[0, :, h]))
    except Exception:
        return False
    return all(checks)


def test_pins_pass_on_the_oracle():
    assert _pins_pass(norm_la.recurrent)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name):
    assert not _pins_pass(_mutant(name))
