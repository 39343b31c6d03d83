"""Pins of the CPU oracle to what the pages and the mathematics fix.

Every test here runs on the CPU. None compares the oracle with a retyping of
its own loop: each expected value is a page's worked example, a closed form,
a brute-force sum of a weaker model the recurrence must reduce to, an
autograd gradient, or another page's form of the rule in that page's own
layout (the check-oracles in ``oracle.forms`` / ``oracle.chunked``).

Pages (titles), cited by the short name in brackets:
  [lesson]  "Gated DeltaNet: o mixer em 48 das 64 camadas"
  [family]  "Uma análise das variantes de atenção linear da família DeltaNet"
  [gdn2]    "Resumo Técnico: Gated DeltaNet-2"
"""
import os

import numpy as np
import pytest

from oracle import forms, chunked

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read_golden(name):
    vals = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, *rest = line.split()
            vals[key] = np.array([float(x) for x in rest])
    return vals


def _unit(rng, *shape):
    x = rng.standard_normal(shape)
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def _one_head(x):
    """[T, d] -> [1, T, 1, d] (one sequence, one head)."""
    return x[None, :, None, :]


def _rel(a, b):
    return np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300)


# ---------------------------------------------------------------------------
# [lesson] "Conceito": the capital-city example.

def test_capital_city_delta_rule_returns_new_value(oracle_mod):
    gd = _read_golden("capital_city.txt")
    k = gd["k"]
    q = np.stack([k, k])
    K = np.stack([k, k])
    V = np.stack([gd["v_paris"], gd["v_brasilia"]])
    beta = np.ones((1, 2, 1))
    o, S = oracle_mod.recurrent(_one_head(q), _one_head(K), _one_head(V), beta=beta)
    # Bit-exact: k is a unit basis vector and the values are dyadic.
    assert np.array_equal(o[0, 0, 0], gd["v_paris"])
    assert np.array_equal(o[0, 1, 0], gd["expect_delta_beta1"])


def test_capital_city_additive_returns_superposition():
    gd = _read_golden("capital_city.txt")
    k = gd["k"]
    o, _ = forms.additive_la(np.stack([k, k]), np.stack([k, k]),
                             np.stack([gd["v_paris"], gd["v_brasilia"]]))
    assert np.array_equal(o[1], gd["expect_additive"])


def test_capital_city_every_form_agrees():
    gd = _read_golden("capital_city.txt")
    k = gd["k"]
    K = np.stack([k, k])
    V = np.stack([gd["v_paris"], gd["v_brasilia"]])
    one = np.ones(2)
    ones_k = np.ones((2, 4))
    expect = gd["expect_delta_beta1"]
    for o in (forms.deltanet_residual(K, K, V, one)[0],
              forms.deltanet_expanded(K, K, V, one)[0],
              forms.gdn_four_step(K, K, V, one, one)[0],
              forms.kda_five_step(K, K, V, one, ones_k, 1.0)[0],
              forms.kda_dplr(K, K, V, one, ones_k, 1.0)[0],
              forms.gdn2_matrix(K, K, V, ones_k, ones_k, ones_k)[0]):
        assert np.array_equal(o[1], expect)


def test_capital_city_random_unit_key(oracle_mod):
    rng = np.random.default_rng(1)
    d = 16
    k = _unit(rng, d)
    vP, vB = rng.standard_normal(d), rng.standard_normal(d)
    o, _ = oracle_mod.recurrent(_one_head(np.stack([k, k])), _one_head(np.stack([k, k])),
                                _one_head(np.stack([vP, vB])), beta=np.ones((1, 2, 1)))
    assert np.max(np.abs(o[0, 1, 0] - vB)) <= 8 * np.finfo(float).eps * np.max(np.abs(vB))


# ---------------------------------------------------------------------------
# [family] "DeltaNet: escrever o erro de previsão em vez do valor".

@pytest.mark.parametrize("alpha", [1.0, 0.7])
def test_immediate_reread_closed_form(oracle_mod, alpha):
    """Reading right after a write with the same key gives
    (1 - beta) S~^T k + beta v, S~ the (decayed) state before the write."""
    rng = np.random.default_rng(2)
    dk, dv = 8, 6
    S0 = rng.standard_normal((dk, dv))
    k = _unit(rng, dk)
    v = rng.standard_normal(dv)
    for beta in (0.0, 0.3, 1.0):
        o, _ = oracle_mod.recurrent(_one_head(k[None]), _one_head(k[None]), _one_head(v[None]),
                                    g=np.full((1, 1, 1), np.log(alpha)), beta=np.full((1, 1, 1), beta),
                                    S0=S0[None, None])
        St = alpha * S0
        expect = (1 - beta) * (St.T @ k) + beta * v
        assert _rel(o[0, 0, 0], expect) < 1e-14


def test_update_is_local_to_the_key(oracle_mod):
    """A query orthogonal to the written key sees no change; only the key
    direction of the state moves ([family], locality of the update; its
    "Transição de estado estruturada": eigenvalue 1 - beta along k, 1 elsewhere)."""
    rng = np.random.default_rng(3)
    dk, dv = 8, 5
    S0 = rng.standard_normal((dk, dv))
    k = _unit(rng, dk)
    x = rng.standard_normal(dk)
    x -= (x @ k) * k
    x /= np.linalg.norm(x)
    v = rng.standard_normal(dv)
    beta = 0.6
    o, S = oracle_mod.recurrent(_one_head(x[None]), _one_head(k[None]), _one_head(v[None]),
                                beta=np.full((1, 1, 1), beta), S0=S0[None, None])
    assert _rel(o[0, 0, 0], S0.T @ x) < 1e-14
    # Eigenstructure of the transition, seen through the state with v = 0:
    c = rng.standard_normal(dv)
    for direction, factor in ((k, 1 - beta), (x, 1.0)):
        _, S = oracle_mod.recurrent(_one_head(k[None]), _one_head(k[None]), _one_head(np.zeros((1, dv))),
                                    beta=np.full((1, 1, 1), beta),
                                    S0=np.outer(direction, c)[None, None])
        assert _rel(S[0, 0], factor * np.outer(direction, c)) < 1e-14


# ---------------------------------------------------------------------------
# No-op and decay-only closed forms.

def test_beta_zero_alpha_one_is_noop(oracle_mod):
    rng = np.random.default_rng(4)
    T, dk, dv = 9, 8, 8
    S0 = rng.standard_normal((1, 1, dk, dv))
    q, k, v = _unit(rng, 1, T, 1, dk), _unit(rng, 1, T, 1, dk), rng.standard_normal((1, T, 1, dv))
    o, S = oracle_mod.recurrent(q, k, v, beta=np.zeros((1, T, 1)), S0=S0)
    assert np.array_equal(S, S0)
    assert _rel(o[0, :, 0], q[0, :, 0] @ S0[0, 0]) < 1e-14
    # Gated DeltaNet-2 with both gates closed, alpha = 1 (g = 0): also a no-op.
    o2, S2 = oracle_mod.recurrent(q, k, v, g=np.zeros((1, T, 1, dk)), b=np.zeros((1, T, 1, dk)),
                                  w=np.zeros((1, T, 1, dv)), S0=S0)
    assert np.array_equal(S2, S0)


@pytest.mark.parametrize("mode", ["scalar", "channel"])
def test_decay_only_closed_form(oracle_mod, mode):
    """beta = 0: the state only decays, S_T = Diag(prod_t alpha_t) S_0."""
    rng = np.random.default_rng(5)
    T, dk, dv = 12, 8, 4
    S0 = rng.standard_normal((1, 1, dk, dv))
    q, k, v = _unit(rng, 1, T, 1, dk), _unit(rng, 1, T, 1, dk), rng.standard_normal((1, T, 1, dv))
    if mode == "scalar":
        alpha = rng.uniform(0.5, 1.0, (1, T, 1))
        prod = np.prod(alpha[0, :, 0]) * np.ones(dk)
    else:
        alpha = rng.uniform(0.5, 1.0, (1, T, 1, dk))
        prod = np.prod(alpha[0, :, 0], axis=0)
    _, S = oracle_mod.recurrent(q, k, v, g=np.log(alpha), beta=np.zeros((1, T, 1)), S0=S0)
    assert _rel(S[0, 0], prod[:, None] * S0[0, 0]) < 1e-13


# ---------------------------------------------------------------------------
# Linear-attention limits ([family] "Da atenção de complexidade quadrática ao
# estado linear": o_t = sum_{i<=t} <k_i, q_t> v_i).

def test_small_beta_limit_is_linear_attention(oracle_mod):
    rng = np.random.default_rng(6)
    T, dk, dv = 16, 8, 8
    q, k = _unit(rng, T, dk), _unit(rng, T, dk)
    v = rng.standard_normal((T, dv))
    beta = 1e-8
    o, _ = oracle_mod.recurrent(_one_head(q), _one_head(k), _one_head(v), beta=np.full((1, T, 1), beta))
    brute = np.zeros((T, dv))
    for t in range(T):
        for i in range(t + 1):
            brute[t] += np.dot(k[i], q[t]) * v[i]
    assert _rel(o[0, :, 0] / beta, brute) < 1e-6


def test_orthonormal_keys_make_delta_additive(oracle_mod):
    """With orthonormal keys every prediction S~^T k_t is 0, so the delta rule
    writes beta_t v_t unchanged: S_T = sum_i beta_i (prod_{m>i} alpha_m) k_i v_i^T."""
    rng = np.random.default_rng(7)
    dk, dv, T = 8, 5, 8
    Qm, _ = np.linalg.qr(rng.standard_normal((dk, dk)))
    k = Qm.T[:T]
    q = _unit(rng, T, dk)
    v = rng.standard_normal((T, dv))
    beta = rng.uniform(0.1, 1.0, T)
    alpha = rng.uniform(0.5, 1.0, T)
    o, S = oracle_mod.recurrent(_one_head(q), _one_head(k), _one_head(v), g=np.log(alpha)[None, :, None],
                                beta=beta[None, :, None])
    expect_S = sum(beta[i] * np.prod(alpha[i + 1:]) * np.outer(k[i], v[i]) for i in range(T))
    assert _rel(S[0, 0], expect_S) < 1e-14
    for t in range(T):
        expect_o = sum(beta[i] * np.prod(alpha[i + 1:t + 1]) * np.dot(k[i], q[t]) * v[i]
                       for i in range(t + 1))
        assert _rel(o[0, t, 0], expect_o) < 1e-13


# ---------------------------------------------------------------------------
# [family] "Derivando a partir da perda de reconstrução": the update is one
# gradient step of size beta on 1/2 ||S~^T k - v||^2 from the decayed state.

@pytest.mark.parametrize("mode", ["scalar", "channel"])
def test_gradient_step_view(oracle_mod, mode):
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(8)
    T, dk, dv = 10, 6, 5
    q, k = _unit(rng, T, dk), _unit(rng, T, dk)
    v = rng.standard_normal((T, dv))
    beta = rng.uniform(0, 1, T)
    alpha = rng.uniform(0.6, 1.0, (T,) if mode == "scalar" else (T, dk))
    S0 = rng.standard_normal((dk, dv))
    S = torch.tensor(S0, dtype=torch.float64)
    outs = []
    for t in range(T):
        a = torch.tensor(alpha[t], dtype=torch.float64)
        St = (a * S) if mode == "scalar" else (a[:, None] * S)
        St = St.detach().requires_grad_(True)
        kt = torch.tensor(k[t], dtype=torch.float64)
        loss = 0.5 * torch.sum((St.T @ kt - torch.tensor(v[t], dtype=torch.float64)) ** 2)
        (grad,) = torch.autograd.grad(loss, St)
        S = (St - beta[t] * grad).detach()
        outs.append((S.T @ torch.tensor(q[t], dtype=torch.float64)).numpy())
    g = np.log(alpha)[None, :, None] if mode == "scalar" else np.log(alpha)[None, :, None, :]
    o, ST = oracle_mod.recurrent(_one_head(q), _one_head(k), _one_head(v), g=g,
                                 beta=beta[None, :, None], S0=S0[None, None])
    assert _rel(ST[0, 0], S.numpy()) < 1e-13
    assert _rel(o[0, :, 0], np.stack(outs)) < 1e-13


# ---------------------------------------------------------------------------
# Other pages' forms, each in its own layout.

def _rand_case(rng, T=11, dk=8, dv=6):
    q, k = _unit(rng, T, dk), _unit(rng, T, dk)
    v = rng.standard_normal((T, dv))
    beta = rng.uniform(0, 1, T)
    alpha_s = rng.uniform(0.5, 1.0, T)
    alpha_c = rng.uniform(0.5, 1.0, (T, dk))
    bg = rng.uniform(0, 1, (T, dk))
    wg = rng.uniform(0, 1, (T, dv))
    S0 = rng.standard_normal((dk, dv))
    return q, k, v, beta, alpha_s, alpha_c, bg, wg, S0


def test_deltanet_forms(oracle_mod):
    rng = np.random.default_rng(9)
    q, k, v, beta, *_, S0 = _rand_case(rng)
    o, S = oracle_mod.recurrent(_one_head(q), _one_head(k), _one_head(v), beta=beta[None, :, None],
                                S0=S0[None, None])
    for f in (forms.deltanet_residual, forms.deltanet_expanded):
        of, Sf = f(q, k, v, beta, S0.T)
        assert _rel(o[0, :, 0], of) < 1e-13
        assert _rel(S[0, 0], Sf.T) < 1e-13


def test_gated_deltanet_four_step(oracle_mod):
    rng = np.random.default_rng(10)
    q, k, v, beta, alpha_s, *_, S0 = _rand_case(rng)
    of, Sf = forms.gdn_four_step(q, k, v, beta, alpha_s, S0.T)
    # Scalar-decay mode, and per-channel mode with every channel equal
    # ([gdn2] "Regra Delta Portão-2": scalar decay recovers Gated DeltaNet).
    for g in (np.log(alpha_s)[None, :, None],
              np.repeat(np.log(alpha_s)[:, None], k.shape[1], axis=1)[None, :, None, :]):
        o, S = oracle_mod.recurrent(_one_head(q), _one_head(k), _one_head(v), g=g,
                                    beta=beta[None, :, None], S0=S0[None, None])
        assert _rel(o[0, :, 0], of) < 1e-13
        assert _rel(S[0, 0], Sf.T) < 1e-13


def test_kda_five_step_and_dplr(oracle_mod):
    rng = np.random.default_rng(11)
    q, k, v, beta, _, alpha_c, *_, S0 = _rand_case(rng)
    scale = k.shape[1] ** -0.5
    of, Sf = forms.kda_five_step(q, k, v, beta, alpha_c, scale, S0.T)
    od, Sd = forms.kda_dplr(q, k, v, beta, alpha_c, scale, S0.T)
    assert _rel(od, of) < 1e-13 and _rel(Sd, Sf) < 1e-13
    o, S = oracle_mod.recurrent(_one_head(q), _one_head(k), _one_head(v), g=np.log(alpha_c)[None, :, None, :],
                                beta=beta[None, :, None], scale=scale, S0=S0[None, None])
    assert _rel(o[0, :, 0], of) < 1e-13
    assert _rel(S[0, 0], Sf.T) < 1e-13


def test_gdn2_literal_matrix_form(oracle_mod):
    rng = np.random.default_rng(12)
    q, k, v, _, _, alpha_c, bg, wg, S0 = _rand_case(rng)
    of, Sf = forms.gdn2_matrix(q, k, v, alpha_c, bg, wg, 1.0, S0)
    o, S = oracle_mod.recurrent(_one_head(q), _one_head(k), _one_head(v), g=np.log(alpha_c)[None, :, None, :],
                                b=bg[None, :, None], w=wg[None, :, None], S0=S0[None, None])
    assert _rel(o[0, :, 0], of) < 1e-13
    assert _rel(S[0, 0], Sf) < 1e-13


def test_gdn2_tied_gates_is_kda(oracle_mod):
    """[gdn2] "Regra Delta Portão-2": b = w = beta 1 recovers KDA."""
    rng = np.random.default_rng(13)
    q, k, v, beta, _, alpha_c, *_, S0 = _rand_case(rng)
    dk, dv = k.shape[1], v.shape[1]
    bg = np.repeat(beta[:, None], dk, axis=1)
    wg = np.repeat(beta[:, None], dv, axis=1)
    om, Sm = forms.gdn2_matrix(q, k, v, alpha_c, bg, wg, 1.0, S0)
    of, Sf = forms.kda_five_step(q, k, v, beta, alpha_c, 1.0, S0.T)
    assert _rel(om, of) < 1e-13 and _rel(Sm, Sf.T) < 1e-13
    o, S = oracle_mod.recurrent(_one_head(q), _one_head(k), _one_head(v), g=np.log(alpha_c)[None, :, None, :],
                                b=bg[None, :, None], w=wg[None, :, None], S0=S0[None, None])
    assert _rel(o[0, :, 0], of) < 1e-13 and _rel(S[0, 0], Sf.T) < 1e-13


# ---------------------------------------------------------------------------
# The chunked schedule equals the sequential one ([family] "Chunkwise KDA";
# [gdn2] "Treinamento Paralelo Eficiente por Blocos").

@pytest.mark.parametrize("C", [1, 3, 16, 64])
@pytest.mark.parametrize("mode", ["gdn", "kda", "gdn2", "deltanet"])
def test_chunked_equals_sequential(oracle_mod, C, mode):
    rng = np.random.default_rng(14 + C)
    T, dk, dv = 100, 8, 6
    q, k, v, beta, alpha_s, alpha_c, bg, wg, S0 = _rand_case(rng, T, dk, dv)
    scale = 0.5
    kw = dict(scale=scale, S0=S0[None, None])
    if mode == "gdn":
        g = np.log(alpha_s)
        kw.update(g=g[None, :, None], beta=beta[None, :, None])
        gc = np.repeat(g[:, None], dk, axis=1)
        e, z = beta[:, None] * k, beta[:, None] * v
    elif mode == "deltanet":
        kw.update(beta=beta[None, :, None])
        gc = np.zeros((T, dk))
        e, z = beta[:, None] * k, beta[:, None] * v
    elif mode == "kda":
        gc = np.log(alpha_c)
        kw.update(g=gc[None, :, None, :], beta=beta[None, :, None])
        e, z = beta[:, None] * k, beta[:, None] * v
    else:
        gc = np.log(alpha_c)
        kw.update(g=gc[None, :, None, :], b=bg[None, :, None], w=wg[None, :, None])
        e, z = bg * k, wg * v
    o, S = oracle_mod.recurrent(_one_head(q), _one_head(k), _one_head(v), **kw)
    for f in (chunked.chunked_provisional, chunked.chunked_wy):
        oc, Sc = f(q, k, e, z, gc, scale, S0, C)
        assert _rel(oc, o[0, :, 0]) < 1e-12, f.__name__
        assert _rel(Sc, S[0, 0]) < 1e-12, f.__name__


# ---------------------------------------------------------------------------
# Structure: state passing, value-column independence, read scale, head groups.

def _multi(rng, B=2, T=20, Hqk=2, Hv=6, dk=8, dv=8, channel=True, bw=False):
    d = dict(q=_unit(rng, B, T, Hqk, dk), k=_unit(rng, B, T, Hqk, dk), v=rng.standard_normal((B, T, Hv, dv)))
    d["g"] = np.log(rng.uniform(0.6, 1, (B, T, Hv, dk) if channel else (B, T, Hv)))
    if bw:
        d["b"] = rng.uniform(0, 1, (B, T, Hv, dk))
        d["w"] = rng.uniform(0, 1, (B, T, Hv, dv))
    else:
        d["beta"] = rng.uniform(0, 1, (B, T, Hv))
    d["S0"] = rng.standard_normal((B, Hv, dk, dv))
    return d


@pytest.mark.parametrize("bw", [False, True])
def test_split_resume(oracle_mod, bw):
    rng = np.random.default_rng(20)
    d = _multi(rng, bw=bw)
    o, S = oracle_mod.recurrent(**d)
    T1 = 7
    first = {n: (a[:, :T1] if n != "S0" else a) for n, a in d.items()}
    second = {n: (a[:, T1:] if n != "S0" else a) for n, a in d.items()}
    o1, S1 = oracle_mod.recurrent(**first)
    second["S0"] = S1
    o2, S2 = oracle_mod.recurrent(**second)
    assert np.array_equal(np.concatenate([o1, o2], axis=1), o)
    assert np.array_equal(S2, S)


def test_column_and_head_subsets(oracle_mod):
    rng = np.random.default_rng(21)
    d = _multi(rng, dv=24)
    o, S = oracle_mod.recurrent(**d)
    os_, Ss = oracle_mod.recurrent(**d, heads=[1, 4], cols=(5, 19))
    assert np.array_equal(os_[:, :, [1, 4], 5:19], o[:, :, [1, 4], 5:19])
    assert np.array_equal(Ss[:, [1, 4], :, 5:19], S[:, [1, 4], :, 5:19])
    assert np.all(np.isnan(os_[:, :, 0])) and np.all(np.isnan(os_[:, :, 1, :5]))


def test_read_scale_is_linear(oracle_mod):
    rng = np.random.default_rng(22)
    d = _multi(rng)
    o1, S1 = oracle_mod.recurrent(**d, scale=1.0)
    o3, S3 = oracle_mod.recurrent(**d, scale=0.125)
    assert np.array_equal(S1, S3)
    assert np.array_equal(o3, 0.125 * o1)      # exact: power-of-two scale


def test_qk_head_serves_contiguous_v_heads(oracle_mod):
    """[lesson] "Conceito": each QK head serves three V heads; V head h reads
    QK head h // 3 here. Each V head must equal a one-head run on its QK head."""
    rng = np.random.default_rng(23)
    d = _multi(rng, B=1, Hqk=2, Hv=6)
    o, S = oracle_mod.recurrent(**d)
    for h in range(6):
        hq = h // 3
        one = dict(q=d["q"][:, :, hq:hq + 1], k=d["k"][:, :, hq:hq + 1], v=d["v"][:, :, h:h + 1],
                   g=d["g"][:, :, h:h + 1], beta=d["beta"][:, :, h:h + 1], S0=d["S0"][:, h:h + 1])
        oh, Sh = oracle_mod.recurrent(**one)
        assert np.array_equal(oh[:, :, 0], o[:, :, h])
        assert np.array_equal(Sh[:, 0], S[:, h])


def test_bf16_upcast_is_exact(oracle_mod):
    bits = np.array([0x3F80, 0xC000, 0x3F81, 0x0000, 0x8000, 0x7F7F], dtype=np.uint16)
    x = oracle_mod.upcast(bits)
    assert x[0] == 1.0 and x[1] == -2.0 and x[2] == 1.0 + 2.0 ** -7 and x[3] == 0.0
    assert np.signbit(x[4]) and x[5] == (2 - 2.0 ** -7) * 2.0 ** 127


def test_oracle_rejects_bad_arguments(oracle_mod):
    rng = np.random.default_rng(24)
    d = _multi(rng, B=1, T=3)
    with pytest.raises(ValueError):
        oracle_mod.recurrent(**{**d, "g": np.abs(d["g"]) + 0.1})      # alpha > 1
    with pytest.raises(ValueError):
        oracle_mod.recurrent(**d, b=np.ones((1, 3, 6, 8)), w=np.ones((1, 3, 6, 8)))
    with pytest.raises(RuntimeError):
        oracle_mod.recurrent(**d, cols=(4, 4))
