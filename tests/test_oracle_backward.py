"""Pins of the backward oracle (oracle/backward.py) to what the mathematics
fixes: central finite differences of the forward oracle, torch's
reverse-mode differentiation of an independent fp64 transcription of the
forward step, and two closed forms (the first-order effect of the gates at
beta = 0, and the decay-only case). A planted-mistake check at the end makes
sure the pins catch plausible slips in the backward formulas. CPU only.

The forward step differentiated is the one the pages define: the page
"Uma análise das variantes de atenção linear da família DeltaNet", section
on Gated DeltaNet (forget, predict, correct, write), generalised to the
decoupled gates of "Resumo Técnico: Gated DeltaNet-2", section "Regra de
Atualização".
"""
import importlib.util
import os

import numpy as np
import pytest

import oracle
from oracle import backward as bw_mod

MODES = ["gdn", "kda", "gdn2", "nodecay"]


def _case(mode, rng, B=1, T=4, Hqk=1, Hv=2, d=3, dv=None, S0=True):
    dv = d if dv is None else dv
    q = rng.standard_normal((B, T, Hqk, d))
    k = rng.standard_normal((B, T, Hqk, d))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    q /= np.linalg.norm(q, axis=-1, keepdims=True)
    v = rng.standard_normal((B, T, Hv, dv))
    x = {"q": q, "k": k, "v": v, "g": None, "beta": None, "b": None, "w": None}
    if mode in ("gdn", "nodecay"):
        x["beta"] = 1.0 / (1.0 + np.exp(-rng.standard_normal((B, T, Hv))))
    if mode == "gdn":
        x["g"] = -0.3 * np.log1p(np.exp(rng.standard_normal((B, T, Hv))))
    if mode in ("kda", "gdn2"):
        x["g"] = -0.3 * np.log1p(np.exp(rng.standard_normal((B, T, Hv, d))))
    if mode == "kda":
        x["beta"] = 1.0 / (1.0 + np.exp(-rng.standard_normal((B, T, Hv))))
    if mode == "gdn2":
        x["b"] = 1.0 / (1.0 + np.exp(-rng.standard_normal((B, T, Hv, d))))
        x["w"] = 1.0 / (1.0 + np.exp(-rng.standard_normal((B, T, Hv, dv))))
    x["S0"] = 0.5 * rng.standard_normal((B, Hv, d, dv)) if S0 else None
    x["do"] = rng.standard_normal((B, T, Hv, dv))
    x["dST"] = rng.standard_normal((B, Hv, d, dv))
    return x


def _loss(x, scale):
    o, ST = oracle.recurrent(x["q"], x["k"], x["v"], g=x["g"], beta=x["beta"], b=x["b"], w=x["w"],
                             S0=x["S0"], scale=scale, nthreads=1)
    return float(np.sum(o * x["do"]) + np.sum(ST * x["dST"]))


def _grads(x, scale, mod=bw_mod):
    return mod.recurrent_bwd(x["q"], x["k"], x["v"], g=x["g"], beta=x["beta"], b=x["b"], w=x["w"], S0=x["S0"],
                             do=x["do"], dST=x["dST"], scale=scale)


GRAD_OF = {"q": "dq", "k": "dk", "v": "dv", "g": "dg", "beta": "dbeta", "b": "db", "w": "dw", "S0": "dS0"}


def _fd_check(x, scale, grads, eps=1e-6):
    """Every gradient entry against a central difference of the loss."""
    for name, gname in GRAD_OF.items():
        if x[name] is None:
            continue
        ref = np.empty_like(x[name])
        it = np.nditer(x[name], flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            keep = x[name][idx]
            x[name][idx] = keep + eps
            lp = _loss(x, scale)
            x[name][idx] = keep - eps
            lm = _loss(x, scale)
            x[name][idx] = keep
            ref[idx] = (lp - lm) / (2 * eps)
        got = grads[gname]
        err = np.max(np.abs(got - ref)) / max(np.max(np.abs(ref)), 1e-12)
        assert err < 1e-6, f"{gname}: relative error {err:.2e} against finite differences"


@pytest.mark.parametrize("mode", MODES)
def test_gradients_match_finite_differences(mode):
    rng = np.random.default_rng(10 + MODES.index(mode))
    x = _case(mode, rng)
    _fd_check(x, 0.7, _grads(x, 0.7))


def test_gradients_match_finite_differences_grouped_heads_no_S0():
    rng = np.random.default_rng(20)
    x = _case("gdn", rng, B=2, T=3, Hqk=1, Hv=3, d=2, dv=3, S0=False)
    _fd_check(x, 1.0, _grads(x, 1.0))


def _torch_grads(x, scale):
    """Reverse-mode gradients by torch autograd through an fp64 torch
    transcription of the forward step (independent of oracle/backward.py)."""
    torch = pytest.importorskip("torch")
    tx = {n: (None if a is None else torch.tensor(a, dtype=torch.float64, requires_grad=True))
          for n, a in x.items() if n not in ("do", "dST")}
    q, k, v = tx["q"], tx["k"], tx["v"]
    B, T, Hqk, d = q.shape
    Hv = v.shape[2]
    grp = Hv // Hqk
    loss = 0.0
    for bi in range(B):
        for h in range(Hv):
            S = tx["S0"][bi, h] if tx["S0"] is not None else torch.zeros(d, v.shape[3], dtype=torch.float64)
            for t in range(T):
                kt, qt = k[bi, t, h // grp], q[bi, t, h // grp]
                if tx["g"] is None:
                    S = S
                elif tx["g"].dim() == 4:
                    S = torch.exp(tx["g"][bi, t, h])[:, None] * S
                else:
                    S = torch.exp(tx["g"][bi, t, h]) * S
                if tx["beta"] is not None:
                    e, z = tx["beta"][bi, t, h] * kt, tx["beta"][bi, t, h] * v[bi, t, h]
                else:
                    e, z = tx["b"][bi, t, h] * kt, tx["w"][bi, t, h] * v[bi, t, h]
                S = S + torch.outer(kt, z - S.T @ e)
                loss = loss + scale * torch.dot(S.T @ qt, torch.tensor(x["do"][bi, t, h]))
            loss = loss + torch.sum(S * torch.tensor(x["dST"][bi, h]))
    loss.backward()
    return {GRAD_OF[n]: t.grad.numpy() for n, t in tx.items() if t is not None}


@pytest.mark.parametrize("mode", MODES)
def test_gradients_match_torch_autograd(mode):
    rng = np.random.default_rng(30 + MODES.index(mode))
    x = _case(mode, rng, B=2, T=7, Hqk=2, Hv=4, d=5, dv=4)
    got = _grads(x, 0.5)
    ref = _torch_grads(x, 0.5)
    for name, r in ref.items():
        err = np.max(np.abs(got[name] - r)) / max(np.max(np.abs(r)), 1e-300)
        assert err < 1e-12, f"{name}: {err:.2e}"


def test_first_order_gate_effect_at_beta_zero():
    """beta = 0, alpha = 1: the state never changes, o_t = s S0^T q_t, and
    the loss is linear in the gates at first order. Perturbing beta_t by
    delta adds delta k_t (v_t - S0^T k_t)^T to every state from t on, so
    dL/dbeta_t = sum_{i>=t} s (q_i . k_t) (v_t - S0^T k_t) . do_i
    + <dS_T, k_t (v_t - S0^T k_t)^T>; dq_t = s S0 do_t; dS0 = dS_T +
    s sum_t q_t do_t^T; dk = dv = 0."""
    rng = np.random.default_rng(40)
    x = _case("nodecay", rng, B=1, T=6, Hqk=1, Hv=1, d=4, dv=3)
    x["beta"][:] = 0.0
    s = 0.8
    gr = _grads(x, s)
    q, k, v, S0, do, dST = (x[n][0, :, 0] if n in ("q", "k", "v", "do") else x[n][0, 0]
                            for n in ("q", "k", "v", "S0", "do", "dST"))
    T = q.shape[0]
    for t in range(T):
        r = v[t] - S0.T @ k[t]
        ref = sum(s * (q[i] @ k[t]) * (r @ do[i]) for i in range(t, T)) + np.sum(dST * np.outer(k[t], r))
        assert abs(gr["dbeta"][0, t, 0] - ref) < 1e-12 * max(1.0, abs(ref))
        assert np.allclose(gr["dq"][0, t, 0], s * S0 @ do[t], rtol=0, atol=1e-13)
    assert np.allclose(gr["dS0"][0, 0], dST + s * sum(np.outer(q[t], do[t]) for t in range(T)), rtol=0, atol=1e-13)
    assert not np.any(gr["dk"]) and not np.any(gr["dv"])


def test_decay_only_closed_form():
    """beta = 0 with a scalar decay: S_t = A_t S0 with A_t = exp(sum_{i<=t} g_i),
    so dL/dg_j = sum_{t>=j} s A_t q_t^T S0 do_t + A_{T-1} <dS_T, S0>."""
    rng = np.random.default_rng(41)
    x = _case("gdn", rng, B=1, T=5, Hqk=1, Hv=1, d=3, dv=3)
    x["beta"][:] = 0.0
    s = 1.3
    gr = _grads(x, s)
    g = x["g"][0, :, 0]
    q, S0, do, dST = x["q"][0, :, 0], x["S0"][0, 0], x["do"][0, :, 0], x["dST"][0, 0]
    A = np.exp(np.cumsum(g))
    T = len(g)
    for j in range(T):
        ref = sum(s * A[t] * (q[t] @ S0 @ do[t]) for t in range(j, T)) + A[-1] * np.sum(dST * S0)
        assert abs(gr["dg"][0, j, 0] - ref) < 1e-12 * max(1.0, abs(ref))
    assert np.allclose(gr["dS0"][0, 0], A[-1] * dST + s * sum(A[t] * np.outer(q[t], do[t]) for t in range(T)),
                       rtol=0, atol=1e-12)


def test_head_subset_matches_full():
    rng = np.random.default_rng(42)
    x = _case("gdn2", rng, B=1, T=5, Hqk=1, Hv=3, d=3)
    full = _grads(x, 1.0)
    sub = bw_mod.recurrent_bwd(x["q"], x["k"], x["v"], g=x["g"], b=x["b"], w=x["w"], S0=x["S0"], do=x["do"],
                               dST=x["dST"], heads=[1])
    assert np.array_equal(sub["dv"][:, :, 1], full["dv"][:, :, 1]) and np.all(np.isnan(sub["dv"][:, :, 0]))
    assert np.array_equal(sub["dS0"][:, 1], full["dS0"][:, 1])


# ---- planted mistakes: each must fail at least one finite-difference check ----
SRC = os.path.join(os.path.dirname(oracle.__file__), "backward.py")
MUTANTS = {
    "dq_before_write": ("out[\"dq\"][bi, t, hq] += scale * (St @ dot)", "out[\"dq\"][bi, t, hq] += scale * (Sbar @ dot)"),
    "no_erase_correction": ("dSbar = dS - np.outer(e, du)", "dSbar = dS"),
    "de_sign": ("de = -(Sbar @ du)", "de = Sbar @ du"),
    "dalpha_on_decayed_state": ("dalpha = np.sum(dSbar * prev[t], axis=1)", "dalpha = np.sum(dSbar * Sbar, axis=1)"),
    "state_grad_not_decayed": ("dS = alpha[:, None] * dSbar", "dS = dSbar"),
    "output_grad_missed_by_step": ("dS = dS + scale * np.outer(qt, dot)", "dS_in = dS + scale * np.outer(qt, dot)"),
    "du_from_state": ("du = dS.T @ kt", "du = St.T @ kt"),
    "erase_key_part_dropped": ("dkt = dkt + bt * de", "dkt = dkt"),
    "write_gate_grad_on_k": ("out[\"dw\"][bi, t, h] = v[bi, t, h] * dz", "out[\"dw\"][bi, t, h] = dz"),
}


def _load_mutant(name):
    old, new = MUTANTS[name]
    with open(SRC) as f:
        src = f.read()
    assert src.count(old) == 1, f"snippet for {name} not found"
    path = os.path.join(os.environ.get("TMPDIR", "/tmp"), f"gdr_bwd_{name}_{os.getpid()}.py")
    with open(path, "w") as f:
        f.write(src.replace(old, new).replace("from . import upcast", "from oracle import upcast"))
    try:
        spec = importlib.util.spec_from_file_location(f"gdr_bwd_{name}", path)
        mod = importlib.util.module_from_spec(spec)
        spec.loader.exec_module(mod)
        return mod
    finally:
        os.remove(path)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name):
    mod = _load_mutant(name)
    caught = False
    for mode in MODES:
        rng = np.random.default_rng(50 + MODES.index(mode))
        x = _case(mode, rng, T=3, d=3, dv=2)
        try:
            _fd_check(x, 0.9, _grads(x, 0.9, mod))
        except AssertionError:  # a numerical mismatch, not a crash
            caught = True
            break
    assert caught, f"no pin catches the mutant {name}"
