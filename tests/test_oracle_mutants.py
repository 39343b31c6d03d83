"""Planted mistakes: the pins must catch every plausible slip in the oracle.

Each case below copies ``oracle/gdr_oracle.c``, replaces one snippet with a
plausible mistake (a dropped term, a wrong sign, a wrong vector or index, a
transposed operand), compiles the copy with gcc into a temporary directory,
and runs a battery of pin checks against it. The unmodified source must pass
every check and each mutant must fail at least one. Everything runs on the
CPU; nothing here touches the GPU library.

Pins used (pages cited by short name as in ``test_oracle_pins``):
capital-city example ([lesson] "Conceito"), immediate re-read closed form
([family] DeltaNet section), decay-only closed form, Gated DeltaNet four-step
and KDA five-step forms in [family]'s layout, the Gated DeltaNet-2 update
equation as a literal matrix product ([gdn2] "Regra Delta Portão-2"), the
QK-to-V head grouping ([lesson] "Conceito").
"""
import os
import subprocess

import numpy as np
import pytest

import oracle
from oracle import forms

SRC = os.path.join(os.path.dirname(oracle.__file__), "gdr_oracle.c")

MUTANTS = {
    "forget_dropped": ("S[(size_t)i * nc + j] *= alpha[i];", ";"),
    "correct_sign": ("u[j] = z[j] - r;", "u[j] = z[j] + r;"),
    "write_along_e": ("S[(size_t)i * nc + j] += kt[i] * u[j];", "S[(size_t)i * nc + j] += e[i] * u[j];"),
    "read_with_k": ("r += S[(size_t)i * nc + j] * qt[i];", "r += S[(size_t)i * nc + j] * kt[i];"),
    "qk_group_index": ("const int hq = h / group;", "const int hq = h % J->Hqk;"),
    "write_gate_dropped": ("z[j] = ww[c0 + j] * vt[c0 + j];", "z[j] = vt[c0 + j];"),
    "erase_gate_dropped": ("e[i] = bb[i] * kt[i];", "e[i] = kt[i];"),
    "erase_gate_on_value_axis": ("e[i] = bb[i] * kt[i];", "e[i] = ww[i] * kt[i];"),
    "channel_decay_reversed": ("alpha[i] = exp(J->g[(bt * J->Hv + h) * dk + i]);",
                               "alpha[i] = exp(J->g[(bt * J->Hv + h) * dk + (dk - 1 - i)]);"),
    "scalar_decay_half": ("alpha[i] = exp(J->g[bt * J->Hv + h]);",
                          "alpha[i] = exp(0.5 * J->g[bt * J->Hv + h]);"),
    "scale_ignored": ("ot[c0 + j] = J->scale * r;", "ot[c0 + j] = r;"),
    "beta_erase_dropped": ("for (int i = 0; i < dk; ++i) e[i] = bt_ * kt[i];",
                           "for (int i = 0; i < dk; ++i) e[i] = kt[i];"),
    "beta_write_dropped": ("for (int j = 0; j < nc; ++j) z[j] = bt_ * vt[c0 + j];",
                           "for (int j = 0; j < nc; ++j) z[j] = vt[c0 + j];"),
    "S0_transposed": ("J->S0[(((size_t)b * J->Hv + h) * dk + i) * dv + c0 + j]",
                      "J->S0[(((size_t)b * J->Hv + h) * dv + c0 + j) * dk + i]"),
    "write_dropped": ("""        /* Write: S = Sbar + k u^T. */
        for (int i = 0; i < dk; ++i)
            for (int j = 0; j < nc; ++j) S[(size_t)i * nc + j] += kt[i] * u[j];
""", ""),
}

_WRITE = """        /* Write: S = Sbar + k u^T. */
        for (int i = 0; i < dk; ++i)
            for (int j = 0; j < nc; ++j) S[(size_t)i * nc + j] += kt[i] * u[j];
"""
_READ = """        /* Read after write: o_t = scale * S^T q_t. */
        double *ot = J->o + (bt * J->Hv + h) * dv;
        for (int j = 0; j < nc; ++j) {
            double r = 0.0;
            for (int i = 0; i < dk; ++i) r += S[(size_t)i * nc + j] * qt[i];
            ot[c0 + j] = J->scale * r;
        }
"""
# The read moved before the write (the output would miss the token's own write).
MUTANTS["read_before_write"] = (_WRITE + "\n" + _READ, _READ + "\n" + _WRITE)


def _build(tmp_path, name, src_text):
    c = tmp_path / f"{name}.c"
    c.write_text(src_text)
    so = tmp_path / f"lib{name}.so"
    subprocess.run(["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fPIC", "-shared", "-pthread",
                    str(c), "-o", str(so), "-lm"], check=True)
    return oracle.load_library(str(so))


def _unit(rng, *shape):
    x = rng.standard_normal(shape)
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def _rel(a, b):
    return np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300)


def _pin_failures(lib):
    """Run the pin battery with ``lib``; return the names of the pins that fail.
    A read-before-write mutant is caught by the re-read closed form; the
    'write dropped' one by the capital-city example; and so on."""
    bad = []
    rng = np.random.default_rng(99)
    one = lambda x: x[None, :, None, :]
    R = lambda *a, **kw: oracle.recurrent(*a, lib=lib, nthreads=2, **kw)

    # Capital city, beta = 1: reading the key returns the newest value.
    k = np.array([1.0, 0, 0, 0])
    vP, vB = np.array([0.5, -1.25, 2.0, 0.75]), np.array([-0.25, 1.5, 0.125, -3.0])
    o, _ = R(one(np.stack([k, k])), one(np.stack([k, k])), one(np.stack([vP, vB])), beta=np.ones((1, 2, 1)))
    if not np.array_equal(o[0, 1, 0], vB):
        bad.append("capital_city")

    # Immediate re-read from a random state with decay.
    dk, dv = 8, 8
    S0 = rng.standard_normal((dk, dv))
    kk = _unit(rng, dk)
    v = rng.standard_normal(dv)
    beta, alpha = 0.3, 0.7
    o, _ = R(one(kk[None]), one(kk[None]), one(v[None]), g=np.full((1, 1, 1), np.log(alpha)),
             beta=np.full((1, 1, 1), beta), S0=S0[None, None])
    if not _rel(o[0, 0, 0], (1 - beta) * (alpha * S0).T @ kk + beta * v) < 1e-13:
        bad.append("reread")

    # Forms of the other pages, random multi-token cases.
    T = 9
    q, kk = _unit(rng, T, dk), _unit(rng, T, dk)
    vv = rng.standard_normal((T, dv))
    bt = rng.uniform(0, 1, T)
    a_s = rng.uniform(0.5, 1, T)
    a_c = rng.uniform(0.5, 1, (T, dk))
    bg, wg = rng.uniform(0, 1, (T, dk)), rng.uniform(0, 1, (T, dv))
    S0 = rng.standard_normal((dk, dv))
    of, Sf = forms.gdn_four_step(q, kk, vv, bt, a_s, S0.T)
    o, S = R(one(q), one(kk), one(vv), g=np.log(a_s)[None, :, None], beta=bt[None, :, None], S0=S0[None, None])
    if not (_rel(o[0, :, 0], of) < 1e-12 and _rel(S[0, 0], Sf.T) < 1e-12):
        bad.append("gdn_four_step")
    sc = dk ** -0.5
    of, Sf = forms.kda_five_step(q, kk, vv, bt, a_c, sc, S0.T)
    o, S = R(one(q), one(kk), one(vv), g=np.log(a_c)[None, :, None, :], beta=bt[None, :, None], scale=sc,
             S0=S0[None, None])
    if not (_rel(o[0, :, 0], of) < 1e-12 and _rel(S[0, 0], Sf.T) < 1e-12):
        bad.append("kda_five_step")
    of, Sf = forms.gdn2_matrix(q, kk, vv, a_c, bg, wg, 1.0, S0)
    o, S = R(one(q), one(kk), one(vv), g=np.log(a_c)[None, :, None, :], b=bg[None, :, None],
             w=wg[None, :, None], S0=S0[None, None])
    if not (_rel(o[0, :, 0], of) < 1e-12 and _rel(S[0, 0], Sf) < 1e-12):
        bad.append("gdn2_matrix")

    # Head grouping: V head h of a (Hqk=2, Hv=6) run equals a one-head run on QK head h // 3.
    B, Hq, Hv = 1, 2, 6
    Q, K = _unit(rng, B, T, Hq, dk), _unit(rng, B, T, Hq, dk)
    V = rng.standard_normal((B, T, Hv, dv))
    Bt = rng.uniform(0, 1, (B, T, Hv))
    o, _ = R(Q, K, V, beta=Bt)
    for h in range(Hv):
        oh, _ = R(Q[:, :, h // 3:h // 3 + 1], K[:, :, h // 3:h // 3 + 1], V[:, :, h:h + 1], beta=Bt[:, :, h:h + 1])
        if not np.array_equal(oh[:, :, 0], o[:, :, h]):
            bad.append("grouping")
            break
    return bad


def test_unmodified_oracle_passes_battery(tmp_path):
    lib = _build(tmp_path, "orig", open(SRC).read())
    assert _pin_failures(lib) == []


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(tmp_path, name):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) >= 1, f"snippet for {name} not found in the oracle source"
    lib = _build(tmp_path, name, src.replace(old, new, 1))
    assert _pin_failures(lib), f"mutant {name} passed every pin"
