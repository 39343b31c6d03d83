"""Gradients of the gated delta-rule recurrence on the CPU in fp64.

TEST INFRASTRUCTURE, like the rest of ``oracle/``: only ``tests/``,
``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline`` leg may use
it, and it shares no code with the GPU library.

What is differentiated. The page "Resumo Técnico: Gated DeltaNet-2", section
"Treinamento Paralelo Eficiente por Blocos", names a gate-aware backward pass
(the per-channel gates b and w enter the gradient accumulation) but prints
no formula. The plain reading: the exact gradient of the forward recurrence
the oracle computes (``oracle.recurrent``), for a scalar loss whose
gradients with respect to the outputs are given, do = dL/do and dS_T =
dL/dS_T. Per (sequence, V head), with the forward step

    Sbar_t = Diag(alpha_t) S_{t-1}          alpha_t = exp(g_t)
    u_t    = z_t - Sbar_t^T e_t             e_t = beta_t k_t  or  b_t . k_t
    S_t    = Sbar_t + k_t u_t^T             z_t = beta_t v_t  or  w_t . v_t
    o_t    = s S_t^T q_t

reverse-mode differentiation gives, walking t = T-1 .. 0 with dS = dS_T:

    dS    += s q_t do_t^T                   (o_t reads S_t)
    dq_t   = s S_t do_t
    du_t   = dS^T k_t                       (S_t = Sbar_t + k_t u_t^T)
    dk_t   = dS u_t  (+ the erase-key part below)
    dSbar  = dS - e_t du_t^T                (u_t = z_t - Sbar_t^T e_t)
    de_t   = -Sbar_t du_t,   dz_t = du_t
    dalpha = rowsum(dSbar . S_{t-1}),  dg_t = alpha_t . dalpha  (summed over
             channels for a scalar decay)
    dS     = Diag(alpha_t) dSbar            (the gradient reaching S_{t-1})

then through the gates: tied, dbeta_t = k_t . de_t + v_t . dz_t (dot
products), dk_t += beta_t de_t, dv_t = beta_t dz_t; decoupled, db_t = k_t . de_t,
dk_t += b_t . de_t, dw_t = v_t . dz_t, dv_t = w_t . dz_t. Queries and keys
shared by several V heads (grouped heads) sum the gradients of those heads.
dS_0 is the dS left after t = 0.

Nothing here is pinned by printing it again: the tests check these
gradients against central finite differences of ``oracle.recurrent`` and
against torch's reverse-mode differentiation of an independent fp64 torch
transcription of the forward step.
"""
from __future__ import annotations

import numpy as np

from . import upcast


def recurrent_bwd(q, k, v, *, g=None, beta=None, b=None, w=None, scale=1.0, S0=None, do=None, dST=None,
                  heads=None):
    """Gradients of the recurrence (fp64).

    Inputs as ``oracle.recurrent`` (stored dtypes widened exactly), plus
    ``do`` [B,T,Hv,dv] (None: zeros) and ``dST`` [B,Hv,dk,dv] (None: zeros).
    ``heads``: V heads whose gradients are formed (default all); the others
    contribute nothing (their dv, dg, dbeta, db, dw, dS0 entries are NaN, and
    dq, dk hold only the selected heads' parts).

    Returns a dict with dq, dk [B,T,Hqk,dk]; dv [B,T,Hv,dv]; dg (shape of g,
    or None); dbeta [B,T,Hv] (tied gates) or db [B,T,Hv,dk] and dw [B,T,Hv,dv]
    (decoupled gates); dS0 [B,Hv,dk,dv].
    """
    q, k, v = (upcast(x) for x in (q, k, v))
    B, T, Hqk, dk = q.shape
    Hv, dv = v.shape[2], v.shape[3]
    grp = Hv // Hqk
    g = upcast(g)
    per_channel = g is not None and g.ndim == 4
    tied = beta is not None
    beta, b, w = upcast(beta), upcast(b), upcast(w)
    S0 = np.zeros((B, Hv, dk, dv)) if S0 is None else upcast(S0)
    do = np.zeros((B, T, Hv, dv)) if do is None else upcast(do)
    dST = np.zeros((B, Hv, dk, dv)) if dST is None else upcast(dST)
    hl = range(Hv) if heads is None else heads

    out = {"dq": np.zeros((B, T, Hqk, dk)), "dk": np.zeros((B, T, Hqk, dk)), "dv": np.full((B, T, Hv, dv), np.nan),
           "dg": None if g is None else np.full(g.shape, np.nan), "dS0": np.full((B, Hv, dk, dv), np.nan)}
    if tied:
        out["dbeta"] = np.full((B, T, Hv), np.nan)
    else:
        out["db"] = np.full((B, T, Hv, dk), np.nan)
        out["dw"] = np.full((B, T, Hv, dv), np.nan)

    for bi in range(B):
        for h in hl:
            hq = h // grp
            # Forward, keeping every state entering a step and every u_t.
            S = S0[bi, h].copy()
            prev = np.empty((T, dk, dv))
            us = np.empty((T, dv))
            alphas = np.empty((T, dk))
            es = np.empty((T, dk))
            for t in range(T):
                prev[t] = S
                if g is None:
                    alpha = np.ones(dk)
                elif per_channel:
                    alpha = np.exp(g[bi, t, h])
                else:
                    alpha = np.full(dk, np.exp(g[bi, t, h]))
                kt = k[bi, t, hq]
                e = beta[bi, t, h] * kt if tied else b[bi, t, h] * kt
                z = beta[bi, t, h] * v[bi, t, h] if tied else w[bi, t, h] * v[bi, t, h]
                Sbar = alpha[:, None] * S
                u = z - Sbar.T @ e
                S = Sbar + np.outer(kt, u)
                us[t], alphas[t], es[t] = u, alpha, e
            # Backward.
            dS = dST[bi, h].copy()
            for t in range(T - 1, -1, -1):
                kt, qt, dot = k[bi, t, hq], q[bi, t, hq], do[bi, t, h]
                alpha, e, u = alphas[t], es[t], us[t]
                Sbar = alpha[:, None] * prev[t]
                St = Sbar + np.outer(kt, u)
                dS = dS + scale * np.outer(qt, dot)
                out["dq"][bi, t, hq] += scale * (St @ dot)
                du = dS.T @ kt
                dkt = dS @ u
                dSbar = dS - np.outer(e, du)
                de = -(Sbar @ du)
                dz = du
                dalpha = np.sum(dSbar * prev[t], axis=1)
                if g is not None:
                    if per_channel:
                        out["dg"][bi, t, h] = alpha * dalpha
                    else:
                        out["dg"][bi, t, h] = alpha[0] * np.sum(dalpha)
                if tied:
                    bt = beta[bi, t, h]
                    out["dbeta"][bi, t, h] = kt @ de + v[bi, t, h] @ dz
                    dkt = dkt + bt * de
                    out["dv"][bi, t, h] = bt * dz
                else:
                    out["db"][bi, t, h] = kt * de
                    dkt = dkt + b[bi, t, h] * de
                    out["dw"][bi, t, h] = v[bi, t, h] * dz
                    out["dv"][bi, t, h] = w[bi, t, h] * dz
                out["dk"][bi, t, hq] += dkt
                dS = alpha[:, None] * dSbar
            out["dS0"][bi, h] = dS
    return out
