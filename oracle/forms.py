"""Check-oracles: each is one page's own statement of a rule, written out
literally, in that page's layout, for a single head and tiny sizes (fp64).

TEST INFRASTRUCTURE (see the package docstring). These functions exist to pin
the production oracle (``oracle.recurrent``): every one of them is an
independent route to the same numbers -- a different layout, a different
algebraic form (expanded matrix, DPLR, explicit d_k x d_k transition), or a
weaker model whose result the recurrence must reduce to.

Pages (titles), cited by the short name in brackets:
  [family]  "Uma análise das variantes de atenção linear da família DeltaNet"
  [gdn2]    "Resumo Técnico: Gated DeltaNet-2"
  [lesson]  "Gated DeltaNet: o mixer em 48 das 64 camadas"

Layouts. [family] stores the state as S' in R^{d_v x d_k} and reads S' q.
[gdn2] stores S in R^{d_k x d_v} and reads S^T q. They hold the same numbers
(S' = S^T); each function below keeps its page's layout and says which.
All inputs are fp64 arrays: q, k [T, d_k]; v [T, d_v]; beta [T];
alpha [T] (scalar) or [T, d_k] (per channel).
"""
from __future__ import annotations

import numpy as np


def additive_la(q, k, v, S0p=None):
    """Unnormalised linear attention, [family] "Da atenção de complexidade
    quadrática ao estado linear": S'_t = S'_{t-1} + v_t k_t^T, o_t = S'_t q_t.
    Layout d_v x d_k. Returns (o [T,d_v], S'_T)."""
    T, dk = k.shape
    dv = v.shape[1]
    S = np.zeros((dv, dk)) if S0p is None else S0p.copy()
    o = np.zeros((T, dv))
    for t in range(T):
        S = S + np.outer(v[t], k[t])
        o[t] = S @ q[t]
    return o, S


def deltanet_residual(q, k, v, beta, S0p=None):
    """DeltaNet, [family] "DeltaNet: escrever o erro de previsão em vez do
    valor": e_t = beta_t (v_t - S'_{t-1} k_t); S'_t = S'_{t-1} + e_t k_t^T;
    read o_t = S'_t q_t. Layout d_v x d_k."""
    T, dk = k.shape
    dv = v.shape[1]
    S = np.zeros((dv, dk)) if S0p is None else S0p.copy()
    o = np.zeros((T, dv))
    for t in range(T):
        e = beta[t] * (v[t] - S @ k[t])
        S = S + np.outer(e, k[t])
        o[t] = S @ q[t]
    return o, S


def deltanet_expanded(q, k, v, beta, S0p=None):
    """DeltaNet expanded, [family] "Transição de estado estruturada":
    S'_t = S'_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T. Layout d_v x d_k."""
    T, dk = k.shape
    dv = v.shape[1]
    S = np.zeros((dv, dk)) if S0p is None else S0p.copy()
    o = np.zeros((T, dv))
    eye = np.eye(dk)
    for t in range(T):
        S = S @ (eye - beta[t] * np.outer(k[t], k[t])) + beta[t] * np.outer(v[t], k[t])
        o[t] = S @ q[t]
    return o, S


def gdn_four_step(q, k, v, beta, alpha, S0p=None):
    """Gated DeltaNet, [family] "Gated DeltaNet: esquecer primeiro o estado
    inteiro", steps 1-4 in order: forget S~ = alpha S'; predict v^ = S~ k;
    correct e = beta (v - v^); write S' = S~ + e k^T. The read is the
    linear-attention read o = S' q ([lesson] "Conceito"). Layout d_v x d_k;
    alpha is one scalar per token."""
    T, dk = k.shape
    dv = v.shape[1]
    S = np.zeros((dv, dk)) if S0p is None else S0p.copy()
    o = np.zeros((T, dv))
    for t in range(T):
        St = alpha[t] * S
        vhat = St @ k[t]
        e = beta[t] * (v[t] - vhat)
        S = St + np.outer(e, k[t])
        o[t] = S @ q[t]
    return o, S


def kda_five_step(q, k, v, beta, alpha, scale, S0p=None):
    """Kimi Delta Attention, [family] "Kimi Delta Attention: atenuação por
    canal", steps 1-5: S~ = S' D_t (D_t = Diag(alpha_t) acts on the key
    channels, the columns of S'); v^ = S~ k; e = beta (v - v^);
    S' = S~ + e k^T; o = S' (scale q). Layout d_v x d_k; alpha [T, d_k]."""
    T, dk = k.shape
    dv = v.shape[1]
    S = np.zeros((dv, dk)) if S0p is None else S0p.copy()
    o = np.zeros((T, dv))
    for t in range(T):
        St = S @ np.diag(alpha[t])
        vhat = St @ k[t]
        e = beta[t] * (v[t] - vhat)
        S = St + np.outer(e, k[t])
        o[t] = S @ (scale * q[t])
    return o, S


def kda_dplr(q, k, v, beta, alpha, scale, S0p=None):
    """KDA as a diagonal-plus-low-rank transition, [family] subsection
    "Transição diagonal-mais-baixo-posto": S'_t = S'_{t-1} A_t + beta_t v_t k_t^T
    with A_t = D_t - b_t a_t^T, b_t = D_t k_t, a_t = beta_t k_t (a d_k x d_k
    matrix built explicitly). Layout d_v x d_k; read S' (scale q)."""
    T, dk = k.shape
    dv = v.shape[1]
    S = np.zeros((dv, dk)) if S0p is None else S0p.copy()
    o = np.zeros((T, dv))
    for t in range(T):
        D = np.diag(alpha[t])
        bt = D @ k[t]
        at = beta[t] * k[t]
        A = D - np.outer(bt, at)
        S = S @ A + beta[t] * np.outer(v[t], k[t])
        o[t] = S @ (scale * q[t])
    return o, S


def gdn2_matrix(q, k, v, alpha, bgate, wgate, scale=1.0, S0=None):
    """Gated DeltaNet-2, [gdn2] "Regra Delta Portão-2", the update equation as
    printed, with the d_k x d_k matrix formed explicitly:
        S_t = (I - k_t (b_t . k_t)^T) D_t S_{t-1} + k_t (w_t . v_t)^T,
    D_t = Diag(alpha_t). Layout d_k x d_v; read o_t = scale * S_t^T q_t.
    alpha [T, d_k]; bgate [T, d_k]; wgate [T, d_v]."""
    T, dk = k.shape
    dv = v.shape[1]
    S = np.zeros((dk, dv)) if S0 is None else S0.copy()
    o = np.zeros((T, dv))
    eye = np.eye(dk)
    for t in range(T):
        erase = eye - np.outer(k[t], bgate[t] * k[t])
        S = erase @ np.diag(alpha[t]) @ S + np.outer(k[t], wgate[t] * v[t])
        o[t] = scale * (S.T @ q[t])
    return o, S
