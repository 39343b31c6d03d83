"""Normalised linear attention on the CPU, fp64.

TEST INFRASTRUCTURE (see the package docstring): only tests/, the smoke run
and the benchmark's CPU baseline use it; the GPU library never imports it.

Page "Linear attention e fast weights", section "Conceito". Replacing the
softmax similarity by a feature map phi, the weight of position i in the
output for token t is proportional to phi(q_t)^T phi(k_i). The two sums over
positions then no longer depend on the query, so they are kept incrementally
as a matrix state and a normaliser, and the output is a single read:

    S_t = S_{t-1} + phi(k_t) v_t^T          (d_k x d_v)
    z_t = z_{t-1} + phi(k_t)                (d_k)
    o_t = S_t^T phi(q_t) / (z_t^T phi(q_t))

The page prints the read and states the two sums in words (its display
equations for S and z are missing from the text). Readings taken:
  - the sums run over positions i <= t, the token's own key and value
    included (the causal read after the write, as in the rest of the path);
  - phi is not fixed by the page, so it is applied by the caller: the q and
    k given here are already phi(q) and phi(k) (for the weights to be a
    mixture, phi must be non-negative and z_t^T phi(q_t) > 0; a zero
    normaliser is rejected here);
  - the state S is kept d_k x d_v and read as S^T phi(q), as in the rest of
    the path; V head h reads QK head h / (H_v / H_qk).

Inputs are the stored arrays (bfloat16 bit patterns as numpy.uint16, or
float32), widened exactly to fp64.
"""
from __future__ import annotations

import numpy as np


def _f64(a):
    from oracle import upcast
    return None if a is None else upcast(a)


def recurrent(phq, phk, v, S0=None, z0=None):
    """The token-by-token recurrence above. phq, phk [B, T, H_qk, D], v
    [B, T, H_v, D_v]; S0 [B, H_v, D, D_v] and z0 [B, H_v, D] (zeros when None).
    Returns (o [B, T, H_v, D], S_T, z_T), all fp64."""
    phq, phk, v = _f64(phq), _f64(phk), _f64(v)
    B, T, Hqk, D = phq.shape
    Hv, Dv = v.shape[2], v.shape[3]
    grp = Hv // Hqk
    S = np.zeros((B, Hv, D, Dv)) if S0 is None else _f64(S0).copy()
    z = np.zeros((B, Hv, D)) if z0 is None else _f64(z0).copy()
    o = np.zeros((B, T, Hv, Dv))
    for b in range(B):
        for h in range(Hv):
            hq = h // grp
            for t in range(T):
                kt, qt = phk[b, t, hq], phq[b, t, hq]
                S[b, h] += np.outer(kt, v[b, t, h])          # write phi(k) v^T
                z[b, h] += kt                                 # normaliser
                den = z[b, h] @ qt
                if den == 0.0:
                    raise ValueError("zero normaliser z^T phi(q)")
                o[b, t, h] = (S[b, h].T @ qt) / den           # read after the write
    return o, S, z


def weighted_average(phq, phk, v):
    """The page's definition of the output for one head, brute force O(T^2):
    o_t is the average of v_i (i <= t) weighted by phi(q_t)^T phi(k_i).
    phq, phk [T, D], v [T, D_v] fp64."""
    T = phq.shape[0]
    o = np.zeros((T, v.shape[1]))
    for t in range(T):
        w = np.array([phq[t] @ phk[i] for i in range(t + 1)])
        o[t] = (w[:, None] * v[: t + 1]).sum(axis=0) / w.sum()
    return o
