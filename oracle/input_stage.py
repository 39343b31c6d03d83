"""The mixer's input stage on the CPU in fp64: the step just before the
recurrence, turning raw projections into q, k, v and gates.

TEST INFRASTRUCTURE, like the rest of ``oracle/``: only ``tests/``,
``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline`` leg may use
it, and it shares no code with the GPU library.

What the pages fix, by page title and section:
  "Gated DeltaNet: o mixer em 48 das 64 camadas", section "Conceito": the
    projected sequences pass through a short causal depthwise convolution
    with kernel 4 before the recurrence.
  "Uma análise das variantes de atenção linear da família DeltaNet",
    section "Notação e ordem da derivação": the keys are normalised.
  "BigSaaS – Posts" (the Gated DeltaNet-2 post), its code listing: the erase
    and write gates are sigmoids of projections of the input.
  The decay alpha lies in (0, 1); it is stored as g = log alpha <= 0, here
  g = -c softplus(x) with a positive constant c per V head (the workloads
  draw it this way with c = 0.1 or 0.05).

Readings where the pages are silent (the plainest ones):
  * The convolution acts on every q, k and v channel with its own 4 taps.
    Tap 3 multiplies the current token and tap 0 the token three back.
    Tokens before the first come from a convolution state that holds the
    3 preceding raw tokens (zeros if there is none). No activation follows.
  * q and k are both L2-normalised per (token, head) over d_k after the
    convolution, as x / sqrt(sum x^2 + 1e-12); v is not normalised.
  * beta, b and w are sigmoids of their inputs.

Channel order of the convolution (taps and state): the H_qk * d_k channels
of q, then those of k, then the H_v * d_v channels of v, each head-major.
"""
from __future__ import annotations

import numpy as np

from . import upcast

NORM_EPS = 1e-12


def causal_conv4(x, taps, state=None):
    """Depthwise causal convolution of kernel 4 along the token axis.

    x: [B, T, Ch]; taps: [Ch, 4]; state: [B, 3, Ch] raw tokens before t = 0,
    or None for zeros. Returns (y [B, T, Ch], the state after the last token
    [B, 3, Ch], i.e. the last 3 raw tokens including the incoming state)."""
    x = upcast(x)
    taps = upcast(taps)
    B, T, Ch = x.shape
    prev = np.zeros((B, 3, Ch)) if state is None else upcast(state)
    xx = np.concatenate([prev, x], axis=1)  # token t sits at row t + 3
    y = np.zeros((B, T, Ch))
    for j in range(4):
        y += taps[:, j] * xx[:, j:j + T, :]
    return y, xx[:, T:T + 3, :].copy()


def l2norm(x):
    x = np.asarray(x, dtype=np.float64)
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + NORM_EPS)


def sigmoid(x):
    x = np.asarray(x, dtype=np.float64)
    out = np.empty_like(x)
    pos = x >= 0
    out[pos] = 1.0 / (1.0 + np.exp(-x[pos]))
    ex = np.exp(x[~pos])
    out[~pos] = ex / (1.0 + ex)
    return out


def softplus(x):
    x = np.asarray(x, dtype=np.float64)
    return np.maximum(x, 0.0) + np.log1p(np.exp(-np.abs(x)))


def conv_channels(Hqk, Hv, dk, dv):
    return 2 * Hqk * dk + Hv * dv


def input_stage(xq, xk, xv, conv_w, *, conv_in=None, g=None, beta=None, b=None, w=None, decay_scale=None):
    """Raw projections to the recurrence's inputs.

    xq, xk: [B, T, H_qk, d_k]; xv: [B, T, H_v, d_v] (stored values).
    conv_w: [2 H_qk d_k + H_v d_v, 4]; conv_in: [B, 3, same] or None.
    g: [B, T, H_v] or [B, T, H_v, d_k] pre-softplus inputs (None: no decay);
    beta: [B, T, H_v] or b [B, T, H_v, d_k] and w [B, T, H_v, d_v], sigmoid
    inputs. decay_scale: [H_v] positive c (None: 1).

    Returns (dict q, k, v, g, beta, b, w of fp64 arrays for ``recurrent``,
    conv_out [B, 3, channels])."""
    xq, xk, xv = upcast(xq), upcast(xk), upcast(xv)
    B, T, Hqk, dk = xq.shape
    Hv, dv = xv.shape[2], xv.shape[3]
    x = np.concatenate([xq.reshape(B, T, Hqk * dk), xk.reshape(B, T, Hqk * dk), xv.reshape(B, T, Hv * dv)], axis=2)
    y, conv_out = causal_conv4(x, conv_w, conv_in)
    nq = Hqk * dk
    out = {
        "q": l2norm(y[:, :, :nq].reshape(B, T, Hqk, dk)),
        "k": l2norm(y[:, :, nq:2 * nq].reshape(B, T, Hqk, dk)),
        "v": y[:, :, 2 * nq:].reshape(B, T, Hv, dv),
        "beta": None if beta is None else sigmoid(upcast(beta)),
        "b": None if b is None else sigmoid(upcast(b)),
        "w": None if w is None else sigmoid(upcast(w)),
        "g": None,
    }
    if g is not None:
        g = upcast(g)
        c = np.ones(Hv) if decay_scale is None else upcast(decay_scale)
        c = c.reshape((1, 1, Hv) + (1,) * (g.ndim - 3))
        out["g"] = -c * softplus(g)
    return out, conv_out
