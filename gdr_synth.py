"""Seeded synthetic inputs for the gated delta-rule mixer.

This module is the only code that both the GPU path's tests/benchmark and the
CPU oracle's callers share. It draws random tensors and rounds them to their
stored dtype; it contains none of the mixer's arithmetic.

Recipe
------
* ``numpy.random.Generator(PCG64)``; one child stream per tensor from
  ``SeedSequence(seed).spawn(8)``, in the fixed order q, k, v, beta, g, b, w,
  S0 (a stream is spawned even when its tensor is absent, so adding a tensor
  never shifts another one's numbers).
* Draws are fp64. q and k are L2-normalised over d_k per (sequence, token,
  head) in fp64. Every tensor is then rounded once, round-to-nearest-even,
  to its stored dtype: bfloat16 (held as ``numpy.uint16`` bit patterns) or
  float32. beta and g are always float32; b, w, q, k, v use the io dtype.
* Distributions follow the workload texts: v ~ N(0,1); beta = sigmoid(N(0,1));
  the decay alpha = exp(g) with g = log(sigmoid(N(2,1))) (small fp32 case),
  g = -0.1 softplus(N(0,1)) (Qwen-shaped GDN prefill and decode), or
  g = -0.05 softplus(N(0,1)) per key channel (KDA, Gated DeltaNet-2);
  b, w = sigmoid(N(0,1)); the decode state S0 = 0.02 N(0,1) (0.02 read as a
  standard deviation).
* Prefill tensors are laid out [B, T, H, d]. Decode tensors are laid out
  step-major, [steps, B, H, d], so each step's slice is contiguous;
  ``as_sequence`` reorders them to [B, steps, H, d] for a sequential run.
"""
from __future__ import annotations

import dataclasses
from dataclasses import dataclass

import numpy as np

ORDER = ("q", "k", "v", "beta", "g", "b", "w", "S0")


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    T: int               # tokens per sequence (prefill) or consecutive steps (decode)
    Hqk: int
    Hv: int
    dk: int
    dv: int
    io: str              # "bf16" | "f32"
    decay: str           # "none" | "scalar" | "channel"
    gates: str           # "beta" (tied) | "bw" (decoupled erase/write gates)
    g_recipe: str        # "logsigmoid_n21" | "softplus_0.1" | "softplus_0.05" | "none"
    S0: str = "zero"     # "zero" | "normal_0.02"
    chunk: int = 64
    scale: float = 1.0
    decode: bool = False

    def scaled(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# The five workloads: small fp32 GDN; Qwen-shaped GDN prefill; GDN decode;
# KDA prefill; Gated DeltaNet-2 long prefill.
GDN_SMALL_F32 = Workload("gdn_small_f32_T64_d32", 1, 64, 1, 1, 32, 32, "f32", "scalar", "beta",
                         "logsigmoid_n21")
QWEN_GDN_PREFILL = Workload("qwen_gdn_prefill_T4096_Hqk16_Hv48_d128", 1, 4096, 16, 48, 128, 128,
                            "bf16", "scalar", "beta", "softplus_0.1")
QWEN_GDN_DECODE = Workload("qwen_gdn_decode_B64_Hv48_d128_256steps", 64, 256, 16, 48, 128, 128,
                           "bf16", "scalar", "beta", "softplus_0.1", S0="normal_0.02", decode=True)
KDA_PREFILL = Workload("kda_prefill_B2_T16384_H32_d128", 2, 16384, 32, 32, 128, 128, "bf16",
                       "channel", "beta", "softplus_0.05")
GDN2_PREFILL = Workload("gdn2_prefill_T65536_H16_d128", 1, 65536, 16, 16, 128, 128, "bf16",
                        "channel", "bw", "softplus_0.05")
WORKLOADS = (GDN_SMALL_F32, QWEN_GDN_PREFILL, QWEN_GDN_DECODE, KDA_PREFILL, GDN2_PREFILL)


def bf16_bits(x) -> np.ndarray:
    """Round fp64 values to bfloat16, nearest-even, in one step; return the bit
    patterns as uint16. Values must lie in the normal float32 range (or be 0)."""
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float64))
    ax = np.abs(x)
    if np.any((ax != 0) & ((ax < 2.0 ** -126) | (ax >= (2.0 - 2.0 ** -8) * 2.0 ** 127))) or not np.all(np.isfinite(x)):
        raise ValueError("value outside the normal float32 range")
    bits = x.view(np.uint64)
    lsb = (bits >> np.uint64(45)) & np.uint64(1)
    bits = (bits + np.uint64((1 << 44) - 1) + lsb) & ~np.uint64((1 << 45) - 1)
    y = bits.view(np.float64).astype(np.float32)   # exact: 8 significant bits
    return (y.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def bf16_to_f32(bits) -> np.ndarray:
    return (np.asarray(bits).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _store(x, dtype):
    return bf16_bits(x) if dtype == "bf16" else np.asarray(x, dtype=np.float64).astype(np.float32)


def _sigmoid(x):
    return 1.0 / (1.0 + np.exp(-x))


def _softplus(x):
    return np.logaddexp(0.0, x)


def _l2n(x):
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True))


def make_inputs(wl: Workload, seed: int = 0) -> dict:
    """Draw every input of ``wl``. Returns a dict of stored arrays (absent
    tensors are None) plus ``"workload"`` and ``"seed"``."""
    streams = dict(zip(ORDER, (np.random.Generator(np.random.PCG64(s))
                               for s in np.random.SeedSequence(seed).spawn(len(ORDER)))))
    lead = (wl.T, wl.B) if wl.decode else (wl.B, wl.T)
    out = {"workload": wl, "seed": seed}
    out["q"] = _store(_l2n(streams["q"].standard_normal(lead + (wl.Hqk, wl.dk))), wl.io)
    out["k"] = _store(_l2n(streams["k"].standard_normal(lead + (wl.Hqk, wl.dk))), wl.io)
    out["v"] = _store(streams["v"].standard_normal(lead + (wl.Hv, wl.dv)), wl.io)
    if wl.gates == "beta":
        out["beta"] = _store(_sigmoid(streams["beta"].standard_normal(lead + (wl.Hv,))), "f32")
        out["b"] = out["w"] = None
    else:
        out["beta"] = None
        out["b"] = _store(_sigmoid(streams["b"].standard_normal(lead + (wl.Hv, wl.dk))), wl.io)
        out["w"] = _store(_sigmoid(streams["w"].standard_normal(lead + (wl.Hv, wl.dv))), wl.io)
    if wl.decay == "none":
        out["g"] = None
    else:
        gshape = lead + ((wl.Hv,) if wl.decay == "scalar" else (wl.Hv, wl.dk))
        x = streams["g"].standard_normal(gshape)
        if wl.g_recipe == "logsigmoid_n21":
            g = -_softplus(-(2.0 + x))          # log(sigmoid(x')), x' ~ N(2, 1)
        elif wl.g_recipe == "softplus_0.1":
            g = -0.1 * _softplus(x)
        elif wl.g_recipe == "softplus_0.05":
            g = -0.05 * _softplus(x)
        else:
            raise ValueError(wl.g_recipe)
        out["g"] = _store(g, "f32")
    if wl.S0 == "normal_0.02":
        out["S0"] = _store(0.02 * streams["S0"].standard_normal((wl.B, wl.Hv, wl.dk, wl.dv)), "f32")
    else:
        out["S0"] = None
    return out


def make_output_grads(wl: Workload, seed: int = 0, dST: bool = True) -> dict:
    """Draw the incoming gradients of a backward pass for ``wl`` (prefill
    layout): do = dL/do ~ N(0, 1) in the io dtype, [B, T, Hv, dv]; dST =
    dL/dS_T ~ 0.1 N(0, 1) float32, [B, Hv, dk, dv] (None when dST is False).
    Two streams of their own, seeded from ``seed``."""
    s_do, s_st = (np.random.Generator(np.random.PCG64(s)) for s in np.random.SeedSequence([seed, 7]).spawn(2))
    out = {"do": _store(s_do.standard_normal((wl.B, wl.T, wl.Hv, wl.dv)), wl.io)}
    out["dST"] = _store(0.1 * s_st.standard_normal((wl.B, wl.Hv, wl.dk, wl.dv)), "f32") if dST else None
    return out


RAW_ORDER = ORDER + ("conv_w", "conv_in")


def make_raw_inputs(wl: Workload, seed: int = 0, conv_state: bool = True) -> dict:
    """Draw the raw inputs of the input stage for ``wl`` (prefill layout
    [B, T, ...]): q, k, v ~ N(0, 1) before the convolution (not normalised);
    per-channel convolution taps ~ N(0, 0.5^2), shape [2 Hqk dk + Hv dv, 4];
    an incoming convolution state of 3 raw tokens ~ N(0, 1) (None when
    conv_state is False); gate inputs ~ N(0, 1) (sigmoid inputs for beta,
    b, w); decay inputs x with a per-V-head constant c such that
    -c softplus(x) follows the workload's decay recipe (x ~ N(0, 1) and
    c = 0.1 or 0.05, or x = -(2 + N(0, 1)) and c = 1 for log sigmoid
    N(2, 1)). Same stream scheme as make_inputs, with two more streams."""
    streams = dict(zip(RAW_ORDER, (np.random.Generator(np.random.PCG64(s))
                                   for s in np.random.SeedSequence(seed).spawn(len(RAW_ORDER)))))
    lead = (wl.B, wl.T)
    ch = 2 * wl.Hqk * wl.dk + wl.Hv * wl.dv
    out = {"workload": wl, "seed": seed}
    out["q"] = _store(streams["q"].standard_normal(lead + (wl.Hqk, wl.dk)), wl.io)
    out["k"] = _store(streams["k"].standard_normal(lead + (wl.Hqk, wl.dk)), wl.io)
    out["v"] = _store(streams["v"].standard_normal(lead + (wl.Hv, wl.dv)), wl.io)
    out["conv_w"] = _store(0.5 * streams["conv_w"].standard_normal((ch, 4)), "f32")
    out["conv_in"] = _store(streams["conv_in"].standard_normal((wl.B, 3, ch)), wl.io) if conv_state else None
    if wl.gates == "beta":
        out["beta"] = _store(streams["beta"].standard_normal(lead + (wl.Hv,)), "f32")
        out["b"] = out["w"] = None
    else:
        out["beta"] = None
        out["b"] = _store(streams["b"].standard_normal(lead + (wl.Hv, wl.dk)), wl.io)
        out["w"] = _store(streams["w"].standard_normal(lead + (wl.Hv, wl.dv)), wl.io)
    out["decay_scale"] = None
    if wl.decay == "none":
        out["g"] = None
    else:
        gshape = lead + ((wl.Hv,) if wl.decay == "scalar" else (wl.Hv, wl.dk))
        x = streams["g"].standard_normal(gshape)
        c = {"logsigmoid_n21": 1.0, "softplus_0.1": 0.1, "softplus_0.05": 0.05}[wl.g_recipe]
        if wl.g_recipe == "logsigmoid_n21":
            x = -(2.0 + x)
        out["g"] = _store(x, "f32")
        out["decay_scale"] = np.full(wl.Hv, c, dtype=np.float32)
    if wl.S0 == "normal_0.02":
        out["S0"] = _store(0.02 * streams["S0"].standard_normal((wl.B, wl.Hv, wl.dk, wl.dv)), "f32")
    else:
        out["S0"] = None
    return out


NLA_ORDER = ("phq", "phk", "v", "S0", "z0")


def make_norm_la_inputs(B, T, Hqk, Hv, D, io="bf16", seed=0, state=False) -> dict:
    """Seeded inputs of the normalised linear-attention read, prefill layout:
    phq, phk [B, T, H_qk, D] and v [B, T, H_v, D] in the io dtype, the
    feature-mapped queries and keys drawn as non-negative values
    elu(x) + 1 with x ~ N(0, 1) (a distribution choice for the inputs; the
    feature map itself is the caller's); v ~ N(0, 1). With state, an incoming
    state S0 = 0.02 N(0, 1) [B, H_v, D, D] and normaliser z0 = |N(0, 1)|
    [B, H_v, D] in float32 (z0 as the sum of earlier non-negative keys would
    be); otherwise None. One child stream per tensor in NLA_ORDER."""
    streams = dict(zip(NLA_ORDER, (np.random.Generator(np.random.PCG64(s))
                                   for s in np.random.SeedSequence([seed, 4]).spawn(len(NLA_ORDER)))))

    def feat(x):
        return np.where(x > 0, x + 1.0, np.exp(np.minimum(x, 0.0)))

    out = {"seed": seed, "io": io}
    out["phq"] = _store(feat(streams["phq"].standard_normal((B, T, Hqk, D))), io)
    out["phk"] = _store(feat(streams["phk"].standard_normal((B, T, Hqk, D))), io)
    out["v"] = _store(streams["v"].standard_normal((B, T, Hv, D)), io)
    if state:
        out["S0"] = _store(0.02 * streams["S0"].standard_normal((B, Hv, D, D)), "f32")
        out["z0"] = _store(np.abs(streams["z0"].standard_normal((B, Hv, D))), "f32")
    else:
        out["S0"] = out["z0"] = None
    return out


def as_sequence(inp: dict) -> dict:
    """Decode inputs are step-major [steps, B, ...]; return a copy with every
    per-step tensor reordered to [B, steps, ...] (a sequential run's layout)."""
    out = dict(inp)
    for name in ("q", "k", "v", "beta", "g", "b", "w"):
        if inp.get(name) is not None:
            out[name] = np.ascontiguousarray(np.swapaxes(inp[name], 0, 1))
    return out
