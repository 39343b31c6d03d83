"""Helpers for the GPU parity tests: move seeded inputs to the GPU, run the
HIP path through the C ABI's Python binding, run the CPU oracle on the same
stored values, and compare.

Comparison (per output tensor, o and S_T separately): max |X - X_ref| divided
by max |X_ref|, against 2e-2 for bfloat16 io with the fp32 state and 1e-4 on
the all-float32 path.
"""
from __future__ import annotations

import sys

import numpy as np

import gdr_synth as gs
import oracle

TOL = {"bf16": 2e-2, "f32": 1e-4}


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def to_dev(a, dev="cuda:0"):
    import torch
    if a is None:
        return None
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def from_dev(t):
    import torch
    if t.dtype == torch.bfloat16:
        return oracle.upcast(t.view(torch.int16).cpu().numpy().view(np.uint16))
    return t.detach().cpu().numpy().astype(np.float64)


def rms_rel_err(x, ref):
    """Root-mean-square error over the root-mean-square of the reference:
    unlike the max-normalised error it is not dominated by the largest
    entries, so an error spread over small outputs shows."""
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert x.shape == ref.shape, (x.shape, ref.shape)
    if not np.all(np.isfinite(x)):
        return float("inf")
    den = np.sqrt(np.mean(ref * ref)) if ref.size else 0.0
    return float(np.sqrt(np.mean((x - ref) ** 2)) / (den if den > 0 else 1.0)) if ref.size else 0.0


def out_err(x, ref):
    """The bound the outputs o meet: both the max-normalised and the
    RMS-relative error."""
    return max(rel_err(x, ref), rms_rel_err(x, ref))


def record(name, **pairs):
    """Print the achieved errors of a parity case (max-normalised and
    RMS-relative per tensor) on one line tagged PARITY."""
    parts = []
    for key, (x, ref) in pairs.items():
        parts.append(f"{key}_max={rel_err(x, ref):.2e} {key}_rms={rms_rel_err(x, ref):.2e}")
    say(f"PARITY {name} " + " ".join(parts))


def rel_err(x, ref):
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert x.shape == ref.shape, (x.shape, ref.shape)
    assert np.all(np.isfinite(ref)), "reference has non-finite entries"
    if not np.all(np.isfinite(x)):
        return float("inf")
    den = np.max(np.abs(ref))
    return float(np.max(np.abs(x - ref)) / (den if den > 0 else 1.0))


def gpu_prefill(inp, S0=None, ST=None, scale=None, T_slice=None):
    """Run gdr_chunk_fwd on the stored inputs; returns torch (o, ST)."""
    import gated_delta_rule_23_amd as gdr
    wl = inp["workload"]
    sl = (lambda a: a) if T_slice is None else (lambda a: None if a is None else np.ascontiguousarray(a[:, T_slice]))
    d = {n: to_dev(sl(inp[n])) for n in ("q", "k", "v", "g", "beta", "b", "w")}
    return gdr.gdr_chunk_fwd(d["q"], d["k"], d["v"], g=d["g"], beta=d["beta"], b=d["b"], w=d["w"],
                             S0=S0, ST=ST, scale=wl.scale if scale is None else scale)


def gpu_recurrent(inp, S0=None, ST=None, scale=None, T_slice=None):
    """Run gdr_recurrent_fwd on the stored [B, T, ...] inputs; returns torch (o, ST)."""
    import gated_delta_rule_23_amd as gdr
    wl = inp["workload"]
    sl = (lambda a: a) if T_slice is None else (lambda a: None if a is None else np.ascontiguousarray(a[:, T_slice]))
    d = {n: to_dev(sl(inp[n])) for n in ("q", "k", "v", "g", "beta", "b", "w")}
    return gdr.gdr_recurrent_fwd(d["q"], d["k"], d["v"], g=d["g"], beta=d["beta"], b=d["b"], w=d["w"],
                                 S0=S0, ST=ST, scale=wl.scale if scale is None else scale)


def gpu_recurrent_in(raw, S0=None, ST=None, conv_in="stored", conv_out=None, T_slice=None):
    """Run gdr_recurrent_fwd_in on raw inputs from gdr_synth.make_raw_inputs;
    returns torch (o, ST, conv_out). conv_in="stored" uses the drawn state."""
    import gated_delta_rule_23_amd as gdr
    wl = raw["workload"]
    sl = (lambda a: a) if T_slice is None else (lambda a: None if a is None else np.ascontiguousarray(a[:, T_slice]))
    d = {n: to_dev(sl(raw[n])) for n in ("q", "k", "v", "g", "beta", "b", "w")}
    cin = to_dev(raw["conv_in"]) if isinstance(conv_in, str) else conv_in
    return gdr.gdr_recurrent_fwd_in(d["q"], d["k"], d["v"], to_dev(raw["conv_w"]), conv_in=cin, conv_out=conv_out,
                                    decay_scale=to_dev(raw["decay_scale"]), g=d["g"], beta=d["beta"], b=d["b"],
                                    w=d["w"], S0=S0, ST=ST, scale=wl.scale)


def gpu_prefill_in(raw, S0=None, ST=None, conv_in="stored", conv_out=None, T_slice=None):
    """Run gdr_chunk_fwd_in on raw inputs; returns torch (o, ST, conv_out)."""
    import gated_delta_rule_23_amd as gdr
    wl = raw["workload"]
    sl = (lambda a: a) if T_slice is None else (lambda a: None if a is None else np.ascontiguousarray(a[:, T_slice]))
    d = {n: to_dev(sl(raw[n])) for n in ("q", "k", "v", "g", "beta", "b", "w")}
    cin = to_dev(raw["conv_in"]) if isinstance(conv_in, str) else conv_in
    return gdr.gdr_chunk_fwd_in(d["q"], d["k"], d["v"], to_dev(raw["conv_w"]), conv_in=cin, conv_out=conv_out,
                                decay_scale=to_dev(raw["decay_scale"]), g=d["g"], beta=d["beta"], b=d["b"],
                                w=d["w"], S0=S0, ST=ST, scale=wl.scale)


def oracle_input_stage(raw, heads=None, cols=None, S0="stored", conv_in="stored"):
    """The input-stage oracle, then the recurrence oracle. Returns (o, S_T,
    conv_out) in fp64."""
    from oracle import input_stage as ist
    wl = raw["workload"]
    cin = raw["conv_in"] if isinstance(conv_in, str) else conv_in
    st, conv_out = ist.input_stage(raw["q"], raw["k"], raw["v"], raw["conv_w"], conv_in=cin, g=raw["g"],
                                   beta=raw["beta"], b=raw["b"], w=raw["w"], decay_scale=raw["decay_scale"])
    o, S = oracle.recurrent(st["q"], st["k"], st["v"], g=st["g"], beta=st["beta"], b=st["b"], w=st["w"],
                            scale=wl.scale, S0=raw["S0"] if isinstance(S0, str) else S0, heads=heads, cols=cols)
    return o, S, conv_out


def oracle_prefill(inp, heads=None, cols=None, S0=None):
    wl = inp["workload"]
    return oracle.recurrent(inp["q"], inp["k"], inp["v"], g=inp["g"], beta=inp["beta"], b=inp["b"], w=inp["w"],
                            scale=wl.scale, S0=S0 if S0 is not None else inp["S0"], heads=heads, cols=cols)


def gpu_decode(inp, steps=None):
    """Run the step-major decode inputs through gdr_decode_step; returns
    (o [steps,B,Hv,D] fp64, final S fp64)."""
    import torch
    import gated_delta_rule_23_amd as gdr
    wl = inp["workload"]
    n = wl.T if steps is None else steps
    dev = {k: to_dev(inp[k]) for k in ("q", "k", "v", "g", "beta", "b", "w")}
    if inp["S0"] is not None:
        S = to_dev(inp["S0"]).clone()
    else:
        S = torch.zeros((wl.B, wl.Hv, wl.dk, wl.dv), dtype=torch.float32, device="cuda:0")
    outs = []
    for s in range(n):
        pick = lambda t: None if t is None else t[s]
        outs.append(gdr.gdr_decode_step(pick(dev["q"]), pick(dev["k"]), pick(dev["v"]), S, g=pick(dev["g"]),
                                        beta=pick(dev["beta"]), b=pick(dev["b"]), w=pick(dev["w"]),
                                        scale=wl.scale))
    torch.cuda.synchronize()
    return np.stack([from_dev(o) for o in outs]), from_dev(S)


def small_workload(io, D, decay, gates, T, B=2, Hqk=1, Hv=2, S0=False, decode=False, scale=1.0):
    g_recipe = {"none": "none", "scalar": "softplus_0.1", "channel": "softplus_0.05"}[decay]
    return gs.Workload(f"small_{io}_D{D}_{decay}_{gates}_T{T}", B, T, Hqk, Hv, D, D, io, decay, gates, g_recipe,
                       S0="normal_0.02" if S0 else "zero", scale=scale, decode=decode)


def strong_channel_decay(g, T, D):
    """Per-channel log decays the chunked prefill must survive: -1.5 held on
    some channels over whole chunks (in-chunk sums near -96, beyond where
    exp(-G) overflows float32), a gradual -2.6 per token over one 16-token
    block (a block sum just past 40), and spikes of -30 and -200 (alpha
    underflows to zero) on single tokens and channels."""
    g = g.copy()
    g[:, 64:min(T, 192), :, : D // 8] = -1.5
    if T > 146:
        g[:, 130:146, 0, D // 4: D // 4 + 2] = -2.6
    g[:, min(20, T - 1), :, 3] = -30.0
    g[:, min(37, T - 1), -1, 5:9] = -200.0
    g[:, min(100, T - 1), 0, :] = -45.0
    return g


def sweep_segments(B, Hv, D, T, io="bf16"):
    """The library's split of a long sweep (256 compute units, at least 16
    chunks per segment, at most 8 segments; half again as many with bf16 io
    at d = 128, whose split sweep runs 64-column work items and whose segment
    pass runs three work items per CU), restated to check that a test takes
    the segmented path."""
    NC = -(-T // 64)
    items = B * Hv * (D // 32)
    p = min(256 // items, NC // 16, 8)
    if p < 2:
        return 1
    if io == "bf16" and D == 128:
        p = min(1 + 384 // items, NC // 16, 8)
    L = -(-NC // p)
    return -(-NC // L)
