"""GPU parity: the HIP path through the C ABI against the fp64 CPU oracle.

Small shapes span several chunks and a ragged tail in every gate mode, value
dimension and io dtype; the five full-size workloads are compared on sampled
(head, value-column) outputs the oracle computes one by one (value columns and
heads evolve independently). Plus properties that hold at any size.
"""
import numpy as np
import pytest

import gdr_synth as gs
from parity_util import sweep_segments as _sweep_segments
from parity_util import (TOL, from_dev, gpu_decode, gpu_prefill, gpu_prefill_in, gpu_recurrent, gpu_recurrent_in,
                         oracle_input_stage, oracle_prefill, out_err, record, rel_err, say, small_workload,
                         strong_channel_decay, to_dev)

torch = pytest.importorskip("torch")
pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

MODES = [("none", "beta"), ("scalar", "beta"), ("channel", "beta"), ("channel", "bw"), ("scalar", "bw")]
PREFILL_DIMS = [("bf16", 32), ("bf16", 64), ("bf16", 128), ("f32", 32), ("f32", 64)]


# ---------------------------------------------------------------------------
# Decode.

@pytest.mark.parametrize("io", ["bf16", "f32"])
@pytest.mark.parametrize("D", [32, 64, 128])
@pytest.mark.parametrize("decay,gates", MODES[:4])
def test_decode_small(io, D, decay, gates):
    wl = small_workload(io, D, decay, gates, T=6, B=3, Hqk=2, Hv=4, S0=True, decode=True,
                        scale=D ** -0.5 if decay == "channel" else 1.0)
    inp = gs.make_inputs(wl, seed=D + len(decay))
    say(f"decode {wl.name}")
    o_gpu, S_gpu = gpu_decode(inp)
    o_ref, S_ref = oracle_prefill(gs.as_sequence(inp))
    assert out_err(o_gpu, np.swapaxes(o_ref, 0, 1)) < TOL[io]
    assert rel_err(S_gpu, S_ref) < TOL[io]


def test_decode_qwen_shape_256_steps():
    """64 sequences x 48 V heads (16 QK heads), 128 x 128 fp32 states, 256
    consecutive steps; every step's outputs and the final states of sampled
    heads against the oracle."""
    wl = gs.QWEN_GDN_DECODE
    inp = gs.make_inputs(wl, seed=2)
    say(f"decode {wl.name}")
    o_gpu, S_gpu = gpu_decode(inp)
    heads = [0, 1, 2, 25, 47]
    o_ref, S_ref = oracle_prefill(gs.as_sequence(inp), heads=heads)
    record(wl.name, o=(o_gpu[:, :, heads], np.swapaxes(o_ref, 0, 1)[:, :, heads]), S=(S_gpu[:, heads], S_ref[:, heads]))
    assert out_err(o_gpu[:, :, heads], np.swapaxes(o_ref, 0, 1)[:, :, heads]) < TOL["bf16"]
    assert rel_err(S_gpu[:, heads], S_ref[:, heads]) < TOL["bf16"]
    assert np.all(np.isfinite(S_gpu))


# ---------------------------------------------------------------------------
# Prefill, small shapes.

@pytest.mark.parametrize("io,D", PREFILL_DIMS)
@pytest.mark.parametrize("decay,gates", MODES)
@pytest.mark.parametrize("T", [1, 64, 150])
def test_prefill_small(io, D, decay, gates, T):
    wl = small_workload(io, D, decay, gates, T=T, B=2, Hqk=1, Hv=2, S0=(T != 64))
    inp = gs.make_inputs(wl, seed=T + D)
    say(f"prefill {wl.name}")
    S0 = to_dev(inp["S0"])
    o, ST = gpu_prefill(inp, S0=S0)
    o_ref, S_ref = oracle_prefill(inp)
    assert out_err(from_dev(o), o_ref) < TOL[io]
    assert rel_err(from_dev(ST), S_ref) < TOL[io]


@pytest.mark.parametrize("io,D", [("bf16", 128), ("f32", 64)])
def test_prefill_grouped_heads_and_scale(io, D):
    """Two QK heads serving three V heads each, read scale d^-1/2, strong
    per-channel decay, many chunks."""
    wl = small_workload(io, D, "channel", "beta", T=333, B=2, Hqk=2, Hv=6, S0=True, scale=D ** -0.5)
    wl = wl.scaled(g_recipe="logsigmoid_n21")
    inp = gs.make_inputs(wl, seed=7)
    say(f"prefill {wl.name}")
    o, ST = gpu_prefill(inp, S0=to_dev(inp["S0"]))
    o_ref, S_ref = oracle_prefill(inp)
    assert out_err(from_dev(o), o_ref) < TOL[io]
    assert rel_err(from_dev(ST), S_ref) < TOL[io]


@pytest.mark.parametrize("io,D,gates,T", [
    ("bf16", 128, "beta", 150), ("bf16", 128, "bw", 200), ("bf16", 64, "beta", 150), ("bf16", 32, "bw", 150),
    ("f32", 64, "bw", 150), ("f32", 32, "beta", 70),
])
def test_prefill_strong_channel_decay(io, D, gates, T):
    """Per-channel decays far stronger than the workloads': the chunked form
    must give the token recurrence, with no overflow inside a chunk."""
    wl = small_workload(io, D, "channel", gates, T=T, B=2, Hqk=1, Hv=2, S0=True, scale=D ** -0.5)
    inp = gs.make_inputs(wl, seed=61 + D)
    inp = dict(inp, g=strong_channel_decay(inp["g"], T, D))
    say(f"prefill strong channel decay {wl.name}")
    o, ST = gpu_prefill(inp, S0=to_dev(inp["S0"]))
    o_ref, S_ref = oracle_prefill(inp)
    assert out_err(from_dev(o), o_ref) < TOL[io]
    assert rel_err(from_dev(ST), S_ref) < TOL[io]


def test_prefill_strong_channel_decay_segmented():
    """The same decays on a long sequence with one head, so the sweep is
    split into segments (transition matrices carry the strong decays)."""
    wl = small_workload("bf16", 128, "channel", "bw", T=2200, B=1, Hqk=1, Hv=1, S0=True)
    assert _sweep_segments(1, 1, 128, 2200) > 1
    inp = gs.make_inputs(wl, seed=66)
    g = strong_channel_decay(inp["g"], 2200, 128)
    g[:, 1000:1400, :, 40:44] = -1.5
    g[:, 1601, :, 90] = -200.0
    inp = dict(inp, g=g)
    say(f"prefill strong channel decay segmented {wl.name}")
    o, ST = gpu_prefill(inp, S0=to_dev(inp["S0"]))
    o_ref, S_ref = oracle_prefill(inp)
    assert out_err(from_dev(o), o_ref) < TOL["bf16"]
    assert rel_err(from_dev(ST), S_ref) < TOL["bf16"]


@pytest.mark.parametrize("io,D,gates", [("bf16", 128, "beta"), ("bf16", 128, "bw"), ("f32", 64, "bw")])
def test_prefill_input_stage_strong_channel_decay(io, D, gates):
    """From raw projections: decay inputs x with g = -c softplus(x) for c = 1,
    so x = 1.5, 30 and 200 give the strong decays above."""
    pytest.skip("held off the GPU: the first case faulted the GPU in an earlier build whose per-chunk kernel "
                "fused the whole input stage (convolution included) with per-channel decay; no cause was found "
                "in that kernel, which has since been removed (the convolution now runs as a pass of its own and "
                "the gate and decay activations in the prefill's load stage, covered on the same kind of decays "
                "by test_prefill_in_stage_pass_strong_channel_decay)")
    T = 150
    wl = small_workload(io, D, "channel", gates, T=T, B=2, Hqk=1, Hv=2, S0=True, scale=D ** -0.5)
    wl = wl.scaled(g_recipe="logsigmoid_n21")  # decay constant c = 1
    raw = gs.make_raw_inputs(wl, seed=71 + D)
    x = raw["g"].copy()
    x[:, 64:128, :, : D // 8] = 1.5
    x[:, 20, :, 3] = 30.0
    x[:, 37, -1, 5:9] = 200.0
    x[:, 130:146, 0, D // 4: D // 4 + 2] = 2.6
    raw = dict(raw, g=x)
    say(f"prefill input stage strong channel decay {wl.name}")
    o, ST, cout = gpu_prefill_in(raw, S0=to_dev(raw["S0"]))
    o_ref, S_ref, c_ref = oracle_input_stage(raw)
    assert out_err(from_dev(o), o_ref) < TOL[io]
    assert rel_err(from_dev(ST), S_ref) < TOL[io]
    assert _conv_equal(cout, c_ref)


@pytest.mark.parametrize("io,D,gates", [("bf16", 128, "bw"), ("bf16", 64, "beta"), ("f32", 32, "bw")])
def test_prefill_in_stage_pass_strong_channel_decay(io, D, gates):
    """gdr_chunk_fwd_in with a per-channel decay runs the convolution and
    normalisation as a pass of their own, then the prefill, which applies the
    gate and decay activations as it loads them. Decay inputs x with g = -softplus(x)
    (decay constant 1) give -1.5 held over two chunks on some channels, a
    block of -2.6, and spikes near -30, -45 and -200."""
    T = 200
    wl = small_workload(io, D, "channel", gates, T=T, B=2, Hqk=1, Hv=2, S0=True, scale=D ** -0.5)
    wl = wl.scaled(g_recipe="logsigmoid_n21")  # decay constant c = 1
    raw = gs.make_raw_inputs(wl, seed=97 + D)
    x = raw["g"].copy()
    x[:, 64:192, :, : D // 8] = 1.25       # softplus(1.25) = 1.52
    x[:, 130:146, 0, D // 4: D // 4 + 2] = 2.5
    x[:, 20, :, 3] = 30.0
    x[:, 100, 0, :] = 45.0
    x[:, 37, -1, 5:9] = 200.0
    raw = dict(raw, g=x)
    say(f"prefill stage pass strong channel decay {wl.name}")
    o, ST, cout = gpu_prefill_in(raw, S0=to_dev(raw["S0"]))
    o_ref, S_ref, c_ref = oracle_input_stage(raw)
    assert out_err(from_dev(o), o_ref) < TOL[io]
    assert rel_err(from_dev(ST), S_ref) < TOL[io]
    assert _conv_equal(cout, c_ref)


# ---------------------------------------------------------------------------
# Prefill, the workloads at full size.

def test_prefill_gdn_small_f32_full():
    wl = gs.GDN_SMALL_F32
    inp = gs.make_inputs(wl, seed=0)
    say(f"prefill {wl.name}")
    o, ST = gpu_prefill(inp)
    o_ref, S_ref = oracle_prefill(inp)
    record(wl.name, o=(from_dev(o), o_ref), S=(from_dev(ST), S_ref))
    assert out_err(from_dev(o), o_ref) < TOL["f32"]
    assert rel_err(from_dev(ST), S_ref) < TOL["f32"]


@pytest.mark.parametrize("wl,heads,cols", [
    (gs.QWEN_GDN_PREFILL, [0, 1, 2, 3, 24, 47], None),
    (gs.KDA_PREFILL, [0, 17, 31], (0, 48)),
    (gs.GDN2_PREFILL, [0, 9, 15], (80, 128)),
], ids=lambda x: getattr(x, "name", None))
def test_prefill_full_size_sampled(wl, heads, cols):
    inp = gs.make_inputs(wl, seed=1)
    say(f"prefill {wl.name}")
    o, ST = gpu_prefill(inp)
    torch.cuda.synchronize()
    o_ref, S_ref = oracle_prefill(inp, heads=heads, cols=cols)
    c0, c1 = cols if cols else (0, wl.dv)
    o_g = from_dev(o[:, :, heads, c0:c1])
    S_g = from_dev(ST[:, heads, :, c0:c1])
    record(wl.name, o=(o_g, o_ref[:, :, heads, c0:c1]), S=(S_g, S_ref[:, heads, :, c0:c1]))
    assert out_err(o_g, o_ref[:, :, heads, c0:c1]) < TOL["bf16"]
    assert rel_err(S_g, S_ref[:, heads, :, c0:c1]) < TOL["bf16"]
    assert bool(torch.isfinite(o.float()).all()) and bool(torch.isfinite(ST).all())


@pytest.mark.parametrize("io,D,decay,gates,T,Hv,B", [
    ("bf16", 64, "scalar", "beta", 2500, 2, 1),
    ("bf16", 128, "scalar", "bw", 4096, 2, 1),
    ("bf16", 128, "channel", "bw", 4113, 1, 1),
    ("f32", 32, "channel", "beta", 2100, 1, 1),
    ("bf16", 64, "channel", "beta", 2100, 1, 2),
    ("bf16", 128, "channel", "bw", 5200, 16, 1),      # five segments, the last one shorter
])
def test_prefill_segmented_sweep(io, D, decay, gates, T, Hv, B):
    """Long sequences with few heads split the sequential sweep into segments
    that run in parallel from entry states found by a scan over the segments'
    transitions; the result is still the token-by-token recurrence, here from
    a non-zero initial state and with a partial last chunk in one case."""
    assert _sweep_segments(B, Hv, D, T, io) > 1
    wl = small_workload(io, D, decay, gates, T, B=B, Hqk=1, Hv=Hv, S0=True)
    inp = gs.make_inputs(wl, seed=7)
    say(f"segmented {wl.name}")
    o, ST = gpu_prefill(inp, S0=to_dev(inp["S0"]))
    o_ref, S_ref = oracle_prefill(inp)
    assert out_err(from_dev(o), o_ref) < TOL[io]
    assert rel_err(from_dev(ST), S_ref) < TOL[io]


def test_prefill_segmented_sweep_in_place():
    """With the sweep split, the first segment starts from a copy of S0 that
    the segment scan keeps, so S_T may alias S0: the in-place call gives the
    out-of-place result bit for bit."""
    wl = small_workload("bf16", 128, "scalar", "beta", 3000, B=1, Hqk=1, Hv=2, S0=True)
    assert _sweep_segments(1, 2, 128, 3000) > 1
    inp = gs.make_inputs(wl, seed=9)
    S0 = to_dev(inp["S0"])
    o1, S1 = gpu_prefill(inp, S0=S0)
    S = S0.clone()
    o2, S2 = gpu_prefill(inp, S0=S, ST=S)
    assert torch.equal(o1, o2) and torch.equal(S, S1)
    o_ref, S_ref = oracle_prefill(inp)
    assert out_err(from_dev(o2), o_ref) < TOL["bf16"] and rel_err(from_dev(S), S_ref) < TOL["bf16"]


# ---------------------------------------------------------------------------
# Properties.

def test_prefill_split_resume_matches_one_pass():
    wl = small_workload("bf16", 128, "channel", "bw", T=300, B=1, Hqk=2, Hv=4, S0=True)
    inp = gs.make_inputs(wl, seed=11)
    S0 = to_dev(inp["S0"])
    o_all, S_all = gpu_prefill(inp, S0=S0)
    o1, S1 = gpu_prefill(inp, S0=S0, T_slice=slice(0, 100))
    o2, S2 = gpu_prefill(inp, S0=S1, T_slice=slice(100, 300))
    assert rel_err(from_dev(torch.cat([o1, o2], dim=1)), from_dev(o_all)) < TOL["bf16"]
    assert rel_err(from_dev(S2), from_dev(S_all)) < TOL["bf16"]


def test_prefill_equals_decode_steps():
    wl = small_workload("f32", 64, "channel", "beta", T=70, B=2, Hqk=1, Hv=2, S0=True)
    inp = gs.make_inputs(wl, seed=12)
    o_p, S_p = gpu_prefill(inp, S0=to_dev(inp["S0"]))
    step_major = {n: (None if inp[n] is None else np.ascontiguousarray(np.swapaxes(inp[n], 0, 1)))
                  for n in ("q", "k", "v", "g", "beta", "b", "w")}
    dec = dict(inp, **step_major)
    dec["workload"] = wl.scaled(decode=True)
    o_d, S_d = gpu_decode(dec)
    assert rel_err(np.swapaxes(o_d, 0, 1), from_dev(o_p)) < TOL["f32"]
    assert rel_err(S_d, from_dev(S_p)) < TOL["f32"]


def test_prefill_in_place_state_and_determinism():
    wl = small_workload("bf16", 64, "scalar", "beta", T=200, B=2, Hqk=1, Hv=2, S0=True)
    inp = gs.make_inputs(wl, seed=13)
    S0 = to_dev(inp["S0"])
    o1, S1 = gpu_prefill(inp, S0=S0)
    o2, S2 = gpu_prefill(inp, S0=S0)
    assert torch.equal(o1, o2) and torch.equal(S1, S2)          # run to run, bit for bit
    S_inplace = S0.clone()
    o3, S3 = gpu_prefill(inp, S0=S_inplace, ST=S_inplace)       # ST aliases S0
    assert S3.data_ptr() == S_inplace.data_ptr()
    assert torch.equal(o3, o1) and torch.equal(S_inplace, S1)


def test_hip_graph_replay_matches_eager():
    """Prefill and decode calls captured in a HIP graph, as a serving loop
    would run them, give the eager result bit for bit on every replay, with
    eager work and synchronisations between the replays. The library enqueues
    only kernels (no memset or allocation) once its workspace is given."""
    import gated_delta_rule_23_amd as gdr
    cur = torch.cuda.current_stream
    for wl in (small_workload("bf16", 128, "scalar", "beta", T=300, B=1, Hqk=1, Hv=3, S0=True),
               small_workload("bf16", 64, "channel", "bw", T=2100, B=1, Hqk=1, Hv=1, S0=True),
               small_workload("bf16", 128, "channel", "bw", T=2100, B=1, Hqk=1, Hv=1, S0=True)):
        inp = gs.make_inputs(wl, seed=21)
        say(f"graph {wl.name}")
        d = {n: to_dev(inp[n]) for n in ("q", "k", "v", "g", "beta", "b", "w")}
        S0 = to_dev(inp["S0"])
        desc = gdr.make_desc(wl.B, wl.T, wl.Hqk, wl.Hv, wl.dk, gdr.GDR_BF16,
                             gdr.GDR_DECAY_SCALAR if wl.decay == "scalar" else gdr.GDR_DECAY_CHANNEL)
        ws = torch.empty(gdr.gdr_chunk_workspace_bytes(desc), dtype=torch.uint8, device="cuda:0")
        o = torch.empty((wl.B, wl.T, wl.Hv, wl.dv), dtype=torch.bfloat16, device="cuda:0")
        ST = torch.empty((wl.B, wl.Hv, wl.dk, wl.dv), dtype=torch.float32, device="cuda:0")

        def call():
            gdr.gdr_chunk_fwd(d["q"], d["k"], d["v"], g=d["g"], beta=d["beta"], b=d["b"], w=d["w"], S0=S0, o=o,
                              ST=ST, workspace=ws, stream=cur())

        call()
        torch.cuda.synchronize()
        o_ref, S_ref = o.clone(), ST.clone()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            call()
        for _ in range(3):
            o.zero_()
            ST.zero_()
            torch.cuda.synchronize()
            graph.replay()
            torch.cuda.synchronize()
            assert torch.equal(o, o_ref) and torch.equal(ST, S_ref)

    wl = gs.QWEN_GDN_DECODE.scaled(B=4, Hqk=2, Hv=6, T=8)
    inp = gs.make_inputs(wl, seed=22)
    dd = {n: to_dev(inp[n]) for n in ("q", "k", "v", "g", "beta", "b", "w")}
    S_init = to_dev(inp["S0"])
    S = S_init.clone()
    outs = [torch.empty((wl.B, wl.Hv, wl.dv), dtype=torch.bfloat16, device="cuda:0") for _ in range(wl.T)]

    def steps():
        for s in range(wl.T):
            gdr.gdr_decode_step(dd["q"][s], dd["k"][s], dd["v"][s], S, g=dd["g"][s], beta=dd["beta"][s],
                                scale=wl.scale, o=outs[s], stream=cur())

    steps()
    torch.cuda.synchronize()
    o_ref, S_ref = [x.clone() for x in outs], S.clone()
    S.copy_(S_init)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        steps()
    for _ in range(3):
        S.copy_(S_init)
        for x in outs:
            x.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(S, S_ref) and all(torch.equal(x, r) for x, r in zip(outs, o_ref))


def test_prefill_empty_sequence_copies_state():
    import gated_delta_rule_23_amd as gdr
    wl = small_workload("bf16", 64, "scalar", "beta", T=8, B=2, Hqk=1, Hv=2, S0=True)
    inp = gs.make_inputs(wl, seed=14)
    S0 = to_dev(inp["S0"])
    o, ST = gpu_prefill(inp, S0=S0, T_slice=slice(0, 0))
    torch.cuda.synchronize()
    assert o.shape[1] == 0 and torch.equal(ST, S0)
    o, ST = gpu_prefill(inp, S0=None, T_slice=slice(0, 0))
    torch.cuda.synchronize()
    assert torch.count_nonzero(ST) == 0
    assert gdr.gdr_last_error() == ""


# ---------------------------------------------------------------------------
# Multi-token recurrent forward (short runs from a live state).

def _recurrent_wide(B, Hv, D):
    """True when the library runs 32 value columns per wave (many heads);
    with fewer heads it runs 16 (d >= 64). Restated so that a test can check
    which variant it exercises."""
    return D == 32 or B * Hv * (D // 32) >= 4096


@pytest.mark.parametrize("io", ["bf16", "f32"])
@pytest.mark.parametrize("D", [32, 64, 128])
@pytest.mark.parametrize("decay,gates", MODES)
@pytest.mark.parametrize("T", [1, 9, 20])
def test_recurrent_small(io, D, decay, gates, T):
    wl = small_workload(io, D, decay, gates, T=T, B=2, Hqk=1, Hv=2, S0=True)
    inp = gs.make_inputs(wl, seed=3 * T + D)
    say(f"recurrent {wl.name}")
    o, ST = gpu_recurrent(inp, S0=to_dev(inp["S0"]))
    o_ref, S_ref = oracle_prefill(inp)
    assert out_err(from_dev(o), o_ref) < TOL[io]
    assert rel_err(from_dev(ST), S_ref) < TOL[io]


@pytest.mark.parametrize("io,D,decay,gates,T", [
    ("bf16", 128, "scalar", "beta", 4),
    ("bf16", 128, "channel", "bw", 11),
    ("f32", 64, "channel", "beta", 3),
    ("bf16", 64, "scalar", "bw", 8),
])
def test_recurrent_many_heads(io, D, decay, gates, T):
    """Serving shapes (64 sequences, 48 or 64 V heads, 16 QK heads): the
    variant with 32 value columns per wave; a few new tokens per sequence from
    a non-zero state, sampled heads against the oracle."""
    Hv = 48 if D == 128 else 64
    assert _recurrent_wide(64, Hv, D)
    wl = small_workload(io, D, decay, gates, T=T, B=64, Hqk=16, Hv=Hv, S0=True, scale=D ** -0.5)
    inp = gs.make_inputs(wl, seed=31)
    say(f"recurrent {wl.name}")
    o, ST = gpu_recurrent(inp, S0=to_dev(inp["S0"]))
    heads = [0, 5, Hv // 2, Hv - 1]
    o_ref, S_ref = oracle_prefill(inp, heads=heads)
    assert out_err(from_dev(o[:, :, heads]), o_ref[:, :, heads]) < TOL[io]
    assert rel_err(from_dev(ST[:, heads]), S_ref[:, heads]) < TOL[io]
    assert bool(torch.isfinite(o.float()).all()) and bool(torch.isfinite(ST).all())


@pytest.mark.parametrize("io,D", [("bf16", 128), ("f32", 64), ("f32", 128)])
def test_recurrent_grouped_heads_strong_decay(io, D):
    wl = small_workload(io, D, "channel", "beta", T=37, B=2, Hqk=2, Hv=6, S0=True, scale=D ** -0.5)
    wl = wl.scaled(g_recipe="logsigmoid_n21")
    inp = gs.make_inputs(wl, seed=8)
    say(f"recurrent {wl.name}")
    o, ST = gpu_recurrent(inp, S0=to_dev(inp["S0"]))
    o_ref, S_ref = oracle_prefill(inp)
    assert out_err(from_dev(o), o_ref) < TOL[io]
    assert rel_err(from_dev(ST), S_ref) < TOL[io]


def test_recurrent_equals_decode_steps_and_chunked():
    """The three schedules compute one recurrence: a T-token recurrent call
    equals T decode steps (float32, same per-token arithmetic up to reduction
    order) and the chunked prefill (bfloat16 io, within its tolerance)."""
    wl = small_workload("f32", 64, "channel", "bw", T=12, B=2, Hqk=1, Hv=2, S0=True)
    inp = gs.make_inputs(wl, seed=15)
    o_r, S_r = gpu_recurrent(inp, S0=to_dev(inp["S0"]))
    step_major = {n: (None if inp[n] is None else np.ascontiguousarray(np.swapaxes(inp[n], 0, 1)))
                  for n in ("q", "k", "v", "g", "beta", "b", "w")}
    dec = dict(inp, **step_major)
    dec["workload"] = wl.scaled(decode=True)
    o_d, S_d = gpu_decode(dec)
    assert out_err(from_dev(o_r), np.swapaxes(o_d, 0, 1)) < 1e-5
    assert rel_err(from_dev(S_r), S_d) < 1e-5

    wl = small_workload("bf16", 128, "scalar", "beta", T=100, B=1, Hqk=1, Hv=3, S0=True)
    inp = gs.make_inputs(wl, seed=16)
    S0 = to_dev(inp["S0"])
    o_r, S_r = gpu_recurrent(inp, S0=S0)
    o_c, S_c = gpu_prefill(inp, S0=S0)
    assert out_err(from_dev(o_r), from_dev(o_c)) < TOL["bf16"]
    assert rel_err(from_dev(S_r), from_dev(S_c)) < TOL["bf16"]


def test_recurrent_split_resume_in_place_and_determinism():
    """Verify-k style use: the state advances in place over consecutive short
    calls and ends where one call over all the tokens ends, bit for bit (the
    same per-token arithmetic in the same order); repeated calls agree bit for
    bit."""
    wl = small_workload("bf16", 128, "channel", "bw", T=21, B=3, Hqk=1, Hv=4, S0=True)
    inp = gs.make_inputs(wl, seed=17)
    S0 = to_dev(inp["S0"])
    o_all, S_all = gpu_recurrent(inp, S0=S0)
    o_again, S_again = gpu_recurrent(inp, S0=S0)
    assert torch.equal(o_all, o_again) and torch.equal(S_all, S_again)
    S = S0.clone()
    outs = []
    for a, b in ((0, 5), (5, 6), (6, 14), (14, 21)):
        o, S_ret = gpu_recurrent(inp, S0=S, ST=S, T_slice=slice(a, b))
        assert S_ret.data_ptr() == S.data_ptr()
        outs.append(o)
    assert torch.equal(torch.cat(outs, dim=1), o_all) and torch.equal(S, S_all)


@pytest.mark.parametrize("io,decay,D", [("f32", "channel", 64), ("bf16", "channel", 128), ("f32", "scalar", 32),
                                         ("bf16", "scalar", 128)])
def test_recurrent_extreme_decay(io, decay, D):
    """Very negative log decays: whole key channels (or heads) forgetting
    within a few tokens, including alpha that underflows to zero in fp32
    (g = -200), against the oracle."""
    wl = small_workload(io, D, decay, "beta", T=21, B=2, Hqk=1, Hv=2, S0=True)
    inp = gs.make_inputs(wl, seed=19)
    g = inp["g"].copy()
    if decay == "channel":
        g[:, 3, :, : D // 4] = -30.0
        g[:, 4, :, : D // 8] = -15.0
        g[:, 10, 1, 5] = -200.0            # alpha = 0 in fp32
        g[:, 17, 0, :] = -45.0             # every channel of one head at once
    else:
        g[:, 2, :] = -45.0
        g[:, 9, 1] = -200.0
        g[:, 12, 0] = -25.0
        g[:, 13, 0] = -25.0
    inp = dict(inp, g=g)
    say(f"recurrent extreme decay {wl.name}")
    o, ST = gpu_recurrent(inp, S0=to_dev(inp["S0"]))
    o_ref, S_ref = oracle_prefill(inp)
    assert out_err(from_dev(o), o_ref) < TOL[io]
    assert rel_err(from_dev(ST), S_ref) < TOL[io]


def test_recurrent_zero_tokens_copies_state():
    import gated_delta_rule_23_amd as gdr
    wl = small_workload("bf16", 64, "scalar", "beta", T=8, B=2, Hqk=1, Hv=2, S0=True)
    inp = gs.make_inputs(wl, seed=18)
    S0 = to_dev(inp["S0"])
    o, ST = gpu_recurrent(inp, S0=S0, T_slice=slice(0, 0))
    torch.cuda.synchronize()
    assert o.shape[1] == 0 and torch.equal(ST, S0)
    ST.fill_(1.0)
    o, ST = gpu_recurrent(inp, S0=None, ST=ST, T_slice=slice(0, 0))
    torch.cuda.synchronize()
    assert torch.count_nonzero(ST) == 0
    assert gdr.gdr_last_error() == ""


def test_recurrent_graph_replay_matches_eager():
    import gated_delta_rule_23_amd as gdr
    wl = small_workload("bf16", 128, "channel", "beta", T=4, B=8, Hqk=2, Hv=6, S0=True)
    inp = gs.make_inputs(wl, seed=23)
    d = {n: to_dev(inp[n]) for n in ("q", "k", "v", "g", "beta", "b", "w")}
    S_init = to_dev(inp["S0"])
    S = S_init.clone()
    o = torch.empty((wl.B, wl.T, wl.Hv, wl.dv), dtype=torch.bfloat16, device="cuda:0")

    def call():
        gdr.gdr_recurrent_fwd(d["q"], d["k"], d["v"], g=d["g"], beta=d["beta"], S0=S, ST=S, o=o,
                              stream=torch.cuda.current_stream())

    call()
    torch.cuda.synchronize()
    o_ref, S_ref = o.clone(), S.clone()
    S.copy_(S_init)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call()
    for _ in range(3):
        S.copy_(S_init)
        o.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref) and torch.equal(S, S_ref)


# ---------------------------------------------------------------------------
# Input stage fused into the recurrent forward (raw projections in).

def _conv_equal(c_gpu, c_ref):
    """The convolution state is a copy of stored raw values: exact."""
    return np.array_equal(from_dev(c_gpu), np.asarray(c_ref, dtype=np.float64))


@pytest.mark.parametrize("io", ["bf16", "f32"])
@pytest.mark.parametrize("D", [32, 64, 128])
@pytest.mark.parametrize("decay,gates", MODES)
@pytest.mark.parametrize("T", [1, 2, 9])
def test_recurrent_input_stage_small(io, D, decay, gates, T):
    """T = 1 and 2 take part of the convolution window from the incoming
    convolution state; T = 9 spans two staged blocks."""
    wl = small_workload(io, D, decay, gates, T=T, B=2, Hqk=1, Hv=2, S0=True, scale=D ** -0.5)
    raw = gs.make_raw_inputs(wl, seed=5 * T + D)
    say(f"input stage {wl.name}")
    o, ST, cout = gpu_recurrent_in(raw, S0=to_dev(raw["S0"]))
    o_ref, S_ref, c_ref = oracle_input_stage(raw)
    assert out_err(from_dev(o), o_ref) < TOL[io]
    assert rel_err(from_dev(ST), S_ref) < TOL[io]
    assert _conv_equal(cout, c_ref)


@pytest.mark.parametrize("io,D,decay,gates", [("bf16", 128, "scalar", "beta"), ("bf16", 64, "channel", "bw")])
def test_recurrent_input_stage_without_conv_state(io, D, decay, gates):
    wl = small_workload(io, D, decay, gates, T=5, B=3, Hqk=2, Hv=4, S0=False)
    raw = gs.make_raw_inputs(wl, seed=41, conv_state=False)
    o, ST, cout = gpu_recurrent_in(raw, conv_in=None)
    o_ref, S_ref, c_ref = oracle_input_stage(raw, conv_in=None)
    assert out_err(from_dev(o), o_ref) < TOL[io]
    assert rel_err(from_dev(ST), S_ref) < TOL[io]
    assert _conv_equal(cout, c_ref)


def test_recurrent_input_stage_serving_shape():
    """64 sequences, 16 QK heads, 48 V heads, d = 128, 4 raw tokens per call
    from a live state and convolution state (the variant with 32 value
    columns per wave); sampled heads against the oracle, the whole
    convolution state exactly."""
    wl = gs.QWEN_GDN_DECODE.scaled(T=4, decode=False)
    raw = gs.make_raw_inputs(wl, seed=43)
    say(f"input stage {wl.name}")
    o, ST, cout = gpu_recurrent_in(raw, S0=to_dev(raw["S0"]))
    heads = [0, 1, 2, 30, 47]
    o_ref, S_ref, c_ref = oracle_input_stage(raw, heads=heads)
    assert out_err(from_dev(o[:, :, heads]), o_ref[:, :, heads]) < TOL["bf16"]
    assert rel_err(from_dev(ST[:, heads]), S_ref[:, heads]) < TOL["bf16"]
    assert _conv_equal(cout, c_ref)


def test_recurrent_input_stage_decode_steps_equal_one_call():
    """Decode as T = 1 calls with the convolution state alternating between
    two buffers and the state updated in place gives, bit for bit, what one
    call over all the tokens gives (same per-token arithmetic)."""
    wl = small_workload("bf16", 128, "channel", "bw", T=7, B=2, Hqk=2, Hv=4, S0=True)
    raw = gs.make_raw_inputs(wl, seed=44)
    S0 = to_dev(raw["S0"])
    o_all, S_all, c_all = gpu_recurrent_in(raw, S0=S0)
    S = S0.clone()
    bufs = [to_dev(raw["conv_in"]).clone(), torch.empty_like(c_all)]
    outs = []
    for t in range(wl.T):
        o, _, _ = gpu_recurrent_in(raw, S0=S, ST=S, conv_in=bufs[t % 2], conv_out=bufs[(t + 1) % 2],
                                   T_slice=slice(t, t + 1))
        outs.append(o)
    assert torch.equal(torch.cat(outs, dim=1), o_all) and torch.equal(S, S_all)
    assert torch.equal(bufs[wl.T % 2], c_all)


def test_recurrent_input_stage_zero_tokens():
    wl = small_workload("bf16", 64, "scalar", "beta", T=4, B=2, Hqk=1, Hv=2, S0=True)
    raw = gs.make_raw_inputs(wl, seed=45)
    S0 = to_dev(raw["S0"])
    o, ST, cout = gpu_recurrent_in(raw, S0=S0, T_slice=slice(0, 0))
    torch.cuda.synchronize()
    assert torch.equal(ST, S0) and torch.equal(cout, to_dev(raw["conv_in"]))


# ---------------------------------------------------------------------------
# Float32 io at d = 128: tied gates with a scalar decay or none.

@pytest.mark.parametrize("decay", ["none", "scalar"])
@pytest.mark.parametrize("T,B,Hqk,Hv", [(1, 2, 1, 2), (64, 2, 1, 2), (150, 2, 1, 2), (333, 2, 2, 6),
                                        (2100, 1, 1, 1)])
def test_prefill_f32_d128(decay, T, B, Hqk, Hv):
    """Several chunks and a ragged tail, grouped heads (three V heads per QK
    head), and one head over 33 chunks, which the sweep splits into segments."""
    wl = small_workload("f32", 128, decay, "beta", T=T, B=B, Hqk=Hqk, Hv=Hv, S0=True, scale=128 ** -0.5)
    inp = gs.make_inputs(wl, seed=T + 128)
    say(f"prefill {wl.name}")
    o, ST = gpu_prefill(inp, S0=to_dev(inp["S0"]))
    o_ref, S_ref = oracle_prefill(inp)
    record(wl.name, o=(from_dev(o), o_ref), S=(from_dev(ST), S_ref))
    assert out_err(from_dev(o), o_ref) < TOL["f32"]
    assert rel_err(from_dev(ST), S_ref) < TOL["f32"]


def test_prefill_f32_d128_strong_decay_in_place():
    """Decays down to -30 per token (whole chunks decay below float32's
    range), the state updated in place."""
    wl = small_workload("f32", 128, "scalar", "beta", T=200, B=1, Hqk=1, Hv=3, S0=True)
    inp = gs.make_inputs(wl, seed=5)
    rng = np.random.default_rng(5)
    inp["g"] = np.where(rng.random(inp["g"].shape) < 0.1, -30.0, inp["g"]).astype(np.float32)
    say(f"prefill {wl.name} strong decay")
    S = to_dev(inp["S0"])
    o, ST = gpu_prefill(inp, S0=S, ST=S)
    o_ref, S_ref = oracle_prefill(inp)
    assert ST.data_ptr() == S.data_ptr()
    assert out_err(from_dev(o), o_ref) < TOL["f32"]
    assert rel_err(from_dev(S), S_ref) < TOL["f32"]


# ---------------------------------------------------------------------------
# Input stage fused into the chunked prefill's load stage.

@pytest.mark.parametrize("io,D", PREFILL_DIMS)
@pytest.mark.parametrize("decay,gates", MODES)
@pytest.mark.parametrize("T", [1, 2, 64, 150])
def test_prefill_input_stage_small(io, D, decay, gates, T):
    """T = 1 and 2: the whole window and part of the outgoing state come from
    the incoming convolution state; T = 150: chunks 2 and 3 take their first
    window from the chunk before."""
    wl = small_workload(io, D, decay, gates, T=T, B=2, Hqk=1, Hv=2, S0=True, scale=D ** -0.5)
    raw = gs.make_raw_inputs(wl, seed=7 * T + D)
    say(f"prefill input stage {wl.name}")
    o, ST, cout = gpu_prefill_in(raw, S0=to_dev(raw["S0"]))
    o_ref, S_ref, c_ref = oracle_input_stage(raw)
    assert out_err(from_dev(o), o_ref) < TOL[io]
    assert rel_err(from_dev(ST), S_ref) < TOL[io]
    assert _conv_equal(cout, c_ref)


@pytest.mark.parametrize("io,D,decay,gates,T,Hqk,Hv,B", [
    ("bf16", 128, "scalar", "beta", 333, 2, 6, 2),      # grouped heads, no incoming convolution state
    ("bf16", 64, "channel", "bw", 2500, 1, 2, 1),       # segmented sweep
    ("f32", 64, "scalar", "bw", 200, 1, 3, 2),
])
def test_prefill_input_stage_larger(io, D, decay, gates, T, Hqk, Hv, B):
    wl = small_workload(io, D, decay, gates, T=T, B=B, Hqk=Hqk, Hv=Hv, S0=True)
    raw = gs.make_raw_inputs(wl, seed=47, conv_state=(T != 333))
    say(f"prefill input stage {wl.name}")
    o, ST, cout = gpu_prefill_in(raw, S0=to_dev(raw["S0"]), conv_in="stored" if T != 333 else None)
    o_ref, S_ref, c_ref = oracle_input_stage(raw, conv_in="stored" if T != 333 else None)
    assert out_err(from_dev(o), o_ref) < TOL[io]
    assert rel_err(from_dev(ST), S_ref) < TOL[io]
    assert _conv_equal(cout, c_ref)


def test_prefill_input_stage_qwen_full_size_sampled():
    """The Qwen-shaped layer (T = 4096, 16 QK heads, 48 V heads, d = 128)
    from raw projections, as the benchmark times it: sampled heads against
    the oracle, the whole outgoing convolution state exactly."""
    wl = gs.QWEN_GDN_PREFILL
    raw = gs.make_raw_inputs(wl, seed=48)
    say(f"prefill input stage {wl.name}")
    o, ST, cout = gpu_prefill_in(raw)
    torch.cuda.synchronize()
    heads = [0, 2, 25, 47]
    o_ref, S_ref, c_ref = oracle_input_stage(raw, heads=heads, S0=None)
    assert out_err(from_dev(o[:, :, heads]), o_ref[:, :, heads]) < TOL["bf16"]
    assert rel_err(from_dev(ST[:, heads]), S_ref[:, heads]) < TOL["bf16"]
    assert _conv_equal(cout, c_ref)


def test_prefill_input_stage_wide_groups_sampled():
    """Four V heads per QK head and enough chunks that the load stage runs
    several V heads of a QK head back to back in one workgroup (the later
    ones reusing the first one's convolved and normalised q and k): sampled
    heads at every position in a group against the oracle."""
    wl = small_workload("bf16", 128, "scalar", "beta", T=4096, B=4, Hqk=2, Hv=8, S0=True, scale=128 ** -0.5)
    raw = gs.make_raw_inputs(wl, seed=51)
    say(f"prefill input stage {wl.name}")
    o, ST, cout = gpu_prefill_in(raw, S0=to_dev(raw["S0"]))
    torch.cuda.synchronize()
    heads = [0, 1, 6, 7]
    o_ref, S_ref, c_ref = oracle_input_stage(raw, heads=heads)
    assert out_err(from_dev(o[:, :, heads]), o_ref[:, :, heads]) < TOL["bf16"]
    assert rel_err(from_dev(ST[:, heads]), S_ref[:, heads]) < TOL["bf16"]
    assert _conv_equal(cout, c_ref)


def test_prefill_input_stage_split_and_serving_handoff():
    """A prefill in two calls, the second taking the first's convolution state
    and final state, equals one call; decode steps from there (T = 1 calls of
    the recurrent forward with the handed-over states) equal the tail of one
    long recurrent call."""
    wl = small_workload("bf16", 128, "scalar", "beta", T=210, B=2, Hqk=2, Hv=4, S0=True)
    raw = gs.make_raw_inputs(wl, seed=49)
    S0 = to_dev(raw["S0"])
    o_all, S_all, c_all = gpu_prefill_in(raw, S0=S0)
    o1, S1, c1 = gpu_prefill_in(raw, S0=S0, T_slice=slice(0, 130))
    o2, S2, c2 = gpu_prefill_in(raw, S0=S1, conv_in=c1, T_slice=slice(130, 200))
    o3, S3, c3 = gpu_prefill_in(raw, S0=S2, conv_in=c2, T_slice=slice(200, 210))
    assert rel_err(from_dev(torch.cat([o1, o2, o3], dim=1)), from_dev(o_all)) < TOL["bf16"]
    assert rel_err(from_dev(S3), from_dev(S_all)) < TOL["bf16"]
    assert torch.equal(c3, c_all)
    o_r, S_r, c_r = gpu_recurrent_in(raw, S0=S0)
    assert out_err(from_dev(o_r), from_dev(o_all)) < TOL["bf16"]
    assert torch.equal(c_r, c_all)
    S = S2.clone()
    bufs = [c2.clone(), torch.empty_like(c2)]
    for t in range(200, 210):
        o, _, _ = gpu_recurrent_in(raw, S0=S, ST=S, conv_in=bufs[t % 2], conv_out=bufs[(t + 1) % 2],
                                   T_slice=slice(t, t + 1))
        assert out_err(from_dev(o), from_dev(o_all[:, t:t + 1])) < TOL["bf16"]
    assert torch.equal(bufs[210 % 2], c_all)
    assert rel_err(from_dev(S), from_dev(S_all)) < TOL["bf16"]


def test_prefill_input_stage_zero_tokens():
    wl = small_workload("bf16", 64, "channel", "bw", T=4, B=2, Hqk=1, Hv=2, S0=True)
    raw = gs.make_raw_inputs(wl, seed=50)
    S0 = to_dev(raw["S0"])
    o, ST, cout = gpu_prefill_in(raw, S0=S0, T_slice=slice(0, 0))
    torch.cuda.synchronize()
    assert torch.equal(ST, S0) and torch.equal(cout, to_dev(raw["conv_in"]))
    o, ST, cout = gpu_prefill_in(raw, S0=S0, conv_in=None, T_slice=slice(0, 0))
    torch.cuda.synchronize()
    assert torch.count_nonzero(cout) == 0


# ---------------------------------------------------------------------------
# Seeded random configurations across every entry point.

def _random_config(seed):
    rng = np.random.default_rng(1000 + seed)
    io = ["bf16", "f32"][rng.integers(2)]
    D = [32, 64, 128][seed % 3]
    decay, gates = MODES[rng.integers(len(MODES))]
    B, Hqk = int(rng.integers(1, 4)), int(rng.integers(1, 3))
    Hv = Hqk * int(rng.integers(1, 4))
    T = int(rng.integers(1, 300))
    scale = [1.0, D ** -0.5][rng.integers(2)]
    return io, D, decay, gates, B, Hqk, Hv, T, bool(rng.integers(2)), scale


@pytest.mark.parametrize("seed", range(15))
def test_random_configurations(seed):
    """Dtype, head dimension, gate and decay mode, batch, head grouping,
    length, initial state and read scale drawn from a fixed seed; the
    chunked prefill (where the dtype and dimension are supported), the
    recurrent forward and both input-stage entry points against the oracle."""
    io, D, decay, gates, B, Hqk, Hv, T, has_s0, scale = _random_config(seed)
    wl = small_workload(io, D, decay, gates, T=T, B=B, Hqk=Hqk, Hv=Hv, S0=has_s0, scale=scale)
    inp = gs.make_inputs(wl, seed=seed)
    say(f"random {seed}: {wl.name} B={B} Hqk={Hqk} Hv={Hv} scale={scale:.3f}")
    S0 = to_dev(inp["S0"])
    o_ref, S_ref = oracle_prefill(inp)
    if io == "bf16" or D <= 64:
        o, ST = gpu_prefill(inp, S0=S0)
        assert out_err(from_dev(o), o_ref) < TOL[io] and rel_err(from_dev(ST), S_ref) < TOL[io]
    o, ST = gpu_recurrent(inp, S0=S0)
    assert out_err(from_dev(o), o_ref) < TOL[io] and rel_err(from_dev(ST), S_ref) < TOL[io]
    raw = gs.make_raw_inputs(wl, seed=seed, conv_state=bool(seed % 2))
    cin = "stored" if seed % 2 else None
    o_ref, S_ref, c_ref = oracle_input_stage(raw, conv_in=cin)
    S0 = to_dev(raw["S0"])
    runs = [gpu_recurrent_in(raw, S0=S0, conv_in=cin)]
    if io == "bf16" or D <= 64:
        runs.append(gpu_prefill_in(raw, S0=S0, conv_in=cin))
    for o, ST, cout in runs:
        assert out_err(from_dev(o), o_ref) < TOL[io] and rel_err(from_dev(ST), S_ref) < TOL[io]
        assert _conv_equal(cout, c_ref)


def test_state_alloc_is_zeroed():
    import gated_delta_rule_23_amd as gdr
    ptr, n = gdr.gdr_state_alloc(2, 3, 64, 64)
    try:
        assert n == 2 * 3 * 64 * 64 * 4
        # Use the library-allocated state as the decode state: with beta = 0 and
        # no decay the step is a no-op and the read returns S^T q = 0.
        class _View:
            __cuda_array_interface__ = {"shape": (2, 3, 64, 64), "typestr": "<f4", "data": (ptr, False),
                                        "version": 3, "strides": None}
        S = torch.as_tensor(_View(), device="cuda:0")
        torch.cuda.synchronize()
        assert torch.count_nonzero(S) == 0
    finally:
        gdr.gdr_state_free(ptr)
