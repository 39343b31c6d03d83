"""GPU parity of the backward pass (gdr_recurrent_bwd, through the C ABI)
against the fp64 backward oracle (oracle/backward.py, itself pinned by finite
differences and torch autograd): every gradient tensor in every gate and
decay mode, value dimension and io dtype; token counts inside one block of 4
tokens, on block boundaries and with a ragged tail; grouped heads; S0 and dL/dS_T
given or absent; the Qwen-shaped layer at full size on one sampled QK group;
and properties (T = 0, determinism).

Tolerance: both sides start from the same stored inputs and the GPU works in
fp32 throughout (nothing is rounded to bf16 inside), so the bound is fp32
rounding accumulated over the reverse recurrence: max |X - X_ref| / max
|X_ref| per tensor <= 1e-4 up to a few hundred tokens, 1e-3 at T = 4096.
"""
import numpy as np
import pytest

import gdr_synth as gs
from oracle import backward as obw
from parity_util import rel_err, say, small_workload, to_dev

torch = pytest.importorskip("torch")
pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

MODES = [("none", "beta"), ("scalar", "beta"), ("channel", "beta"), ("channel", "bw"), ("scalar", "bw")]


def _run(wl, seed=0, dST=True, heads=None, S0_dev=True):
    import gated_delta_rule_23_amd as gdr
    inp = gs.make_inputs(wl, seed)
    gr = gs.make_output_grads(wl, seed, dST=dST)
    d = {n: to_dev(inp[n]) for n in ("q", "k", "v", "g", "beta", "b", "w", "S0")}
    say(f"backward {wl.name} seed={seed} dST={dST}")
    out = gdr.gdr_recurrent_bwd(d["q"], d["k"], d["v"], to_dev(gr["do"]), g=d["g"], beta=d["beta"], b=d["b"],
                                w=d["w"], S0=d["S0"], dST=to_dev(gr["dST"]), scale=wl.scale)
    torch.cuda.synchronize()
    got = {k: v.cpu().numpy().astype(np.float64) for k, v in out.items()}
    ref = obw.recurrent_bwd(inp["q"], inp["k"], inp["v"], g=inp["g"], beta=inp["beta"], b=inp["b"], w=inp["w"],
                            S0=inp["S0"], do=gr["do"], dST=gr["dST"], scale=wl.scale, heads=heads)
    return got, ref


def _check(got, ref, tol, heads=None, qk_heads=None):
    assert set(got) == {k for k, v in ref.items() if v is not None}, (set(got), set(ref))
    for name, r in ref.items():
        if r is None:
            continue
        x = got[name]
        if heads is not None:
            if name in ("dq", "dk"):
                x, r = x[:, :, qk_heads], r[:, :, qk_heads]
            elif name == "dS0":
                x, r = x[:, heads], r[:, heads]
            else:
                x, r = x[:, :, heads], r[:, :, heads]
        err = rel_err(x, r)
        say(f"  {name}: {err:.2e}")
        assert err < tol, f"{name}: {err:.3e}"


@pytest.mark.parametrize("io", ["bf16", "f32"])
@pytest.mark.parametrize("D", [32, 64, 128])
@pytest.mark.parametrize("decay,gates", MODES)
@pytest.mark.parametrize("T", [1, 3, 8, 21])
def test_backward_small(io, D, decay, gates, T):
    wl = small_workload(io, D, decay, gates, T=T, B=2, Hqk=1, Hv=2, S0=True, scale=0.7)
    got, ref = _run(wl, seed=T)
    _check(got, ref, 1e-4)


@pytest.mark.parametrize("decay,gates", [("scalar", "beta"), ("channel", "bw")])
def test_backward_without_S0_and_dST(decay, gates):
    wl = small_workload("bf16", 64, decay, gates, T=19, B=1, Hqk=2, Hv=4, S0=False)
    got, ref = _run(wl, seed=3, dST=False)
    _check(got, ref, 1e-4)


@pytest.mark.parametrize("decay,gates", MODES[1:])
def test_backward_grouped_heads(decay, gates):
    """Three V heads per QK head: dq and dk sum the three heads' parts."""
    wl = small_workload("bf16", 128, decay, gates, T=45, B=2, Hqk=2, Hv=6, S0=True, scale=0.5)
    got, ref = _run(wl, seed=5)
    _check(got, ref, 1e-4)


@pytest.mark.parametrize("decay,gates", [("channel", "beta"), ("scalar", "bw")])
def test_backward_ungrouped_heads(decay, gates):
    """As many QK heads as V heads (the KDA and GDN-2 layouts)."""
    wl = small_workload("bf16", 64, decay, gates, T=37, B=2, Hqk=3, Hv=3, S0=True, scale=0.5)
    got, ref = _run(wl, seed=15)
    _check(got, ref, 1e-4)


def test_backward_qwen_shape_medium():
    wl = gs.QWEN_GDN_PREFILL.scaled(T=300, Hqk=2, Hv=6, name="qwen_like_T300")
    got, ref = _run(wl, seed=7)
    _check(got, ref, 1e-4)


def test_backward_qwen_full_size_sampled_group():
    """The Qwen-shaped layer (T = 4096, 16 QK heads, 48 V heads, d = 128,
    bf16) on the GPU; the oracle forms the gradients of QK head 5's group (V
    heads 15-17), which dq and dk of QK head 5 need in full."""
    wl = gs.QWEN_GDN_PREFILL
    heads = [15, 16, 17]
    got, ref = _run(wl, seed=11, heads=heads)
    _check(got, ref, 1e-3, heads=heads, qk_heads=[5])


def test_backward_zero_tokens_passes_dST_through():
    import gated_delta_rule_23_amd as gdr
    wl = small_workload("bf16", 64, "scalar", "beta", T=0, B=2, Hqk=1, Hv=2, S0=True)
    inp = gs.make_inputs(wl, 0)
    gr = gs.make_output_grads(wl, 0)
    d = {n: to_dev(inp[n]) for n in ("q", "k", "v", "g", "beta", "S0")}
    out = gdr.gdr_recurrent_bwd(d["q"], d["k"], d["v"], to_dev(gr["do"]), g=d["g"], beta=d["beta"], S0=d["S0"],
                                dST=to_dev(gr["dST"]))
    torch.cuda.synchronize()
    assert np.array_equal(out["dS0"].cpu().numpy(), gr["dST"])


def test_backward_is_deterministic():
    import gated_delta_rule_23_amd as gdr
    wl = small_workload("bf16", 128, "channel", "bw", T=77, B=1, Hqk=2, Hv=4, S0=True)
    inp = gs.make_inputs(wl, 1)
    gr = gs.make_output_grads(wl, 1)
    d = {n: to_dev(inp[n]) for n in ("q", "k", "v", "g", "b", "w", "S0")}
    runs = [gdr.gdr_recurrent_bwd(d["q"], d["k"], d["v"], to_dev(gr["do"]), g=d["g"], b=d["b"], w=d["w"],
                                  S0=d["S0"], dST=to_dev(gr["dST"])) for _ in range(2)]
    torch.cuda.synchronize()
    for name in runs[0]:
        assert torch.equal(runs[0][name], runs[1][name]), name


def test_backward_graph_replay_matches_eager():
    """The backward captured into a HIP graph (its three kernels, no memory
    set) and replayed three times, with eager work between the replays,
    gives the eager call's gradients bit for bit each time."""
    import gated_delta_rule_23_amd as gdr
    wl = small_workload("bf16", 64, "scalar", "beta", T=37, B=2, Hqk=1, Hv=3, S0=True)
    inp = gs.make_inputs(wl, 4)
    gr = gs.make_output_grads(wl, 4)
    d = {n: to_dev(inp[n]) for n in ("q", "k", "v", "g", "beta", "S0")}
    do, dST = to_dev(gr["do"]), to_dev(gr["dST"])
    ref = gdr.gdr_recurrent_bwd(d["q"], d["k"], d["v"], do, g=d["g"], beta=d["beta"], S0=d["S0"], dST=dST)
    torch.cuda.synchronize()
    ref = {k: v.clone() for k, v in ref.items()}
    desc = gdr.make_desc(2, 37, 1, 3, 64, gdr.GDR_BF16, gdr.GDR_DECAY_SCALAR, 1.0)
    ws = torch.empty(gdr.gdr_recurrent_bwd_workspace_bytes(desc), dtype=torch.uint8, device="cuda")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        out = gdr.gdr_recurrent_bwd(d["q"], d["k"], d["v"], do, g=d["g"], beta=d["beta"], S0=d["S0"], dST=dST,
                                    workspace=ws)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        gout = gdr.gdr_recurrent_bwd(d["q"], d["k"], d["v"], do, g=d["g"], beta=d["beta"], S0=d["S0"], dST=dST,
                                     workspace=ws)
    for rep in range(3):
        for t in gout.values():
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for name in ref:
            assert torch.equal(gout[name], ref[name]), (rep, name)
        _ = torch.ones(1 << 20, device="cuda").sum()  # eager work between replays
        torch.cuda.synchronize()
    del graph
