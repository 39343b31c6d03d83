"""GPU parity of the chunked backward pass (gdr_chunk_bwd, through the C ABI)
against the fp64 backward oracle (oracle/backward.py, pinned by finite
differences and torch autograd): every gradient tensor in every gate and
decay mode, value dimension and io dtype; token counts of one token, just
under, on and just over a chunk of 64, and several chunks with a ragged
tail; grouped heads; S0 and dL/dS_T given or absent; a strong scalar decay
(the log-sigmoid recipe, in-chunk decay sums far below the float range of
exp(-G)); the Qwen-shaped layer at full size on one sampled QK group; and
properties (T = 0, determinism, graph replay, agreement with the recurrent
form of the same gradients).

Tolerance: the inputs are the same stored values and the GPU works in fp32
throughout, so the bound is fp32 rounding through the chunk's triangular
solves and the sweeps over chunks: max |X - X_ref| / max |X_ref| per
tensor <= 1e-4 up to a few hundred tokens, 1e-3 at T = 4096.
"""
import numpy as np
import pytest

import gdr_synth as gs
from oracle import backward as obw
from parity_util import rel_err, say, small_workload, strong_channel_decay, to_dev

torch = pytest.importorskip("torch")
pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

MODES = [("none", "beta"), ("scalar", "beta"), ("channel", "beta"), ("channel", "bw"), ("scalar", "bw")]


def _dev_inputs(wl, seed, dST=True, g_fn=None):
    inp = gs.make_inputs(wl, seed)
    if g_fn is not None:
        inp = dict(inp, g=g_fn(inp["g"]))
    gr = gs.make_output_grads(wl, seed, dST=dST)
    d = {n: to_dev(inp[n]) for n in ("q", "k", "v", "g", "beta", "b", "w", "S0")}
    return inp, gr, d


def _call(fn, d, gr, wl):
    return fn(d["q"], d["k"], d["v"], to_dev(gr["do"]), g=d["g"], beta=d["beta"], b=d["b"], w=d["w"], S0=d["S0"],
              dST=to_dev(gr["dST"]), scale=wl.scale)


def _run(wl, seed=0, dST=True, heads=None, g_fn=None):
    import gated_delta_rule_23_amd as gdr
    inp, gr, d = _dev_inputs(wl, seed, dST, g_fn)
    say(f"chunk backward {wl.name} seed={seed} dST={dST}")
    out = _call(gdr.gdr_chunk_bwd, d, gr, wl)
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
        assert np.all(np.isfinite(x)), name
        err = rel_err(x, r)
        say(f"  {name}: {err:.2e}")
        assert err < tol, f"{name}: {err:.3e}"


@pytest.mark.parametrize("io", ["bf16", "f32"])
@pytest.mark.parametrize("D", [32, 64, 128])
@pytest.mark.parametrize("decay,gates", MODES)
@pytest.mark.parametrize("T", [1, 63, 64, 65, 150])
def test_chunk_backward_small(io, D, decay, gates, T):
    wl = small_workload(io, D, decay, gates, T=T, B=2, Hqk=1, Hv=2, S0=True, scale=0.7)
    got, ref = _run(wl, seed=T)
    _check(got, ref, 1e-4)


@pytest.mark.parametrize("decay,gates", [("scalar", "beta"), ("channel", "bw")])
def test_chunk_backward_without_S0_and_dST(decay, gates):
    wl = small_workload("bf16", 64, decay, gates, T=130, B=1, Hqk=2, Hv=4, S0=False)
    got, ref = _run(wl, seed=3, dST=False)
    _check(got, ref, 1e-4)


@pytest.mark.parametrize("decay,gates", MODES[1:])
def test_chunk_backward_grouped_heads(decay, gates):
    """Three V heads per QK head: dq and dk sum the three heads' parts."""
    wl = small_workload("bf16", 128, decay, gates, T=145, B=2, Hqk=2, Hv=6, S0=True, scale=0.5)
    got, ref = _run(wl, seed=5)
    _check(got, ref, 1e-4)


@pytest.mark.parametrize("decay,gates", [("channel", "beta"), ("scalar", "bw"), ("none", "beta")])
def test_chunk_backward_ungrouped_heads(decay, gates):
    """As many QK heads as V heads (the KDA and GDN-2 layouts): dq and dk are
    written directly, without the sum over grouped heads."""
    wl = small_workload("bf16", 64, decay, gates, T=130, B=2, Hqk=3, Hv=3, S0=True, scale=0.5)
    got, ref = _run(wl, seed=15)
    _check(got, ref, 1e-4)


@pytest.mark.parametrize("io,D", [("f32", 32), ("bf16", 128)])
def test_chunk_backward_strong_scalar_decay(io, D):
    """Per-token decays exp(g) with g = log sigmoid(-(2 + N(0, 1))): over a
    chunk the decay sums reach about -135, where exp(-G) overflows fp32; the
    scalar path keeps every factor as exp(G_t - G_j) <= 1."""
    wl = gs.Workload(f"strong_decay_{io}_D{D}", 2, 200, 1, 2, D, D, io, "scalar", "beta", "logsigmoid_n21",
                     S0="normal_0.02", scale=D ** -0.5)
    got, ref = _run(wl, seed=9)
    _check(got, ref, 1e-4)


@pytest.mark.parametrize("io,D,gates,T,Hv", [
    ("f32", 32, "beta", 150, 2), ("f32", 64, "bw", 200, 2), ("bf16", 128, "bw", 200, 2), ("bf16", 128, "beta", 150, 2),
    ("bf16", 64, "beta", 150, 3),
])
def test_chunk_backward_strong_channel_decay(io, D, gates, T, Hv):
    """Per-channel decays far stronger than the workloads' (-1.5 held over
    whole chunks, one block past 40, spikes of -30, -45 and -200): the
    chunked gradients must match the recurrence's, with no factor
    overflowing inside a chunk."""
    wl = small_workload(io, D, "channel", gates, T=T, B=2, Hqk=1, Hv=Hv, S0=True, scale=D ** -0.5)
    got, ref = _run(wl, seed=81 + D, g_fn=lambda g: strong_channel_decay(g, T, D))
    _check(got, ref, 1e-4)


@pytest.mark.parametrize("D,B,H,decay,gates", [(128, 1, 40, "channel", "bw"), (128, 1, 40, "scalar", "beta"),
                                                (64, 2, 36, "channel", "beta")])
def test_chunk_backward_many_heads(D, B, H, decay, gates):
    """Enough (sequence, head) pairs that the two sweeps' workgroups do not
    fit on the GPU at once: the backward sweep then forms every product of
    its step itself (with fewer pairs, as in the other tests, the
    dS_next-independent products come from a pass of their own). Sampled
    heads against the oracle."""
    wl = small_workload("bf16", D, decay, gates, T=130, B=B, Hqk=H, Hv=H, S0=True, scale=D ** -0.5)
    heads = [0, H // 2 - 1, H - 1]
    got, ref = _run(wl, seed=21 + D, heads=heads)
    _check(got, ref, 1e-4, heads=heads, qk_heads=heads)


def test_chunk_backward_qwen_shape_medium():
    wl = gs.QWEN_GDN_PREFILL.scaled(T=300, Hqk=2, Hv=6, name="qwen_like_T300")
    got, ref = _run(wl, seed=7)
    _check(got, ref, 1e-4)


def test_chunk_backward_qwen_full_size_sampled_group():
    """The Qwen-shaped layer (T = 4096, 16 QK heads, 48 V heads, d = 128,
    bf16) on the GPU; the oracle forms the gradients of QK head 5's group (V
    heads 15-17), which dq and dk of QK head 5 need in full."""
    wl = gs.QWEN_GDN_PREFILL
    heads = [15, 16, 17]
    got, ref = _run(wl, seed=11, heads=heads)
    _check(got, ref, 1e-3, heads=heads, qk_heads=[5])


@pytest.mark.parametrize("decay,gates", [("scalar", "beta"), ("channel", "bw")])
def test_chunk_backward_matches_recurrent_form(decay, gates):
    """The chunked and the recurrent gradients of one call agree to fp32
    rounding over 1000 tokens (16 chunks, a ragged last one)."""
    import gated_delta_rule_23_amd as gdr
    wl = small_workload("bf16", 128, decay, gates, T=1000, B=1, Hqk=2, Hv=4, S0=True, scale=128 ** -0.5)
    _, gr, d = _dev_inputs(wl, 13)
    a = _call(gdr.gdr_chunk_bwd, d, gr, wl)
    r = _call(gdr.gdr_recurrent_bwd, d, gr, wl)
    torch.cuda.synchronize()
    assert set(a) == set(r)
    for name in a:
        err = rel_err(a[name].cpu().numpy().astype(np.float64), r[name].cpu().numpy().astype(np.float64))
        say(f"  {name}: {err:.2e}")
        assert err < 1e-4, f"{name}: {err:.3e}"


def test_chunk_backward_zero_tokens_passes_dST_through():
    import gated_delta_rule_23_amd as gdr
    wl = small_workload("bf16", 64, "scalar", "beta", T=0, B=2, Hqk=1, Hv=2, S0=True)
    _, gr, d = _dev_inputs(wl, 0)
    out = _call(gdr.gdr_chunk_bwd, d, gr, wl)
    torch.cuda.synchronize()
    assert np.array_equal(out["dS0"].cpu().numpy(), gr["dST"])


def test_chunk_backward_is_deterministic():
    import gated_delta_rule_23_amd as gdr
    wl = small_workload("bf16", 128, "channel", "bw", T=177, B=1, Hqk=2, Hv=4, S0=True)
    _, gr, d = _dev_inputs(wl, 1)
    runs = [_call(gdr.gdr_chunk_bwd, d, gr, wl) for _ in range(2)]
    torch.cuda.synchronize()
    for name in runs[0]:
        assert torch.equal(runs[0][name], runs[1][name]), name


def test_chunk_backward_graph_replay_matches_eager():
    """The chunked backward captured into a HIP graph (its kernels, no memory
    set) and replayed three times, with eager work between the replays,
    gives the eager call's gradients bit for bit each time."""
    import gated_delta_rule_23_amd as gdr
    wl = small_workload("bf16", 64, "scalar", "beta", T=137, B=2, Hqk=1, Hv=3, S0=True)
    _, gr, d = _dev_inputs(wl, 4)
    do, dST = to_dev(gr["do"]), to_dev(gr["dST"])
    ref = gdr.gdr_chunk_bwd(d["q"], d["k"], d["v"], do, g=d["g"], beta=d["beta"], S0=d["S0"], dST=dST)
    torch.cuda.synchronize()
    ref = {k: v.clone() for k, v in ref.items()}
    desc = gdr.make_desc(2, 137, 1, 3, 64, gdr.GDR_BF16, gdr.GDR_DECAY_SCALAR, 1.0)
    ws = torch.empty(gdr.gdr_chunk_bwd_workspace_bytes(desc), dtype=torch.uint8, device="cuda")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        gdr.gdr_chunk_bwd(d["q"], d["k"], d["v"], do, g=d["g"], beta=d["beta"], S0=d["S0"], dST=dST, workspace=ws)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        gout = gdr.gdr_chunk_bwd(d["q"], d["k"], d["v"], do, g=d["g"], beta=d["beta"], S0=d["S0"], dST=dST,
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
