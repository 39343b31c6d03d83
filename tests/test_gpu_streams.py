"""Calls made on a stream other than the current one: the tensors the
binding allocates (outputs, workspace) belong to the call's stream, so the
caching allocator cannot hand their memory to work on the current stream
while the call's kernels still run. Each call is compared bit for bit with
the same call on the current stream."""
import numpy as np
import pytest

import gdr_synth as gs
from parity_util import from_dev, say, small_workload, to_dev

torch = pytest.importorskip("torch")
pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def _scribble(nbytes):
    """Allocations on the current stream, filled with NaN: they would take
    freed memory of another stream's call if that memory had been made on
    the current stream."""
    return [torch.full((max(nbytes // 4, 1),), float("nan"), device="cuda:0") for _ in range(3)]


@pytest.mark.parametrize("handle", [False, True])
def test_chunk_fwd_on_a_side_stream(handle):
    import gated_delta_rule_23_amd as gdr
    wl = small_workload("bf16", 128, "channel", "beta", T=700, B=2, Hqk=2, Hv=4, S0=True, scale=128 ** -0.5)
    inp = gs.make_inputs(wl, seed=21)
    d = {n: to_dev(inp[n]) for n in ("q", "k", "v", "g", "beta", "b", "w", "S0")}
    args = dict(g=d["g"], beta=d["beta"], b=d["b"], w=d["w"], S0=d["S0"], scale=wl.scale)
    o_ref, ST_ref = gdr.gdr_chunk_fwd(d["q"], d["k"], d["v"], **args)
    o_ref, ST_ref = from_dev(o_ref), from_dev(ST_ref)
    say(f"side stream chunk_fwd handle={handle}")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    nbytes = 0
    for _ in range(4):
        o, ST = gdr.gdr_chunk_fwd(d["q"], d["k"], d["v"], stream=side.cuda_stream if handle else side, **args)
        nbytes = o.numel() * 2
        junk = _scribble(nbytes)
        side.synchronize()
        assert np.array_equal(from_dev(o), o_ref) and np.array_equal(from_dev(ST), ST_ref)
        del junk, o, ST


def test_chunk_bwd_and_norm_la_on_a_side_stream():
    import gated_delta_rule_23_amd as gdr
    wl = small_workload("f32", 64, "scalar", "bw", T=300, B=2, Hqk=1, Hv=2, S0=True)
    inp = gs.make_inputs(wl, seed=22)
    gr = gs.make_output_grads(wl, seed=22)
    d = {n: to_dev(inp[n]) for n in ("q", "k", "v", "g", "beta", "b", "w", "S0")}
    do, dST = to_dev(gr["do"]), to_dev(gr["dST"])
    args = dict(g=d["g"], beta=d["beta"], b=d["b"], w=d["w"], S0=d["S0"], dST=dST, scale=wl.scale)
    ref = {k: from_dev(v) for k, v in gdr.gdr_chunk_bwd(d["q"], d["k"], d["v"], do, **args).items()}
    nin = gs.make_norm_la_inputs(1, 1500, 1, 2, 64, io="bf16", seed=23, state=True)
    nq, nk, nv, nS, nz = (to_dev(nin[n]) for n in ("phq", "phk", "v", "S0", "z0"))
    nref = [from_dev(x) for x in gdr.gdr_norm_la_fwd(nq, nk, nv, S0=nS, z0=nz)]
    say("side stream chunk_bwd and norm_la_fwd")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    out = gdr.gdr_chunk_bwd(d["q"], d["k"], d["v"], do, stream=side, **args)
    nout = gdr.gdr_norm_la_fwd(nq, nk, nv, S0=nS, z0=nz, stream=side)
    junk = _scribble(64 << 20)
    side.synchronize()
    for k, v in out.items():
        assert np.array_equal(from_dev(v), ref[k]), k
    for x, r in zip(nout, nref):
        assert np.array_equal(from_dev(x), r)
    del junk
