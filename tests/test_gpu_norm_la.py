"""GPU parity of normalised linear attention (gdr_norm_la_fwd and
gdr_norm_la_decode_step, through the C ABI) against the fp64 oracle
(oracle/norm_la.py, pinned by the brute-force weighted average, closed
forms and invariances).

Shapes span several chunks and a ragged tail, both io dtypes and every
head dimension; grouped heads; an incoming state or none; sequences split
into segments that run side by side; in-place state updates; T = 0;
consecutive decode steps; and a Qwen-like layer at full size (B = 1,
T = 4096, 16 QK heads, 48 V heads, d = 128, bf16) on sampled heads.
Tolerance as for the rest of the path: max |x - ref| / max |ref| below 2e-2
with bf16 io (the state enters Q S rounded to bf16), 1e-4 with fp32 io.
"""
import numpy as np
import pytest

import gdr_synth as gs
from oracle import norm_la
from parity_util import TOL, from_dev, out_err, rel_err, say, to_dev

torch = pytest.importorskip("torch")
pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def _gpu(inp, S0=None, z0=None, ST=None, zT=None):
    import gated_delta_rule_23_amd as gdr
    o, S, z = gdr.gdr_norm_la_fwd(to_dev(inp["phq"]), to_dev(inp["phk"]), to_dev(inp["v"]), S0=S0, z0=z0,
                                  ST=ST, zT=zT)
    torch.cuda.synchronize()
    return from_dev(o), from_dev(S), from_dev(z)


def _check(got, ref, io):
    for name, x, r in zip(("o", "S_T", "z_T"), got, ref):
        assert np.all(np.isfinite(x)), name
        err = out_err(x, r) if name == "o" else rel_err(x, r)
        say(f"  {name}: {err:.2e}")
        assert err < TOL[io], f"{name}: {err:.3e}"


@pytest.mark.parametrize("io", ["bf16", "f32"])
@pytest.mark.parametrize("D", [32, 64, 128])
@pytest.mark.parametrize("T", [1, 63, 64, 65, 150])
@pytest.mark.parametrize("state", [False, True])
def test_norm_la_small(io, D, T, state):
    inp = gs.make_norm_la_inputs(2, T, 1, 2, D, io=io, seed=T + D, state=state)
    say(f"norm_la B2 T{T} D{D} {io} state={state}")
    got = _gpu(inp, S0=to_dev(inp["S0"]), z0=to_dev(inp["z0"]))
    _check(got, norm_la.recurrent(inp["phq"], inp["phk"], inp["v"], inp["S0"], inp["z0"]), io)


@pytest.mark.parametrize("io,D", [("bf16", 128), ("f32", 64)])
def test_norm_la_grouped_heads(io, D):
    inp = gs.make_norm_la_inputs(2, 333, 2, 6, D, io=io, seed=5, state=True)
    say(f"norm_la grouped heads D{D} {io}")
    got = _gpu(inp, S0=to_dev(inp["S0"]), z0=to_dev(inp["z0"]))
    _check(got, norm_la.recurrent(inp["phq"], inp["phk"], inp["v"], inp["S0"], inp["z0"]), io)


@pytest.mark.parametrize("io,D,T", [("bf16", 64, 2000), ("f32", 32, 1500), ("bf16", 128, 1100)])
def test_norm_la_segments_side_by_side(io, D, T):
    """Few heads and a long sequence: the sequence runs as segments side by
    side (the segment sums, their running sum, then the segment sweeps)."""
    import gated_delta_rule_23_amd as gdr
    inp = gs.make_norm_la_inputs(1, T, 1, 2, D, io=io, seed=T, state=True)
    desc = gdr.make_desc(1, T, 1, 2, D, gdr.GDR_BF16 if io == "bf16" else gdr.GDR_F32, gdr.GDR_DECAY_NONE)
    assert gdr.gdr_norm_la_workspace_bytes(desc) > 0  # more than one segment
    say(f"norm_la segments T{T} D{D} {io}")
    got = _gpu(inp, S0=to_dev(inp["S0"]), z0=to_dev(inp["z0"]))
    _check(got, norm_la.recurrent(inp["phq"], inp["phk"], inp["v"], inp["S0"], inp["z0"]), io)


@pytest.mark.parametrize("T", [150, 2000])
def test_norm_la_in_place_state(T):
    """ST = S0 and zT = z0: the update in place gives the out-of-place result,
    with one segment and with several."""
    inp = gs.make_norm_la_inputs(1, T, 1, 2, 64, io="f32", seed=3, state=True)
    say(f"norm_la in place T{T}")
    S, z = to_dev(inp["S0"]), to_dev(inp["z0"])
    got = _gpu(inp, S0=S, z0=z, ST=S, zT=z)
    ref = _gpu(inp, S0=to_dev(inp["S0"]), z0=to_dev(inp["z0"]))
    assert np.array_equal(got[0], ref[0]) and np.array_equal(got[1], ref[1])
    assert rel_err(got[2], ref[2]) < 1e-6  # z_T in place is summed by a pass of its own
    _check(got, norm_la.recurrent(inp["phq"], inp["phk"], inp["v"], inp["S0"], inp["z0"]), "f32")


def test_norm_la_zero_tokens_pass_the_state_through():
    import gated_delta_rule_23_amd as gdr
    inp = gs.make_norm_la_inputs(2, 1, 1, 2, 32, io="f32", seed=4, state=True)
    q = torch.empty((2, 0, 1, 32), dtype=torch.float32, device="cuda:0")
    v = torch.empty((2, 0, 2, 32), dtype=torch.float32, device="cuda:0")
    say("norm_la T = 0")
    o, S, z = gdr.gdr_norm_la_fwd(q, q, v, S0=to_dev(inp["S0"]), z0=to_dev(inp["z0"]))
    torch.cuda.synchronize()
    assert o.shape == (2, 0, 2, 32)
    assert np.array_equal(from_dev(S), inp["S0"]) and np.array_equal(from_dev(z), inp["z0"])


@pytest.mark.parametrize("io,D", [("bf16", 128), ("f32", 64), ("bf16", 32)])
def test_norm_la_decode_steps(io, D):
    """Consecutive decode steps from a state equal the prefill of the same
    tokens: each step's output and the final state against the oracle."""
    import gated_delta_rule_23_amd as gdr
    steps, B = 20, 3
    inp = gs.make_norm_la_inputs(B, steps, 2, 4, D, io=io, seed=D, state=True)
    S, z = to_dev(inp["S0"]), to_dev(inp["z0"])
    q, k, v = to_dev(inp["phq"]), to_dev(inp["phk"]), to_dev(inp["v"])
    say(f"norm_la decode {steps} steps D{D} {io}")
    outs = []
    for t in range(steps):
        outs.append(from_dev(gdr.gdr_norm_la_decode_step(q[:, t].contiguous(), k[:, t].contiguous(),
                                                         v[:, t].contiguous(), S, z)))
    torch.cuda.synchronize()
    got = (np.stack(outs, axis=1), from_dev(S), from_dev(z))
    _check(got, norm_la.recurrent(inp["phq"], inp["phk"], inp["v"], inp["S0"], inp["z0"]), io)


def test_norm_la_qwen_like_full_size_sampled_heads():
    """B = 1, T = 4096, 16 QK heads and 48 V heads of d = 128, bf16: every
    output of the sampled V heads and their final states and normalisers."""
    B, T, Hqk, Hv, D = 1, 4096, 16, 48, 128
    inp = gs.make_norm_la_inputs(B, T, Hqk, Hv, D, io="bf16", seed=11, state=False)
    say("norm_la Qwen-like T4096 Hqk16 Hv48 d128")
    o, S, z = _gpu(inp)
    for h in (0, 1, 25, 47):
        hq = h // (Hv // Hqk)
        ref = norm_la.recurrent(inp["phq"][:, :, hq:hq + 1], inp["phk"][:, :, hq:hq + 1], inp["v"][:, :, h:h + 1])
        _check((o[:, :, h:h + 1], S[:, h:h + 1], z[:, h:h + 1]), ref, "bf16")
