"""Pins of the input-stage oracle (oracle/input_stage.py) against values the
mathematics fixes: a hand-worked convolution, numpy's own convolution,
impulse and shift taps, continuation through the convolution state, unit
norms, closed forms of sigmoid and softplus, and the end-to-end identity
with the recurrence when the stage is made transparent."""
import math

import numpy as np
import pytest

import gdr_synth as gs
import oracle
from oracle import input_stage as ist


def test_conv_hand_worked():
    # One channel, taps (1, 2, 3, 4), three state tokens (-1, 0, 1) then
    # x = 1..5. Worked by hand: y_0 = -1*1 + 0*2 + 1*3 + 1*4 = 6,
    # y_1 = 0 + 2 + 3 + 8 = 13, y_2 = 1 + 2 + 6 + 12 = 21,
    # y_3 = 1 + 4 + 9 + 16 = 30, y_4 = 2 + 6 + 12 + 20 = 40.
    x = np.array([1.0, 2.0, 3.0, 4.0, 5.0]).reshape(1, 5, 1)
    taps = np.array([[1.0, 2.0, 3.0, 4.0]])
    state = np.array([-1.0, 0.0, 1.0]).reshape(1, 3, 1)
    y, new_state = ist.causal_conv4(x, taps, state)
    assert y.ravel().tolist() == [6.0, 13.0, 21.0, 30.0, 40.0]
    assert new_state.ravel().tolist() == [3.0, 4.0, 5.0]


def test_conv_matches_numpy_convolve():
    rng = np.random.default_rng(0)
    B, T, Ch = 2, 11, 5
    x = rng.standard_normal((B, T, Ch))
    taps = rng.standard_normal((Ch, 4))
    state = rng.standard_normal((B, 3, Ch))
    y, _ = ist.causal_conv4(x, taps, state)
    for b in range(B):
        for c in range(Ch):
            xx = np.concatenate([state[b, :, c], x[b, :, c]])
            ref = np.convolve(xx, taps[c, ::-1], mode="valid")   # correlation with the taps
            assert np.allclose(y[b, :, c], ref, rtol=0, atol=1e-13)


def test_conv_impulse_and_shift_taps():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((1, 7, 3))
    state = rng.standard_normal((1, 3, 3))
    y, st = ist.causal_conv4(x, np.tile([0.0, 0.0, 0.0, 1.0], (3, 1)), state)
    assert np.array_equal(y, x) and np.array_equal(st, x[:, 4:7])
    y, _ = ist.causal_conv4(x, np.tile([0.0, 0.0, 1.0, 0.0], (3, 1)), state)
    assert np.array_equal(y[:, 1:], x[:, :-1]) and np.array_equal(y[:, 0], state[:, 2])
    y, _ = ist.causal_conv4(x, np.tile([1.0, 0.0, 0.0, 0.0], (3, 1)), None)
    assert np.array_equal(y[:, 3:], x[:, :-3]) and not np.any(y[:, :3])


def test_conv_state_continuation_and_short_calls():
    """Convolving T tokens at once equals convolving them in pieces, each
    piece starting from the state the previous one left, including pieces of
    1 and 2 tokens (shorter than the state)."""
    rng = np.random.default_rng(2)
    x = rng.standard_normal((2, 13, 4))
    taps = rng.standard_normal((4, 4))
    s0 = rng.standard_normal((2, 3, 4))
    y_all, s_all = ist.causal_conv4(x, taps, s0)
    s, ys = s0, []
    for a, b in ((0, 1), (1, 3), (3, 4), (4, 10), (10, 13)):
        y, s = ist.causal_conv4(x[:, a:b], taps, s)
        ys.append(y)
    assert np.allclose(np.concatenate(ys, axis=1), y_all, rtol=0, atol=1e-14)
    assert np.array_equal(s, s_all)


def test_l2norm_unit_and_zero():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((3, 4, 128)) * 7.0
    n = ist.l2norm(x)
    assert np.allclose(np.linalg.norm(n, axis=-1), 1.0, rtol=0, atol=1e-14)
    assert np.allclose(n * np.linalg.norm(x, axis=-1, keepdims=True), x, rtol=1e-13)
    assert not np.any(ist.l2norm(np.zeros((2, 8))))


def test_stage_normalises_q_and_k_not_v():
    """From arbitrary raw inputs (impulse taps), q and k leave the stage with
    unit norm per (token, head) and their directions unchanged; v keeps its
    raw values."""
    rng = np.random.default_rng(8)
    B, T, Hqk, Hv, d = 2, 5, 2, 4, 16
    xq, xk = 3.0 * rng.standard_normal((B, T, Hqk, d)), 0.2 * rng.standard_normal((B, T, Hqk, d))
    xv = 5.0 * rng.standard_normal((B, T, Hv, d))
    taps = np.tile([0.0, 0.0, 0.0, 1.0], (ist.conv_channels(Hqk, Hv, d, d), 1))
    out, _ = ist.input_stage(xq, xk, xv, taps, beta=np.zeros((B, T, Hv)))
    for name, raw in (("q", xq), ("k", xk)):
        assert np.allclose(np.linalg.norm(out[name], axis=-1), 1.0, rtol=0, atol=1e-10)   # eps 1e-12 inside the root
        assert np.allclose(out[name] * np.linalg.norm(raw, axis=-1, keepdims=True), raw, rtol=1e-10)
    assert np.array_equal(out["v"], xv)


def test_gate_functions_closed_forms():
    assert ist.sigmoid(np.array([0.0]))[0] == 0.5
    xs = np.array([-30.0, -2.5, -0.1, 0.3, 4.0, 700.0, -700.0])
    assert np.allclose(ist.sigmoid(xs) + ist.sigmoid(-xs), 1.0, rtol=0, atol=1e-15)
    assert abs(ist.sigmoid(np.array([math.log(3.0)]))[0] - 0.75) < 1e-15
    assert abs(ist.softplus(np.array([0.0]))[0] - math.log(2.0)) < 1e-16
    assert np.allclose(ist.softplus(xs) - ist.softplus(-xs), xs, rtol=0, atol=1e-12)
    assert ist.softplus(np.array([1000.0]))[0] == 1000.0          # no overflow
    assert 0.0 < ist.softplus(np.array([-50.0]))[0] < 2e-22


def test_decay_mapping_and_scale():
    """g = -c softplus(x) per V head: g <= 0, alpha = exp(g) in (0, 1], and
    c = 1 with x = -y gives log sigmoid(y)."""
    rng = np.random.default_rng(4)
    xq = rng.standard_normal((1, 5, 1, 4))
    xv = rng.standard_normal((1, 5, 3, 4))
    taps = np.tile([0.0, 0.0, 0.0, 1.0], (2 * 4 + 3 * 4, 1))
    y = rng.standard_normal((1, 5, 3))
    out, _ = ist.input_stage(xq, xq, xv, taps, g=-y, beta=y, decay_scale=np.array([1.0, 0.1, 0.05]))
    assert np.allclose(out["g"][..., 0], np.log(ist.sigmoid(y[..., 0])), rtol=0, atol=1e-14)
    assert np.allclose(out["g"][..., 1], 0.1 * np.log(ist.sigmoid(y[..., 1])), rtol=0, atol=1e-14)
    assert np.all(out["g"] <= 0.0)
    assert np.allclose(out["beta"], ist.sigmoid(y))


def test_channel_order_of_the_stage():
    """The taps and the state are ordered q channels, k channels, v
    channels: an impulse on one tap column of one block shows up only in that
    tensor."""
    rng = np.random.default_rng(5)
    B, T, Hqk, Hv, d = 1, 4, 2, 4, 8
    xq, xk = rng.standard_normal((B, T, Hqk, d)), rng.standard_normal((B, T, Hqk, d))
    xv = rng.standard_normal((B, T, Hv, d))
    ch = ist.conv_channels(Hqk, Hv, d, d)
    taps = np.zeros((ch, 4))
    taps[2 * Hqk * d:, 3] = 1.0          # v passes through, q and k are zeroed
    out, _ = ist.input_stage(xq, xk, xv, taps, beta=np.zeros((B, T, Hv)))
    assert np.array_equal(out["v"], xv)
    assert not np.any(out["q"]) and not np.any(out["k"])
    taps = np.zeros((ch, 4))
    taps[Hqk * d:2 * Hqk * d, 3] = 2.0   # only k passes (scaled, then normalised)
    out, _ = ist.input_stage(xq, xk, xv, taps, beta=np.zeros((B, T, Hv)))
    assert np.allclose(out["k"], ist.l2norm(xk)) and not np.any(out["q"]) and not np.any(out["v"])


def test_transparent_stage_equals_plain_recurrence():
    """With impulse taps, already unit-norm q and k, gate inputs equal to the
    logits of stored gates and decay inputs whose softplus is the stored
    -g, the stage feeds the recurrence the stored values, so the outputs
    equal the plain oracle's."""
    wl = gs.Workload("t", 2, 9, 1, 2, 16, 16, "f32", "channel", "bw", "softplus_0.05", S0="normal_0.02")
    inp = gs.make_inputs(wl, seed=6)
    q, k, v = (oracle.upcast(inp[n]) for n in ("q", "k", "v"))
    q, k = ist.l2norm(q), ist.l2norm(k)
    b, w, g = (oracle.upcast(inp[n]) for n in ("b", "w", "g"))
    logit = lambda p: np.log(p) - np.log1p(-p)
    g_in = np.log(np.expm1(-g))                  # softplus(g_in) = -g
    ch = ist.conv_channels(1, 2, 16, 16)
    taps = np.tile([0.0, 0.0, 0.0, 1.0], (ch, 1))
    st, _ = ist.input_stage(q, k, v, taps, g=g_in, b=logit(b), w=logit(w))
    o1, S1 = oracle.recurrent(st["q"], st["k"], st["v"], g=st["g"], b=st["b"], w=st["w"], S0=inp["S0"])
    o2, S2 = oracle.recurrent(q, k, v, g=g, b=b, w=w, S0=inp["S0"])
    assert np.allclose(o1, o2, rtol=0, atol=1e-10) and np.allclose(S1, S2, rtol=0, atol=1e-10)


@pytest.mark.parametrize("io", ["bf16", "f32"])
def test_raw_input_recipe(io):
    """The raw-input generator's shapes and the decay recipe it encodes."""
    wl = gs.Workload("r", 2, 6, 2, 4, 32, 32, io, "scalar", "beta", "softplus_0.1")
    r = gs.make_raw_inputs(wl, seed=0)
    ch = ist.conv_channels(2, 4, 32, 32)
    assert r["conv_w"].shape == (ch, 4) and r["conv_in"].shape == (2, 3, ch)
    assert np.all(r["decay_scale"] == np.float32(0.1))
    out, conv_out = ist.input_stage(r["q"], r["k"], r["v"], r["conv_w"], conv_in=r["conv_in"], g=r["g"],
                                    beta=r["beta"], decay_scale=r["decay_scale"])
    assert np.all(out["g"] <= 0) and np.all((out["beta"] > 0) & (out["beta"] < 1))
    assert np.array_equal(conv_out[:, 2, :2 * 32], oracle.upcast(r["q"])[:, -1].reshape(2, -1))
