"""The seeded input generator: rounding, determinism, recipe."""
import numpy as np
import pytest

import gdr_synth as gs


def test_bf16_round_to_nearest_even_ties():
    one = 1.0
    x = np.array([one, one + 2.0 ** -8, one + 3 * 2.0 ** -8, one + 2.0 ** -8 + 2.0 ** -40,
                  -(one + 2.0 ** -8), 0.0, 3.0e38, 1.5e-38])
    bits = gs.bf16_bits(x)
    # 1 + 2^-8 is halfway between 1 and 1 + 2^-7: ties go to the even mantissa (1.0).
    # 1 + 3*2^-8 is halfway between 1 + 2^-7 and 1 + 2^-6: goes to 1 + 2^-6.
    assert list(bits[:6]) == [0x3F80, 0x3F80, 0x3F82, 0x3F81, 0xBF80, 0x0000]
    # Near the ends of the range the rounding is still one step from fp64.
    assert bits[6] == 0x7F62 and bits[7] == 0x00A3


def test_bf16_matches_torch_on_float32_inputs():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(0)
    x = rng.standard_normal(100000).astype(np.float32)
    ours = gs.bf16_bits(x.astype(np.float64))
    theirs = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, theirs)


def test_bf16_rejects_out_of_range():
    with pytest.raises(ValueError):
        gs.bf16_bits(np.array([1e-40]))
    with pytest.raises(ValueError):
        gs.bf16_bits(np.array([np.inf]))


@pytest.mark.parametrize("wl", gs.WORKLOADS, ids=lambda w: w.name)
def test_recipe_small_versions(wl):
    small = wl.scaled(T=min(wl.T, 70), B=min(wl.B, 2))
    a = gs.make_inputs(small, seed=3)
    b = gs.make_inputs(small, seed=3)
    for name in gs.ORDER:
        if a[name] is None:
            assert b[name] is None
        else:
            assert np.array_equal(a[name], b[name])
    io = np.uint16 if wl.io == "bf16" else np.float32
    lead = (small.T, small.B) if small.decode else (small.B, small.T)
    assert a["q"].dtype == io and a["q"].shape == lead + (small.Hqk, small.dk)
    assert a["v"].shape == lead + (small.Hv, small.dv)
    qf = a["q"].astype(np.float64) if io == np.float32 else gs.bf16_to_f32(a["q"]).astype(np.float64)
    norms = np.linalg.norm(qf, axis=-1)
    assert np.all(np.abs(norms - 1) < (1e-6 if io == np.float32 else 2e-2))
    if a["g"] is not None:
        assert a["g"].dtype == np.float32 and np.all(a["g"] < 0)
    if a["beta"] is not None:
        assert np.all((a["beta"] > 0) & (a["beta"] < 1))
    else:
        assert a["b"] is not None and a["w"] is not None
    assert (a["S0"] is None) == (wl.S0 == "zero")


def test_different_seeds_differ_and_streams_are_independent():
    wl = gs.KDA_PREFILL.scaled(T=8, B=1, Hqk=2, Hv=2)
    a, b = gs.make_inputs(wl, 1), gs.make_inputs(wl, 2)
    assert not np.array_equal(a["q"], b["q"])
    # Same seed, a different gate layout: q, k, v are unchanged (one stream per tensor).
    c = gs.make_inputs(wl.scaled(gates="bw"), 1)
    assert np.array_equal(a["q"], c["q"]) and np.array_equal(a["v"], c["v"]) and np.array_equal(a["g"], c["g"])


def test_decode_layout_roundtrip():
    wl = gs.QWEN_GDN_DECODE.scaled(T=5, B=3, Hqk=2, Hv=6, dk=8, dv=8)
    a = gs.make_inputs(wl, 0)
    s = gs.as_sequence(a)
    assert s["q"].shape == (3, 5, 2, 8) and np.array_equal(s["q"][1, 4], a["q"][4, 1])
    assert s["beta"].shape == (3, 5, 6)
