"""Planted mistakes in the input-stage oracle: its pins must catch each one.

Each case copies ``oracle/input_stage.py``, replaces one snippet with a
plausible mistake (taps reversed, the incoming state ignored, the window or
the outgoing state shifted, the norm over the wrong axis or without its
square root, a sign slip in the sigmoid or the decay, the max term of
softplus or the per-head decay constant dropped, q left unnormalised, v
normalised, q and k channels swapped), loads the copy as a module and runs
the pins of ``test_oracle_input_stage`` against it. The unmodified source
must pass every pin and each mutant must fail at least one. CPU only.
"""
import importlib.util
import os
import sys

import pytest

import oracle
import test_oracle_input_stage as pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "input_stage.py")

MUTANTS = {
    "taps_reversed": ("y += taps[:, j] * xx[:, j:j + T, :]", "y += taps[:, 3 - j] * xx[:, j:j + T, :]"),
    "state_ignored": ("prev = np.zeros((B, 3, Ch)) if state is None else upcast(state)",
                      "prev = np.zeros((B, 3, Ch))"),
    "window_shifted": ("y += taps[:, j] * xx[:, j:j + T, :]", "y += taps[:, j] * xx[:, max(j - 1, 0):max(j - 1, 0) + T, :]"),
    "state_out_shifted": ("return y, xx[:, T:T + 3, :].copy()", "return y, xx[:, T - 1:T + 2, :].copy()"),
    "norm_wrong_axis": ("np.sum(x * x, axis=-1, keepdims=True)", "np.sum(x * x, axis=-2, keepdims=True)"),
    "norm_without_sqrt": ("x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + NORM_EPS)",
                          "x / (np.sum(x * x, axis=-1, keepdims=True) + NORM_EPS)"),
    "sigmoid_sign": ("out[pos] = 1.0 / (1.0 + np.exp(-x[pos]))", "out[pos] = 1.0 / (1.0 + np.exp(x[pos]))"),
    "softplus_without_max": ("return np.maximum(x, 0.0) + np.log1p(np.exp(-np.abs(x)))",
                             "return np.log1p(np.exp(-np.abs(x)))"),
    "decay_sign": ('out["g"] = -c * softplus(g)', 'out["g"] = c * softplus(g)'),
    "decay_scale_ignored": ("c = np.ones(Hv) if decay_scale is None else upcast(decay_scale)", "c = np.ones(Hv)"),
    "q_unnormalised": ('"q": l2norm(y[:, :, :nq].reshape(B, T, Hqk, dk)),', '"q": y[:, :, :nq].reshape(B, T, Hqk, dk),'),
    "v_normalised": ('"v": y[:, :, 2 * nq:].reshape(B, T, Hv, dv),', '"v": l2norm(y[:, :, 2 * nq:].reshape(B, T, Hv, dv)),'),
    "q_k_channels_swapped": ('"q": l2norm(y[:, :, :nq].reshape(B, T, Hqk, dk)),\n        "k": l2norm(y[:, :, nq:2 * nq].reshape(B, T, Hqk, dk)),',
                             '"q": l2norm(y[:, :, nq:2 * nq].reshape(B, T, Hqk, dk)),\n        "k": l2norm(y[:, :, :nq].reshape(B, T, Hqk, dk)),'),
}

PINS = [getattr(pins, n) for n in dir(pins) if n.startswith("test_") and n != "test_raw_input_recipe"]


def _load(src, name):
    path = os.path.join(os.environ.get("TMPDIR", "/tmp"), f"gdr_ist_{name}_{os.getpid()}.py")
    with open(path, "w") as f:
        f.write(src.replace("from . import upcast", "from oracle import upcast"))
    try:
        spec = importlib.util.spec_from_file_location(f"gdr_ist_{name}", path)
        mod = importlib.util.module_from_spec(spec)
        spec.loader.exec_module(mod)
        return mod
    finally:
        os.remove(path)


def _failures(mod):
    """Names of the pins that fail when the pins run against module mod."""
    saved = pins.ist
    pins.ist = mod
    failed = []
    try:
        for pin in PINS:
            try:
                pin()
            except Exception:  # an assertion or a crash both count as caught
                failed.append(pin.__name__)
    finally:
        pins.ist = saved
    return failed


def test_unmodified_source_passes_every_pin():
    with open(SRC) as f:
        src = f.read()
    assert _failures(_load(src, "original")) == []


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    old, new = MUTANTS[name]
    with open(SRC) as f:
        src = f.read()
    assert src.count(old) >= 1, f"snippet for {name} not found"
    failed = _failures(_load(src.replace(old, new), name))
    assert failed, f"no pin catches the mutant {name}"
