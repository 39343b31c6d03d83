"""The C-ABI library on the CPU: it loads, exports every declared symbol, and
rejects bad arguments before any HIP call (so no GPU is needed here)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gdr.h")

gdr = pytest.importorskip("gated_delta_rule_23_amd")


def _declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(gdr_[a-z_]+)\s*\(", src)))


def test_every_declared_symbol_is_exported():
    names = _declared_functions()
    assert set(names) == set(gdr.EXPORTS)
    raw = ctypes.CDLL(gdr.LIB_PATH)
    for n in names:
        assert hasattr(raw, n), n


def test_version():
    assert gdr.gdr_version() == 1


def test_state_size_pin():
    """"Gated DeltaNet: o mixer em 48 das 64 camadas", "Conceito": 48 V heads of
    128 x 128 fp32 state are about 3 MiB per layer; "Linear attention e fast
    weights", "Conceito": about 144 MiB over the 48 DeltaNet layers."""
    per_layer = gdr.gdr_state_bytes(1, 48, 128, 128)
    assert per_layer == 3 * 2 ** 20
    assert 48 * per_layer == 144 * 2 ** 20
    assert gdr.gdr_state_bytes(0, 48, 128, 128) == 0


def _a256(x):
    return (x + 255) // 256 * 256


def test_workspace_bytes():
    """Scalar decay: Y, U_z^T and A per (sequence, V head, chunk), two per-token
    decay tables, and one k^T and one q per (sequence, QK head, chunk).
    Per-channel decay: also Q~ and Kend^T per unit, and gamma in the table."""
    NC, units = 64, 48 * 64
    d = gdr.make_desc(1, 4096, 16, 48, 128, gdr.GDR_BF16, gdr.GDR_DECAY_SCALAR)
    io = units * (2 * 64 * 128 + 64 * 64) * 2
    expect = _a256(io) + _a256(units * 128 * 4) + _a256(16 * NC * 2 * 128 * 64 * 2)
    assert gdr.gdr_chunk_workspace_bytes(d) == expect
    dc = gdr.make_desc(1, 4096, 16, 48, 128, gdr.GDR_BF16, gdr.GDR_DECAY_CHANNEL)
    io = units * (4 * 64 * 128 + 64 * 64) * 2
    assert gdr.gdr_chunk_workspace_bytes(dc) == _a256(io) + _a256(units * 128 * 4)
    d0 = gdr.make_desc(1, 0, 16, 48, 128, gdr.GDR_BF16, gdr.GDR_DECAY_SCALAR)
    assert gdr.gdr_chunk_workspace_bytes(d0) == 0


@pytest.mark.parametrize("io,segments", [(gdr.GDR_BF16, 7), (gdr.GDR_F32, 4)])
def test_workspace_bytes_split_sweep(io, segments):
    """A long sequence with few heads (T = 65536, 16 heads, d = 128): 64 sweep
    work items of 32 columns fill a quarter of the 256 CUs, so the sweep is
    split into 4 segments, or 1 + 384 / 64 = 7 with bf16 io (whose split sweep
    takes 64 columns per work item and whose segment pass runs three work
    items per CU); the workspace adds three d x d fp32 matrices
    (transition, end state, next entry state) per head and segment but the
    last."""
    NC, units = 1024, 16 * 1024
    esz = 2 if io == gdr.GDR_BF16 else 4
    d = gdr.make_desc(1, 65536, 16, 16, 128, io, gdr.GDR_DECAY_CHANNEL)
    expect = (_a256(units * (4 * 64 * 128 + 64 * 64) * esz) + _a256(units * 128 * 4)
              + _a256(3 * 16 * (segments - 1) * 128 * 128 * 4))
    assert gdr.gdr_chunk_workspace_bytes(d) == expect


@pytest.mark.parametrize("io", [gdr.GDR_BF16, gdr.GDR_F32])
@pytest.mark.parametrize("B,T,Hv,D", [(1, 65536, 16, 128), (1, 4113, 1, 128), (1, 2200, 1, 128), (1, 4096, 48, 128),
                                      (2, 16384, 32, 128), (1, 2500, 2, 64), (2, 2100, 1, 64), (1, 2100, 1, 32),
                                      (1, 5200, 16, 128), (3, 9000, 4, 128), (1, 640, 2, 128)])
def test_workspace_matches_segment_policy(io, B, T, Hv, D):
    """The segment count the GPU tests restate (to know which cases take the
    split sweep) is the one the library sizes its workspace for: three d x d
    fp32 matrices per (sequence, V head, segment but the last)."""
    from parity_util import sweep_segments
    NC, units = -(-T // 64), B * Hv * -(-T // 64)
    esz = 2 if io == gdr.GDR_BF16 else 4
    P = sweep_segments(B, Hv, D, T, "bf16" if io == gdr.GDR_BF16 else "f32")
    d = gdr.make_desc(B, T, Hv, Hv, D, io, gdr.GDR_DECAY_CHANNEL)
    expect = (_a256(units * (4 * 64 * D + 64 * 64) * esz) + _a256(units * 128 * 4)
              + (_a256(3 * B * Hv * (P - 1) * D * D * 4) if P > 1 else 0))
    assert gdr.gdr_chunk_workspace_bytes(d) == expect


def test_norm_la_workspace_bytes_segments():
    """Normalised linear attention on the Qwen-like layer (T = 4096, 48 V
    heads, d = 128): 96 sweep work items of 64 columns per segment at two per
    CU, so 5 segments fill the 256 CUs in one round; the workspace holds each
    segment's d x d sum and its d-vector normaliser in fp32."""
    d = gdr.make_desc(1, 4096, 16, 48, 128, gdr.GDR_BF16, gdr.GDR_DECAY_NONE)
    assert gdr.gdr_norm_la_workspace_bytes(d) == 48 * 5 * (128 * 128 + 128) * 4


P = 0x1000  # a fake non-NULL device pointer: validation never dereferences it


def _fwd(desc, q=P, k=P, v=P, g=P, beta=P, b=None, w=None, S0=None, o=P, ST=P, ws=P, wsz=1 << 40):
    return gdr.lib.gdr_chunk_fwd(ctypes.byref(desc), q, k, v, g, beta, b, w, S0, o, ST, ws, wsz, None)


def _dec(desc, q=P, k=P, v=P, g=P, beta=P, b=None, w=None, S=P, o=P):
    return gdr.lib.gdr_decode_step(ctypes.byref(desc), q, k, v, g, beta, b, w, S, o, None)


def _desc(**kw):
    base = dict(B=1, T=128, Hqk=2, Hv=6, D=64, io=gdr.GDR_BF16, decay=gdr.GDR_DECAY_SCALAR)
    base.update(kw)
    return gdr.make_desc(base["B"], base["T"], base["Hqk"], base["Hv"], base["D"], base["io"], base["decay"])


@pytest.mark.parametrize("case,expect", [
    (dict(desc=dict(Hv=5)), gdr.GDR_E_INVAL),
    (dict(desc=dict(Hqk=0)), gdr.GDR_E_INVAL),
    (dict(desc=dict(B=-1)), gdr.GDR_E_INVAL),
    (dict(desc=dict(T=-3)), gdr.GDR_E_INVAL),
    (dict(desc=dict(D=96)), gdr.GDR_E_UNSUPPORTED),
    (dict(desc=dict(D=256)), gdr.GDR_E_UNSUPPORTED),
    (dict(desc=dict(io=7)), gdr.GDR_E_INVAL),
    (dict(desc=dict(decay=5)), gdr.GDR_E_INVAL),
    (dict(desc=dict(io=gdr.GDR_F32, D=128, decay=gdr.GDR_DECAY_CHANNEL)), gdr.GDR_E_UNSUPPORTED),
    (dict(desc=dict(io=gdr.GDR_F32, D=128), args=dict(beta=None, b=P, w=P)), gdr.GDR_E_UNSUPPORTED),
    (dict(args=dict(q=None)), gdr.GDR_E_INVAL),
    (dict(args=dict(o=None)), gdr.GDR_E_INVAL),
    (dict(args=dict(ST=None)), gdr.GDR_E_INVAL),
    (dict(args=dict(g=None)), gdr.GDR_E_INVAL),                      # decay scalar needs g
    (dict(desc=dict(decay=gdr.GDR_DECAY_NONE)), gdr.GDR_E_INVAL),    # g given without decay
    (dict(args=dict(b=P, w=P)), gdr.GDR_E_INVAL),                    # beta and b, w together
    (dict(args=dict(beta=None, b=P)), gdr.GDR_E_INVAL),              # b without w
    (dict(args=dict(beta=None)), gdr.GDR_E_INVAL),                   # no gate at all
    (dict(args=dict(ws=None)), gdr.GDR_E_INVAL),
    (dict(args=dict(wsz=100)), gdr.GDR_E_INVAL),
    (dict(args=dict(q=P + 8)), gdr.GDR_E_INVAL),                     # 16-byte alignment
    (dict(args=dict(o=P + 4)), gdr.GDR_E_INVAL),
    (dict(args=dict(ws=P + 8)), gdr.GDR_E_INVAL),
    (dict(args=dict(beta=P + 2)), gdr.GDR_E_INVAL),
])
def test_prefill_rejections(case, expect):
    d = _desc(**case.get("desc", {}))
    rc = _fwd(d, **case.get("args", {}))
    assert rc == expect
    assert gdr.gdr_last_error() != ""


def test_prefill_rejects_other_chunk_sizes():
    d = _desc()
    d.chunk = 32
    assert _fwd(d) == gdr.GDR_E_UNSUPPORTED
    assert "chunk" in gdr.gdr_last_error()


def test_zero_batch_is_a_noop_without_gpu():
    assert _fwd(_desc(B=0)) == gdr.GDR_OK
    assert gdr.gdr_last_error() == ""
    assert _dec(_desc(B=0)) == gdr.GDR_OK


@pytest.mark.parametrize("case,expect", [
    (dict(desc=dict(Hv=4, Hqk=3)), gdr.GDR_E_INVAL),
    (dict(desc=dict(D=48)), gdr.GDR_E_UNSUPPORTED),
    (dict(args=dict(S=None)), gdr.GDR_E_INVAL),
    (dict(args=dict(g=None)), gdr.GDR_E_INVAL),
    (dict(args=dict(beta=None, b=P, w=None)), gdr.GDR_E_INVAL),
    (dict(args=dict(S=P + 8)), gdr.GDR_E_INVAL),
    (dict(args=dict(k=P + 2)), gdr.GDR_E_INVAL),
])
def test_decode_rejections(case, expect):
    d = _desc(**case.get("desc", {}))
    assert _dec(d, **case.get("args", {})) == expect


def _rec(desc, q=P, k=P, v=P, g=P, beta=P, b=None, w=None, S0=None, o=P, ST=P):
    return gdr.lib.gdr_recurrent_fwd(ctypes.byref(desc), q, k, v, g, beta, b, w, S0, o, ST, None)


@pytest.mark.parametrize("case,expect", [
    (dict(desc=dict(Hv=5)), gdr.GDR_E_INVAL),
    (dict(desc=dict(T=-1)), gdr.GDR_E_INVAL),
    (dict(desc=dict(D=96)), gdr.GDR_E_UNSUPPORTED),
    (dict(args=dict(ST=None)), gdr.GDR_E_INVAL),
    (dict(args=dict(v=None)), gdr.GDR_E_INVAL),
    (dict(args=dict(g=None)), gdr.GDR_E_INVAL),
    (dict(args=dict(beta=None, w=P)), gdr.GDR_E_INVAL),
    (dict(args=dict(S0=P + 8)), gdr.GDR_E_INVAL),                    # misaligned
    (dict(args=dict(S0=P, ST=P + 4096)), gdr.GDR_E_INVAL),           # overlapping, not equal
    (dict(args=dict(S0=P + 4096, ST=P)), gdr.GDR_E_INVAL),
])
def test_recurrent_rejections(case, expect):
    d = _desc(**case.get("desc", {}))
    assert _rec(d, **case.get("args", {})) == expect
    assert gdr.gdr_last_error() != ""


def _rec_in(desc, stage, q=P, k=P, v=P, g=P, beta=P, b=None, w=None, S0=None, o=P, ST=P):
    st = None if stage is None else ctypes.byref(gdr.gdr_input_stage(*stage))
    return gdr.lib.gdr_recurrent_fwd_in(ctypes.byref(desc), st, q, k, v, g, beta, b, w, S0, o, ST, None)


@pytest.mark.parametrize("stage,expect", [
    (None, gdr.GDR_E_INVAL),                                        # no stage
    ((None, None, None, None), gdr.GDR_E_INVAL),                    # no taps
    ((P + 8, None, None, None), gdr.GDR_E_INVAL),                   # misaligned taps
    ((P, P + 4, P + (1 << 20), None), gdr.GDR_E_INVAL),            # misaligned conv_in
    ((P, P, P + 64, None), gdr.GDR_E_INVAL),                        # conv_out overlaps conv_in
    ((P, P + 64, P, None), gdr.GDR_E_INVAL),
    ((P, None, None, P + 2), gdr.GDR_E_INVAL),                      # misaligned decay_scale
])
def test_recurrent_input_stage_rejections(stage, expect):
    assert _rec_in(_desc(), stage) == expect
    assert gdr.gdr_last_error() != ""


def test_recurrent_input_stage_zero_batch_and_separate_conv_buffers():
    d = _desc(B=0)
    assert _rec_in(d, (P, P, P + (1 << 20), P)) == gdr.GDR_OK
    assert gdr.gdr_last_error() == ""


def test_recurrent_accepts_what_the_chunked_path_does_not():
    """No chunk-length or float32-dimension limits: the chunk field is
    ignored and float32 io runs at d = 128. B = 0 is a no-op on the CPU."""
    d = _desc(B=0, io=gdr.GDR_F32, D=128)
    d.chunk = 32
    assert _rec(d) == gdr.GDR_OK
    assert gdr.gdr_last_error() == ""


# Backward: distinct, non-overlapping fake buffers 4 GiB apart, so a case fails
# only for the one thing it changes (validation never dereferences them).
_BWD_NAMES = ("q", "k", "v", "g", "beta", "b", "w", "S0", "dO", "dST", "dq", "dk", "dv", "dg", "dbeta", "db",
              "dw", "dS0", "ws")
_BWD_BASE = {n: (i + 1) << 32 for i, n in enumerate(_BWD_NAMES)}


def _bwd(desc, wsz=1 << 40, entry="gdr_recurrent_bwd", **kw):
    ptr = dict(_BWD_BASE, b=None, w=None, db=None, dw=None)
    ptr.update(kw)
    return getattr(gdr.lib, entry)(ctypes.byref(desc), *(ptr[n] for n in _BWD_NAMES), wsz, None)


def test_backward_workspace_bytes():
    """Checkpoints of the state entering every block of 4 tokens, then the
    per-tile partial sums (four [B,T,H_v,D] arrays and one [B,T,H_v] per 32
    value columns), each rounded up to 256 bytes."""
    d = gdr.make_desc(1, 100, 2, 4, 128, gdr.GDR_BF16, gdr.GDR_DECAY_SCALAR)
    ck = 25 * 4 * 128 * 128 * 4
    part = (4 * 4 * 100 * 4 * 128 + 4 * 100 * 4) * 4
    assert gdr.gdr_recurrent_bwd_workspace_bytes(d) == _a256(ck) + _a256(part)
    assert gdr.gdr_recurrent_bwd_workspace_bytes(gdr.make_desc(1, 0, 2, 4, 128, gdr.GDR_BF16,
                                                               gdr.GDR_DECAY_SCALAR)) == 0


def test_chunk_backward_workspace_bytes():
    """Per chunk unit (sequence, V head, chunk of 64): ten 64 x D arrays,
    four 64 x 64, two D x D and two of D floats; with grouped heads two more
    [B,T,H_v,D] arrays; each array rounded up to 256 bytes."""
    d = gdr.make_desc(1, 100, 2, 4, 128, gdr.GDR_BF16, gdr.GDR_DECAY_SCALAR)
    units = 1 * 4 * 2
    per = [64 * 128] * 10 + [64 * 64] * 4 + [128 * 128] * 2 + [128] * 2
    want = sum(_a256(units * f * 4) for f in per) + 2 * _a256(100 * 4 * 128 * 4)
    assert gdr.gdr_chunk_bwd_workspace_bytes(d) == want
    d = gdr.make_desc(2, 64, 4, 4, 64, gdr.GDR_F32, gdr.GDR_DECAY_CHANNEL)  # no grouping, float32 io, d = 64
    units = 2 * 4 * 1
    per = [64 * 64] * 10 + [64 * 64] * 4 + [64 * 64] * 2 + [64] * 2
    assert gdr.gdr_chunk_bwd_workspace_bytes(d) == sum(_a256(units * f * 4) for f in per)
    assert gdr.gdr_chunk_bwd_workspace_bytes(gdr.make_desc(1, 0, 2, 4, 128, gdr.GDR_BF16,
                                                           gdr.GDR_DECAY_SCALAR)) == 0
    d = gdr.make_desc(1, 100, 2, 4, 128, gdr.GDR_BF16, gdr.GDR_DECAY_SCALAR, chunk=32)
    with pytest.raises(gdr.GdrError):
        gdr.gdr_chunk_bwd_workspace_bytes(d)


def test_chunk_backward_rejects_other_chunk_lengths():
    d = _desc()
    d.chunk = 32
    assert _bwd(d, entry="gdr_chunk_bwd") == gdr.GDR_E_UNSUPPORTED
    assert gdr.gdr_last_error() != ""


@pytest.mark.parametrize("entry", ["gdr_recurrent_bwd", "gdr_chunk_bwd"])
@pytest.mark.parametrize("case,expect", [
    (dict(desc=dict(D=96)), gdr.GDR_E_UNSUPPORTED),
    (dict(desc=dict(Hv=5)), gdr.GDR_E_INVAL),
    (dict(args=dict(dO=None)), gdr.GDR_E_INVAL),
    (dict(args=dict(dq=None)), gdr.GDR_E_INVAL),
    (dict(args=dict(dv=None)), gdr.GDR_E_INVAL),
    (dict(args=dict(dg=None)), gdr.GDR_E_INVAL),                       # g given, dg missing
    (dict(desc=dict(decay=gdr.GDR_DECAY_NONE), args=dict(g=None)), gdr.GDR_E_INVAL),  # dg without g
    (dict(args=dict(dbeta=None)), gdr.GDR_E_INVAL),                    # beta given, dbeta missing
    (dict(args=dict(db=_BWD_BASE["db"], dw=_BWD_BASE["dw"])), gdr.GDR_E_INVAL),      # db, dw with tied gates
    (dict(args=dict(beta=None, dbeta=None, b=_BWD_BASE["b"], w=_BWD_BASE["w"],
                    db=_BWD_BASE["db"], dw=None)), gdr.GDR_E_INVAL),   # decoupled gates, dw missing
    (dict(args=dict(ws=None)), gdr.GDR_E_INVAL),
    (dict(wsz=100), gdr.GDR_E_INVAL),
    (dict(args=dict(dq=_BWD_BASE["q"])), gdr.GDR_E_INVAL),             # gradient over an input
    (dict(args=dict(dk=_BWD_BASE["dq"] + 64)), gdr.GDR_E_INVAL),       # two gradients overlap
    (dict(args=dict(dS0=_BWD_BASE["dST"])), gdr.GDR_E_INVAL),
    (dict(args=dict(dv=_BWD_BASE["ws"] + 256)), gdr.GDR_E_INVAL),      # gradient inside the workspace
    (dict(args=dict(dq=_BWD_BASE["dq"] + 4)), gdr.GDR_E_INVAL),        # 16-byte alignment
    (dict(args=dict(dg=_BWD_BASE["dg"] + 2)), gdr.GDR_E_INVAL),
    (dict(args=dict(dbeta=_BWD_BASE["dbeta"] + 1)), gdr.GDR_E_INVAL),
    (dict(args=dict(dST=_BWD_BASE["dST"] + 8)), gdr.GDR_E_INVAL),
])
def test_backward_rejections(entry, case, expect):
    d = _desc(**case.get("desc", {}))
    assert _bwd(d, wsz=case.get("wsz", 1 << 40), entry=entry, **case.get("args", {})) == expect
    assert gdr.gdr_last_error() != ""


@pytest.mark.parametrize("entry", ["gdr_recurrent_bwd", "gdr_chunk_bwd"])
def test_backward_zero_batch_is_a_noop_without_gpu(entry):
    assert _bwd(_desc(B=0), entry=entry) == gdr.GDR_OK
    assert gdr.gdr_last_error() == ""


def test_state_alloc_rejects_bad_sizes():
    p, n = ctypes.c_void_p(), ctypes.c_size_t()
    assert gdr.lib.gdr_state_alloc(0, 48, 128, 128, ctypes.byref(p), ctypes.byref(n), None) == gdr.GDR_E_INVAL
    assert gdr.lib.gdr_state_alloc(1, 48, 128, 128, None, None, None) == gdr.GDR_E_INVAL
    assert gdr.lib.gdr_state_free(None) == gdr.GDR_OK


def test_binding_rejects_bad_tensors():
    torch = pytest.importorskip("torch")
    q = torch.zeros(1, 4, 1, 32, dtype=torch.float64)
    with pytest.raises((TypeError, ValueError)):
        gdr.gdr_chunk_fwd(q, q, q, beta=torch.zeros(1, 4, 1))


def test_header_is_plain_c_and_links(tmp_path):
    """include/gdr.h compiles as C99 with warnings as errors, and a C program
    linked against libgdr.so gets the documented results from the calls that
    need no GPU (tests/c_abi/abi_check.c)."""
    import shutil
    import subprocess
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not found")
    here = os.path.dirname(os.path.abspath(__file__))
    root = os.path.dirname(here)
    libdir = os.path.dirname(gdr.LIB_PATH)
    exe = str(tmp_path / "abi_check")
    cmd = [gcc, "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic", "-I", os.path.join(root, "include"),
           os.path.join(here, "c_abi", "abi_check.c"), "-L", libdir, "-lgdr", "-Wl,-rpath," + libdir, "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and r.stdout.strip() == "ok", r.stdout + r.stderr
