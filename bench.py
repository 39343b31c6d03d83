"""Benchmark of the gated delta-rule hot path on one MI355X.

One step = one chunked prefill (gdr_chunk_fwd) of the Gated DeltaNet-2 long
prefill: B=1, T=65536, 16 heads, d_k = d_v = 128, bf16 io, fp32 state,
chunk 64, per-channel decay, decoupled erase and write gates. That is the
largest configuration that fits one GPU, and the headline "value" is its
tokens/s. In the same run, each as a sub-object of the one JSON line:
  - "prefill_configs": the same call timed on the Qwen3.8-27B-shaped Gated
    DeltaNet layer (B=1, T=4096, 16 QK / 48 V heads, scalar decay) and the
    KDA layer (B=2, T=16384, 32 heads, per-channel decay);
  - "decode": 256 consecutive gdr_decode_step calls for 64 sequences x 48 V
    heads with 128 x 128 fp32 states (also with four layers' states in turn);
  - "input_stage": the headline prefill from raw projections
    (gdr_chunk_fwd_in: convolution, normalisation, gate activations);
  - "backward": gdr_chunk_bwd and gdr_recurrent_bwd on the headline layer;
  - "recurrent": gdr_recurrent_fwd, a few tokens per sequence at the decode
    shape;
  - "norm_la": normalised linear attention, gdr_norm_la_fwd on a Qwen-like
    layer (B=1, T=4096, 16 QK / 48 V heads, d=128, bf16) and 256
    gdr_norm_la_decode_step calls at the decode shape;
  - "copy": a plain 1 GiB device copy, against which every HBM roofline also
    gives "frac_of_copy";
  - "cpu_baseline": the fp64 CPU oracle on the headline layer (all heads, all
    tokens) on this host's cores.
Inputs are seeded synthetic tensors already resident in device memory when
timing starts, after the warmup steps and a further --warmup-s seconds of
untimed calls (the GPU's clocks take that long to settle). The timed calls
are captured once as a HIP graph (the way a serving loop launches them,
without per-launch host overhead) and timed over one replay with HIP events
on the stream the graph runs on; the JSON also gives the eager per-call time
(events around each call) for reference.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

HBM_PEAK_GBPS = 8000.0        # MI355X HBM3E, published
DECODE_COLD_LAYERS = 4        # states cycled in the decode "layers in turn" timing
BF16_PEAK_TFLOPS = 2500.0     # MI355X dense bf16 matrix, published
FP32_VECTOR_PEAK_TFLOPS = 157.3  # MI355X fp32 vector, published
FP32_MFMA_PEAK_TFLOPS = 157.3    # MI355X dense fp32 matrix cores, published

ROOT = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(ROOT, "gated_delta_rule_23_amd", "csrc")
TRAFFIC_RECORD = os.path.join(ROOT, "profiles", "traffic.json")


# The sources each measured call's kernels are built from (device code, the
# shared device helpers, and the argument and workspace layouts).
SOURCES = {
    "prefill": ("chunk.hip", "common.hpp", "kernels.hpp"),
    "input_stage": ("chunk.hip", "stage.hip", "common.hpp", "kernels.hpp"),
    "decode": ("decode.hip", "common.hpp", "kernels.hpp"),
    "recurrent": ("recurrent.hip", "common.hpp", "kernels.hpp"),
    "backward_chunked": ("chunk_bwd.hip", "common.hpp", "kernels.hpp"),
    "norm_la": ("norm_la.hip", "norm_la.hpp", "common.hpp", "kernels.hpp"),
}


def kernel_source_hash(names):
    """sha256 over the named kernel sources with comments and blank space
    removed, to tell whether recorded memory counters still describe the
    kernels as built."""
    import hashlib
    import re
    h = hashlib.sha256()
    for name in sorted(names):
        with open(os.path.join(CSRC, name)) as f:
            src = f.read()
        src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
        src = re.sub(r"//[^\n]*", " ", src)
        src = " ".join(src.split())
        h.update(name.encode() + b"\0" + src.encode())
    return h.hexdigest()


def recorded_traffic(key, kind):
    """HBM bytes per call measured with rocprofv3 FETCH_SIZE / WRITE_SIZE
    (scaled by a plain copy of known size) for the kernels as they were when
    the counters were taken; None once the sources of that call's kernels
    differ."""
    try:
        with open(TRAFFIC_RECORD) as f:
            rec = json.load(f).get("records", {}).get(key)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("sources_sha256") != kernel_source_hash(SOURCES[kind]):
        return None
    return rec.get("bytes_per_call")


def prefill_algorithmic(wl):
    """Bytes and flops the prefill must move / compute (each input read once,
    each QK head's q, k counted once, outputs and the final state written once;
    chunked-form flops with dense C x C tiles)."""
    esz = 2 if wl.io == "bf16" else 4
    B, T, Hqk, Hv, D = wl.B, wl.T, wl.Hqk, wl.Hv, wl.dk
    by = 2 * B * T * Hqk * D * esz + B * T * Hv * D * esz          # q, k, v
    by += B * T * Hv * 4 if wl.gates == "beta" else 2 * B * T * Hv * D * esz   # beta or b, w
    by += {"none": 0, "scalar": B * T * Hv * 4, "channel": B * T * Hv * D * 4}[wl.decay]
    by += B * T * Hv * D * esz + B * Hv * D * D * 4                # o, S_T
    C = wl.chunk
    flops_per_token_head = 2 * C * (3 * D + 2 * D) + 6 * D * D
    return by, flops_per_token_head * B * T * Hv


def decode_algorithmic(wl):
    esz = 2 if wl.io == "bf16" else 4
    B, Hqk, Hv, D = wl.B, wl.Hqk, wl.Hv, wl.dk
    state = 2 * B * Hv * D * D * 4
    io = 2 * B * Hqk * D * esz + 2 * B * Hv * D * esz + 2 * B * Hv * 4
    return state, state + io


def recurrent_algorithmic(wl):
    """Bytes of one multi-token recurrent call: the state read and written once,
    each token's inputs read once (q, k per QK head) and outputs written once."""
    esz = 2 if wl.io == "bf16" else 4
    B, T, Hqk, Hv, D = wl.B, wl.T, wl.Hqk, wl.Hv, wl.dk
    by = 2 * B * Hv * D * D * 4 + 2 * B * T * Hqk * D * esz + 2 * B * T * Hv * D * esz
    by += B * T * Hv * 4 if wl.gates == "beta" else 2 * B * T * Hv * D * esz
    by += {"none": 0, "scalar": B * T * Hv * 4, "channel": B * T * Hv * D * 4}[wl.decay]
    return by


def backward_algorithmic(wl):
    """Bytes and flops of one backward call (gdr_recurrent_bwd) without S0:
    every input read once (q, k per QK head; dO; dL/dS_T) and every gradient
    written once in float32. Flops: the reverse step's 8 multiply-adds per
    state entry and token (dS += s q do^T, dq, du, dk, de, dSbar, dalpha,
    dS = alpha dSbar); the forward recomputation is not counted."""
    esz = 2 if wl.io == "bf16" else 4
    B, T, Hqk, Hv, D = wl.B, wl.T, wl.Hqk, wl.Hv, wl.dk
    gate = B * T * Hv * 4 if wl.gates == "beta" else 2 * B * T * Hv * D
    dec = {"none": 0, "scalar": B * T * Hv, "channel": B * T * Hv * D}[wl.decay]
    reads = 2 * B * T * Hqk * D * esz + 2 * B * T * Hv * D * esz + B * Hv * D * D * 4
    reads += (gate if wl.gates == "beta" else gate * esz) + dec * 4
    writes = (2 * B * T * Hqk * D + B * T * Hv * D + B * Hv * D * D) * 4 + dec * 4
    writes += B * T * Hv * 4 if wl.gates == "beta" else 2 * B * T * Hv * D * 4
    return reads + writes, 16 * B * T * Hv * D * D


def norm_la_algorithmic(B, T, Hqk, Hv, D, esz=2, C=64):
    """Bytes and flops of one normalised linear-attention prefill: phi(q),
    phi(k) read once per QK head, v read and o written once, the final state
    and normaliser written (and read when given); flops of the chunked form
    on dense C x C tiles: A = Q K^T, Q S, A V and K^T V per (token, V head)."""
    by = 2 * B * T * Hqk * D * esz + 2 * B * T * Hv * D * esz + B * Hv * (D * D + D) * 4
    return by, (2 * C * D + 2 * D * D + 2 * C * D + 2 * D * D) * B * T * Hv


def chunk_backward_flops(wl, C=64):
    """Flops of one gdr_chunk_bwd call, the chunked form's dense products
    counted once (triangular ones at half): per chunk unit 8 C D^2 + 6 C^2 D
    multiply-adds (the factors' products and solve, both sweeps over chunks,
    the gradient products); elementwise work is not counted."""
    D = wl.dk
    units = wl.B * wl.Hv * -(-wl.T // C)
    return 2 * units * (8 * C * D * D + 6 * C * C * D)


def cpu_baseline(wl, inp, heads, min_seconds=10.0, max_reps=200):
    """Time the fp64 oracle (as it stands) on the given V heads of the prefill
    workload, repeating the run until about min_seconds of CPU work."""
    import oracle
    reps, total = 0, 0.0
    while reps < max_reps and (reps == 0 or total < min_seconds):
        t0 = time.perf_counter()
        oracle.recurrent(inp["q"], inp["k"], inp["v"], g=inp["g"], beta=inp["beta"], b=inp["b"], w=inp["w"],
                         scale=wl.scale, S0=inp["S0"], heads=heads)
        total += time.perf_counter() - t0
        reps += 1
    dt = total / reps
    toks = wl.B * wl.T * len(heads) / wl.Hv
    return {"value": toks / dt, "unit": "tokens/s", "cores": oracle.default_threads(), "kind": "oracle",
            "sample": f"fp64 token-by-token oracle on {len(heads)} of {wl.Hv} V heads, all {wl.T} tokens, "
                      f"{reps} runs, {dt:.2f} s per run (tokens/s scaled to the whole layer)"}


PREFILLS = {"gdn2_prefill": "GDN2_PREFILL", "kda_prefill": "KDA_PREFILL", "qwen_gdn_prefill": "QWEN_GDN_PREFILL",
            "gdn_small_f32": "GDN_SMALL_F32"}


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--warmup-s", type=float, default=1.0,
                    help="after the warmup steps, keep running untimed steps for this many seconds so that the "
                         "GPU's clocks have settled before anything is timed")
    ap.add_argument("--decode-steps", type=int, default=256, help="consecutive decode steps timed (0 = skip decode)")
    ap.add_argument("--input-stage", type=int, default=1,
                    help="also time the prefill from raw projections (input stage fused; 0 = skip)")
    ap.add_argument("--norm-la", type=int, default=1,
                    help="also time normalised linear attention: the Qwen-like prefill (T=4096, 16/48 heads, d=128) "
                         "and the decode step at the decode shape (0 = skip)")
    ap.add_argument("--recurrent-T", type=int, default=4,
                    help="tokens per sequence of the multi-token recurrent call timed at the decode shape (0 = skip)")
    ap.add_argument("--backward", type=int, default=1,
                    help="also time gdr_chunk_bwd and gdr_recurrent_bwd on the prefill workload (0 = skip)")
    ap.add_argument("--workload", default="gdn2_prefill", choices=sorted(PREFILLS),
                    help="prefill workload of the timed step (default: the Gated DeltaNet-2 layer, T=65536)")
    ap.add_argument("--sub-prefills", default="qwen_gdn_prefill,kda_prefill",
                    help="comma-separated prefill workloads also timed, each as a sub-object ('' = none)")
    ap.add_argument("--cpu-heads", type=int, default=16, help="V heads in the CPU-oracle sample (0 = skip)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="repeat the CPU-oracle run until this much time has passed (one run at least)")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--copy-mib", type=int, default=1024,
                    help="size of each buffer of the plain device-to-device copy timed in the same run, the "
                         "measured bandwidth the HBM rooflines are also reported against (0 = skip)")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="also run one plain device copy of this many MiB (for scaling memory counters)")
    args = ap.parse_args(argv)
    if args.gpus != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path (the mixer shards over "
              "sequences and heads with no communication); run with --gpus 1", file=sys.stderr)
        return 2

    import numpy as np
    import torch
    import gated_delta_rule_23_amd as gdr
    import gdr_synth as gs

    dev = torch.device("cuda:0")
    t_run = time.perf_counter()

    def progress(msg):
        """One line on stderr per finished section (the JSON line goes to stdout)."""
        print(f"bench: {msg} ({time.perf_counter() - t_run:.0f} s)", file=sys.stderr, flush=True)

    def up(a):
        if a is None:
            return None
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(a).to(dev)

    def settle(fn):
        """Untimed calls of fn for --warmup-s seconds: the GPU's clocks settle under load."""
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < args.warmup_s:
            for _ in range(8):
                fn()
            torch.cuda.synchronize()

    if args.copy_calibration_mib > 0:
        n = args.copy_calibration_mib * 2 ** 20 // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    # ---- measured copy bandwidth: a plain device-to-device copy, read + write bytes ----
    copy = None
    if args.copy_mib > 0:
        n = args.copy_mib * 2 ** 20 // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        settle(lambda: dst.copy_(src))
        c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        reps = 20
        c0.record(torch.cuda.current_stream())
        for _ in range(reps):
            dst.copy_(src)
        c1.record(torch.cuda.current_stream())
        torch.cuda.synchronize()
        copy = {"GBps": 2 * n * 4 * reps / (c0.elapsed_time(c1) * 1e-3) / 1e9, "bytes_per_copy": 2 * n * 4,
                "kind": "torch device-to-device copy of %d MiB (bytes read + written)" % args.copy_mib}
        del src, dst

    cur = torch.cuda.current_stream  # the stream a call is made on (inside a capture: the capture stream)

    def make_desc(w):
        return gdr.make_desc(w.B, w.T, w.Hqk, w.Hv, w.dk, gdr.GDR_BF16 if w.io == "bf16" else gdr.GDR_F32,
                             {"none": gdr.GDR_DECAY_NONE, "scalar": gdr.GDR_DECAY_SCALAR,
                              "channel": gdr.GDR_DECAY_CHANNEL}[w.decay], w.scale)

    # ---- prefill: one gdr_chunk_fwd call per step ----
    def time_prefill(w, inp):
        """Eager per-call time (events around each call), then the timed
        region: the K calls captured once as a HIP graph (as a serving loop
        launches them), replayed untimed for --warmup-s seconds (the GPU
        idles while the graph is captured, and its clocks drop), then timed
        over one replay."""
        d = {n: up(inp[n]) for n in ("q", "k", "v", "g", "beta", "b", "w")}
        io_t = torch.bfloat16 if w.io == "bf16" else torch.float32
        ws = torch.empty(gdr.gdr_chunk_workspace_bytes(make_desc(w)), dtype=torch.uint8, device=dev)
        o = torch.empty((w.B, w.T, w.Hv, w.dv), dtype=io_t, device=dev)
        ST = torch.empty((w.B, w.Hv, w.dk, w.dv), dtype=torch.float32, device=dev)

        def prefill():
            gdr.gdr_chunk_fwd(d["q"], d["k"], d["v"], g=d["g"], beta=d["beta"], b=d["b"], w=d["w"], S0=None,
                              scale=w.scale, o=o, ST=ST, workspace=ws, stream=cur())

        for _ in range(args.warmup):
            prefill()
        torch.cuda.synchronize()
        settle(prefill)
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
        for i in range(args.steps):
            ev[i][0].record(cur())
            prefill()
            ev[i][1].record(cur())
        torch.cuda.synchronize()
        eager_ms = sum(a.elapsed_time(b) for a, b in ev) / args.steps
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for _ in range(args.steps):
                prefill()
        settle(graph.replay)
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0.record(cur())
        graph.replay()
        t1.record(cur())
        torch.cuda.synchronize()
        ms = t0.elapsed_time(t1) / args.steps
        del graph, ws, o, ST
        pbytes, pflops = prefill_algorithmic(w)
        achieved = pbytes / (ms * 1e-3) / 1e9
        kernels = "chunk_prep, [chunk_seg_state, chunk_seg_combine when the sweep is split], chunk_sweep"
        res = {"workload": w.name, "steps": args.steps, "launch": "hip_graph", "ms_per_call": ms,
               "eager_call_ms": eager_ms, "tokens_per_s": w.B * w.T / (ms * 1e-3),
               "roofline": {"kernel": f"gdr_chunk_fwd ({kernels})", "bound": "hbm", "achieved": achieved,
                            "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBPS,
                            "traffic": recorded_traffic(w.name, "prefill"), "algorithmic_bytes": pbytes},
               "mfma": {"algorithmic_tflops": pflops / (ms * 1e-3) / 1e12, "peak": BF16_PEAK_TFLOPS,
                        "frac": pflops / (ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, "algorithmic_flops": pflops}}
        return res, d

    wl = getattr(gs, PREFILLS[args.workload])
    desc = make_desc(wl)
    inp = gs.make_inputs(wl, seed=args.seed)
    progress(f"inputs of {wl.name} drawn")
    head, d = time_prefill(wl, inp)
    progress(f"prefill {wl.name}: {head['ms_per_call']:.4f} ms per call")
    ms_per_step = head["ms_per_call"]
    avg_call_ms = ms_per_step
    tokens = wl.B * wl.T
    pbytes, pflops = prefill_algorithmic(wl)
    t_start, t_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    # ---- the other prefill configurations, each as a sub-object ----
    sub = {}
    for name in [x for x in args.sub_prefills.split(",") if x and x != args.workload]:
        w2 = getattr(gs, PREFILLS[name])
        res, d2 = time_prefill(w2, gs.make_inputs(w2, seed=args.seed))
        sub[w2.name] = res
        del d2
        progress(f"prefill {w2.name}: {res['ms_per_call']:.4f} ms per call")

    # ---- the same layer from raw projections: the input stage in front of the prefill ----
    stage = None
    if args.input_stage:
        raw = gs.make_raw_inputs(wl, seed=args.seed + 3)
        rd = {n: up(raw[n]) for n in ("q", "k", "v", "g", "beta", "b", "w", "conv_w", "conv_in", "decay_scale")}
        conv_out = torch.empty_like(rd["conv_in"])
        ws_in = torch.empty(gdr.gdr_chunk_fwd_in_workspace_bytes(desc), dtype=torch.uint8, device=dev)
        o = torch.empty((wl.B, wl.T, wl.Hv, wl.dv), dtype=torch.bfloat16 if wl.io == "bf16" else torch.float32,
                        device=dev)
        ST = torch.empty((wl.B, wl.Hv, wl.dk, wl.dv), dtype=torch.float32, device=dev)

        def prefill_in():
            gdr.gdr_chunk_fwd_in(rd["q"], rd["k"], rd["v"], rd["conv_w"], conv_in=rd["conv_in"], conv_out=conv_out,
                                 decay_scale=rd["decay_scale"], g=rd["g"], beta=rd["beta"], b=rd["b"], w=rd["w"],
                                 S0=None, scale=wl.scale, o=o, ST=ST, workspace=ws_in, stream=cur())

        for _ in range(args.warmup):
            prefill_in()
        torch.cuda.synchronize()
        settle(prefill_in)
        sgraph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(sgraph):
            for _ in range(args.steps):
                prefill_in()
        settle(sgraph.replay)
        t_start.record(cur())
        sgraph.replay()
        t_end.record(cur())
        torch.cuda.synchronize()
        del sgraph
        s_ms = t_start.elapsed_time(t_end) / args.steps
        s_bytes = pbytes + raw["conv_w"].nbytes + 2 * raw["conv_in"].nbytes + (raw["decay_scale"].nbytes
                                                                               if raw["decay_scale"] is not None else 0)
        fused = wl.decay != "channel"
        stage = {"entry": "gdr_chunk_fwd_in", "ms_per_call": s_ms, "tokens_per_s": tokens / (s_ms * 1e-3),
                 "form": ("fused into the prefill's load stage" if fused else
                          "the convolution and normalisation as a pass of their own (stage_conv) before the prefill, the gate and decay activations in its load stage"),
                 "extra_ms_vs_gdr_chunk_fwd": s_ms - avg_call_ms,
                 "unfused_round_trip_bytes": 2 * (d["q"].nbytes + d["k"].nbytes + d["v"].nbytes) if fused else None,
                 "roofline": {"bound": "hbm", "achieved": s_bytes / (s_ms * 1e-3) / 1e9, "peak": HBM_PEAK_GBPS,
                              "unit": "GB/s", "frac": s_bytes / (s_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS,
                              "traffic": recorded_traffic(wl.name + "_input_stage", "input_stage"),
                              "algorithmic_bytes": s_bytes}}
        del raw, rd, conv_out, ws_in, o, ST
        progress(f"input stage: {s_ms:.4f} ms per call")

    # ---- backward (gradients of the recurrence) on the prefill workload ----
    bwd = None
    if args.backward:
        grads = gs.make_output_grads(wl, seed=args.seed + 3)
        do_d, dST_d = up(grads["do"]), up(grads["dST"])
        bdesc = desc

        def time_backward(fn, ws):
            def call():
                fn(d["q"], d["k"], d["v"], do_d, g=d["g"], beta=d["beta"], b=d["b"], w=d["w"], dST=dST_d,
                   scale=wl.scale, workspace=ws, stream=cur())

            call()
            torch.cuda.synchronize()
            n_b = max(2, min(args.steps, 10))
            bgraph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(bgraph):
                for _ in range(n_b):
                    call()
            settle(bgraph.replay)
            b0, b1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            b0.record(cur())
            bgraph.replay()
            b1.record(cur())
            torch.cuda.synchronize()
            del bgraph
            return b0.elapsed_time(b1) / n_b, n_b

        b_bytes, r_flops = backward_algorithmic(wl)
        c_flops = chunk_backward_flops(wl)
        bws = torch.empty(gdr.gdr_chunk_bwd_workspace_bytes(bdesc), dtype=torch.uint8, device=dev)
        b_ms, n_b = time_backward(gdr.gdr_chunk_bwd, bws)
        del bws
        rws = torch.empty(gdr.gdr_recurrent_bwd_workspace_bytes(bdesc), dtype=torch.uint8, device=dev)
        r_ms, _ = time_backward(gdr.gdr_recurrent_bwd, rws)
        del rws
        bwd = {"entry": "gdr_chunk_bwd", "workload": wl.name, "calls": n_b, "launch": "hip_graph",
               "ms_per_call": b_ms, "tokens_per_s": wl.B * wl.T / (b_ms * 1e-3),
               "roofline": {"kernel": "cb_prep (+ cb_rhs) + cb_sweeps + cb_grad_s + cb_grad_out (+ cb_group_sum)",
                            "bound": "mfma", "dtype": "f32", "achieved": c_flops / (b_ms * 1e-3) / 1e12,
                            "peak": FP32_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                            "frac": c_flops / (b_ms * 1e-3) / 1e12 / FP32_MFMA_PEAK_TFLOPS,
                            "algorithmic_flops": c_flops},
               "hbm": {"achieved": b_bytes / (b_ms * 1e-3) / 1e9, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                       "frac": b_bytes / (b_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, "algorithmic_bytes": b_bytes,
                       "traffic": recorded_traffic(wl.name + "_backward_chunked", "backward_chunked")},
               "recurrent": {"entry": "gdr_recurrent_bwd", "ms_per_call": r_ms,
                             "tokens_per_s": wl.B * wl.T / (r_ms * 1e-3),
                             "roofline": {"kernel": "bwd_ckpt_kernel + bwd_kernel + bwd_reduce_kernel",
                                          "bound": "alu", "achieved": r_flops / (r_ms * 1e-3) / 1e12,
                                          "peak": FP32_VECTOR_PEAK_TFLOPS, "unit": "TFLOP/s",
                                          "frac": r_flops / (r_ms * 1e-3) / 1e12 / FP32_VECTOR_PEAK_TFLOPS,
                                          "algorithmic_flops": r_flops}}}
        del do_d, dST_d
        progress(f"backward: chunked {b_ms:.3f} ms, recurrent {r_ms:.3f} ms per call")

    # ---- decode ----
    dec = None
    if args.decode_steps > 0:
        dwl = gs.QWEN_GDN_DECODE.scaled(T=args.decode_steps,
                                        name=f"qwen_gdn_decode_B64_Hv48_d128_{args.decode_steps}steps")
        dinp = gs.make_inputs(dwl, seed=args.seed + 1)
        dd = {n: up(dinp[n]) for n in ("q", "k", "v", "g", "beta", "b", "w")}
        S0d = up(dinp["S0"])
        S = S0d.clone()
        do = torch.empty((dwl.B, dwl.Hv, dwl.dv), dtype=torch.bfloat16, device=dev)

        def dstep(s):
            pick = lambda t: None if t is None else t[s]
            gdr.gdr_decode_step(pick(dd["q"]), pick(dd["k"]), pick(dd["v"]), S, g=pick(dd["g"]),
                                beta=pick(dd["beta"]), b=pick(dd["b"]), w=pick(dd["w"]), scale=dwl.scale, o=do,
                                stream=cur())

        for s in range(min(8, dwl.T)):
            dstep(s)
        wstep = iter(range(1 << 62))
        settle(lambda: dstep(next(wstep) % dwl.T))
        S.copy_(S0d)
        torch.cuda.synchronize()
        # Reference: events around each eager step.
        dev_ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(dwl.T)]
        for s in range(dwl.T):
            dev_ev[s][0].record(cur())
            dstep(s)
            dev_ev[s][1].record(cur())
        torch.cuda.synchronize()
        d_eager_ms = sum(a.elapsed_time(b) for a, b in dev_ev) / dwl.T
        # Timed: the consecutive steps as one HIP graph replay, from the initial state.
        S.copy_(S0d)
        dgraph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(dgraph):
            for s in range(dwl.T):
                dstep(s)
        settle(dgraph.replay)
        S.copy_(S0d)
        torch.cuda.synchronize()
        d0, d1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        d0.record(cur())
        dgraph.replay()
        d1.record(cur())
        torch.cuda.synchronize()
        del dgraph
        d_step_ms = d0.elapsed_time(d1) / dwl.T
        progress(f"decode: {d_step_ms * 1e3:.1f} us per step")
        # The same steps over the states of LAYERS layers in turn (step s
        # advances layer s % LAYERS), as in a model where every other layer's
        # state passes through the memory-side cache between two steps of one
        # layer: a 201 MB state alone fits the 256 MB cache, so consecutive
        # steps on one state could be served partly from it.
        layers = [S] + [S0d.clone() for _ in range(DECODE_COLD_LAYERS - 1)]

        def dstep_layer(s):
            pick = lambda t: None if t is None else t[s]
            gdr.gdr_decode_step(pick(dd["q"]), pick(dd["k"]), pick(dd["v"]), layers[s % len(layers)],
                                g=pick(dd["g"]), beta=pick(dd["beta"]), b=pick(dd["b"]), w=pick(dd["w"]),
                                scale=dwl.scale, o=do, stream=cur())

        cgraph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(cgraph):
            for s in range(dwl.T):
                dstep_layer(s)
        settle(cgraph.replay)
        d0.record(cur())
        cgraph.replay()
        d1.record(cur())
        torch.cuda.synchronize()
        del cgraph, layers
        d_cold_ms = d0.elapsed_time(d1) / dwl.T
        state_bytes, d_bytes = decode_algorithmic(dwl)
        d_achieved = d_bytes / (d_step_ms * 1e-3) / 1e9
        dec = {"workload": dwl.name, "steps": dwl.T, "launch": "hip_graph", "ms_per_step": d_step_ms,
               "eager_ms_per_step": d_eager_ms,
               "state_GBps": state_bytes / (d_step_ms * 1e-3) / 1e9,
               "tokens_per_s": dwl.B / (d_step_ms * 1e-3),
               "layers_in_turn": {"layers": DECODE_COLD_LAYERS, "ms_per_step": d_cold_ms,
                                  "state_GBps": state_bytes / (d_cold_ms * 1e-3) / 1e9,
                                  "hbm_frac": d_bytes / (d_cold_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS},
               "roofline": {"kernel": "decode_kernel", "bound": "hbm", "achieved": d_achieved,
                            "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": d_achieved / HBM_PEAK_GBPS,
                            "traffic": recorded_traffic(dwl.name, "decode") if dwl.T == 256 else None,
                            "algorithmic_bytes": d_bytes}}

    # ---- normalised linear attention: Qwen-like prefill and the decode step ----
    nla = None
    if args.norm_la:
        NB, NT_, NHqk, NHv, ND = 1, 4096, 16, 48, 128
        nin = gs.make_norm_la_inputs(NB, NT_, NHqk, NHv, ND, io="bf16", seed=args.seed + 5)
        nq, nk, nv = up(nin["phq"]), up(nin["phk"]), up(nin["v"])
        ndesc = gdr.make_desc(NB, NT_, NHqk, NHv, ND, gdr.GDR_BF16, gdr.GDR_DECAY_NONE)
        nws = gdr.gdr_norm_la_workspace_bytes(ndesc)
        nws_t = torch.empty(max(nws, 1), dtype=torch.uint8, device=dev)
        no = torch.empty((NB, NT_, NHv, ND), dtype=torch.bfloat16, device=dev)
        nS = torch.empty((NB, NHv, ND, ND), dtype=torch.float32, device=dev)
        nz = torch.empty((NB, NHv, ND), dtype=torch.float32, device=dev)

        def nla_call():
            gdr.gdr_norm_la_fwd(nq, nk, nv, o=no, ST=nS, zT=nz, workspace=nws_t if nws else None, stream=cur())

        for _ in range(args.warmup):
            nla_call()
        torch.cuda.synchronize()
        settle(nla_call)
        ngraph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(ngraph):
            for _ in range(args.steps):
                nla_call()
        settle(ngraph.replay)
        t_start.record(cur())
        ngraph.replay()
        t_end.record(cur())
        torch.cuda.synchronize()
        del ngraph
        n_ms = t_start.elapsed_time(t_end) / args.steps
        n_bytes, n_flops = norm_la_algorithmic(NB, NT_, NHqk, NHv, ND)
        # Decode: 256 consecutive steps at the decode shape (64 sequences x 48 V heads).
        DB, DS = 64, 256
        din = gs.make_norm_la_inputs(DB, DS, NHqk, NHv, ND, io="bf16", seed=args.seed + 6, state=True)
        dq_, dk_, dv_ = up(din["phq"]), up(din["phk"]), up(din["v"])
        S0n, z0n = up(din["S0"]), up(din["z0"])
        Sn, zn = S0n.clone(), z0n.clone()
        dout = torch.empty((DB, NHv, ND), dtype=torch.bfloat16, device=dev)
        steps_q = [(dq_[:, t].contiguous(), dk_[:, t].contiguous(), dv_[:, t].contiguous()) for t in range(DS)]

        def nla_step(t):
            a_, b_, c_ = steps_q[t]
            gdr.gdr_norm_la_decode_step(a_, b_, c_, Sn, zn, o=dout, stream=cur())

        for t in range(8):
            nla_step(t)
        dgraph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(dgraph):
            for t in range(DS):
                nla_step(t)
        settle(dgraph.replay)
        Sn.copy_(S0n)
        zn.copy_(z0n)
        torch.cuda.synchronize()
        t_start.record(cur())
        dgraph.replay()
        t_end.record(cur())
        torch.cuda.synchronize()
        del dgraph
        nd_ms = t_start.elapsed_time(t_end) / DS
        nd_state = 2 * DB * NHv * (ND * ND + ND) * 4
        nd_bytes = nd_state + 2 * DB * NHqk * ND * 2 + 2 * DB * NHv * ND * 2
        nla = {"prefill": {"entry": "gdr_norm_la_fwd", "workload": "norm_la_prefill_T4096_Hqk16_Hv48_d128",
                           "launch": "hip_graph", "steps": args.steps, "ms_per_call": n_ms,
                           "tokens_per_s": NB * NT_ / (n_ms * 1e-3),
                           "roofline": {"kernel": "nla_chunks (segment sums, nla_scan, segment sweeps)",
                                        "bound": "hbm", "achieved": n_bytes / (n_ms * 1e-3) / 1e9,
                                        "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                                        "frac": n_bytes / (n_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS,
                                        "traffic": recorded_traffic("norm_la_prefill_T4096_Hqk16_Hv48_d128", "norm_la"),
                                        "algorithmic_bytes": n_bytes},
                           "mfma": {"algorithmic_tflops": n_flops / (n_ms * 1e-3) / 1e12, "peak": BF16_PEAK_TFLOPS,
                                    "frac": n_flops / (n_ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS,
                                    "algorithmic_flops": n_flops}},
               "decode": {"entry": "gdr_norm_la_decode_step", "workload": "norm_la_decode_B64_Hv48_d128_256steps",
                          "launch": "hip_graph", "steps": DS, "ms_per_step": nd_ms,
                          "tokens_per_s": DB / (nd_ms * 1e-3), "state_GBps": nd_state / (nd_ms * 1e-3) / 1e9,
                          "roofline": {"kernel": "nla_decode", "bound": "hbm",
                                       "achieved": nd_bytes / (nd_ms * 1e-3) / 1e9, "peak": HBM_PEAK_GBPS,
                                       "unit": "GB/s", "frac": nd_bytes / (nd_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS,
                                       "traffic": recorded_traffic("norm_la_decode_B64_Hv48_d128_256steps", "norm_la"),
                                       "algorithmic_bytes": nd_bytes}}}
        del nin, nq, nk, nv, no, nS, nz, nws_t, din, dq_, dk_, dv_, S0n, z0n, Sn, zn, dout, steps_q
        progress(f"normalised linear attention: prefill {n_ms:.4f} ms, decode {nd_ms * 1e3:.1f} us per step")

    # ---- multi-token recurrent forward (a few tokens per sequence from a live state) ----
    rec = None
    if args.recurrent_T > 0:
        rwl = gs.QWEN_GDN_DECODE.scaled(T=args.recurrent_T, decode=False,
                                        name=f"qwen_gdn_verify_B64_Hv48_d128_T{args.recurrent_T}")
        rinp = gs.make_inputs(rwl, seed=args.seed + 2)
        rd = {n: up(rinp[n]) for n in ("q", "k", "v", "g", "beta", "b", "w")}
        r_states = [up(rinp["S0"]) for _ in range(DECODE_COLD_LAYERS)]
        ro = torch.empty((rwl.B, rwl.T, rwl.Hv, rwl.dv), dtype=torch.bfloat16, device=dev)
        n_calls = 64

        def rcall(i):
            Sl = r_states[i % len(r_states)]
            gdr.gdr_recurrent_fwd(rd["q"], rd["k"], rd["v"], g=rd["g"], beta=rd["beta"], b=rd["b"], w=rd["w"],
                                  S0=Sl, ST=Sl, scale=rwl.scale, o=ro, stream=cur())

        for i in range(len(r_states)):
            rcall(i)
        wcall = iter(range(1 << 62))
        settle(lambda: rcall(next(wcall)))
        for Sl in r_states:
            Sl.copy_(up(rinp["S0"]))
        torch.cuda.synchronize()
        rgraph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(rgraph):
            for i in range(n_calls):
                rcall(i)
        settle(rgraph.replay)
        r0, r1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        r0.record(cur())
        rgraph.replay()
        r1.record(cur())
        torch.cuda.synchronize()
        del rgraph, r_states
        r_ms = r0.elapsed_time(r1) / n_calls
        progress(f"recurrent: {r_ms * 1e3:.1f} us per call")
        r_state, _ = decode_algorithmic(rwl)
        r_bytes = recurrent_algorithmic(rwl)
        rec = {"workload": rwl.name, "calls": n_calls, "layers_in_turn": DECODE_COLD_LAYERS, "launch": "hip_graph",
               "ms_per_call": r_ms, "tokens_per_s": rwl.B * rwl.T / (r_ms * 1e-3),
               "state_GBps": r_state / (r_ms * 1e-3) / 1e9,
               "roofline": {"kernel": "recurrent_kernel", "bound": "hbm",
                            "achieved": r_bytes / (r_ms * 1e-3) / 1e9, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                            "frac": r_bytes / (r_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS,
                            "traffic": recorded_traffic(rwl.name, "recurrent"), "algorithmic_bytes": r_bytes}}

    out = {
        "metric": "prefill tokens/s and decode state GB/s for gated delta rule, % of roofline",
        "value": tokens / (ms_per_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "warmup_s": args.warmup_s,
        "ms_per_step": ms_per_step,
        "eager_ms_per_step": head["eager_call_ms"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.io,
        "data": "synthetic (seeded; q,k L2-normalised N(0,1), v N(0,1), gates and decay per the workload recipe)",
        "config": {"workload": wl.name, "B": wl.B, "T": wl.T, "H_qk": wl.Hqk, "H_v": wl.Hv, "d_k": wl.dk,
                   "d_v": wl.dv, "chunk": wl.chunk, "io": wl.io, "decay": wl.decay, "gates": wl.gates,
                   "state": "fp32", "S0": "zeros", "entry": "gdr_chunk_fwd", "launch": "hip_graph"},
        "roofline": dict(head["roofline"], avg_call_ms=avg_call_ms, eager_call_ms=head["eager_call_ms"]),
        "mfma": head["mfma"],
        "prefill_configs": sub,
        "input_stage": stage,
        "backward": bwd,
        "decode": dec,
        "recurrent": rec,
        "norm_la": nla,
    }
    out["copy"] = copy
    if copy:  # the HBM rooflines also against the bandwidth a plain copy reaches on this GPU
        for r in ([out["roofline"], (stage or {}).get("roofline"), (dec or {}).get("roofline"),
                   (rec or {}).get("roofline")] + [x["roofline"] for x in sub.values()] +
                  [x["roofline"] for x in (nla or {}).values()]):
            if r:
                r["frac_of_copy"] = r["achieved"] / copy["GBps"]
    if args.cpu_heads > 0:
        heads = list(range(0, wl.Hv, max(1, wl.Hv // min(args.cpu_heads, wl.Hv))))[:args.cpu_heads]
        out["cpu_baseline"] = cpu_baseline(wl, inp, heads, min_seconds=args.cpu_seconds)
        progress("cpu baseline done")
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
