"""Benchmark of the 8-bit affine weight-only linear layers on one MI355X.

A step is one Llama-3-8B-shaped decode layer at m = 1, group_size 64: the
gemv calls of q [4096,4096], k and v [1024,4096], o [4096,4096], gate and up
[14336,4096], then gemv_silu_gate_resid on down [4096,14336] fed by the gate
and up outputs.  Weights of several layers are cycled so that successive steps
stream different bytes and the 256 MB last-level cache cannot serve them.

value = algorithmic bytes per step (codes + scales + biases + activations in
and out, per call) / measured time per step, in GB/s, with each layer's seven
launches replayed as a HIP graph.  The roofline object reports the dominant
kernel (the gate/up gemv) from HIP events around a batched, graph-replayed
run of that kernel alone.  Secondary lines time dequantize_to and the
gated GEMV of the 70B-shaped FFN, the small-batch gemm (m = 2..16) and the
prefill gemm (m = 512, 2048) in TFLOP/s.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-secondary] [--no-cpu-baseline]
       python bench.py --profile-only     # dominant kernel + calibration copy, for rocprofv3
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

from weight_only_quantized_int8_amd import Int8Weight, load_library, synth  # noqa: E402

HBM_PEAK_GBS = 8000.0
BF16_MFMA_PEAK_TFLOPS = 2500.0
LLC_BYTES = 256 << 20
METRIC = "int8 GEMV achieved HBM GB/s (% of peak) at m=1; prefill GEMM TFLOP/s"
# the sources the gate/up gemv kernel is compiled from (its traffic record is
# void once any of them changes)
GEMV_SOURCES = [os.path.join(ROOT, "weight_only_quantized_int8_amd", "csrc", f)
                for f in ("gemv.hip", "common.h", "launch.h")]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gemv_gate_up_traffic.json")


def gemv_bytes(N, K, gs):
    return N * K + 4 * N * K // gs + 2 * K + 2 * N


def gated_resid_bytes(N, K, gs):
    return N * K + 4 * N * K // gs + 4 * K + 4 * N


def dequant_bytes(N, K, gs):
    return N * K + 4 * N * K // gs + 2 * N * K


def gemm_bytes(N, K, gs, m):
    return N * K + 4 * N * K // gs + 2 * m * K + 2 * m * N


def bits_dev(a, dev):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)


def make_weights(seed, N, K, gs, copies, dev):
    out = []
    for c in range(copies):
        rng = np.random.Generator(np.random.PCG64(seed + 97 * c))
        w = synth.gen_weight(rng, N, K, gs)
        out.append(Int8Weight.from_arrays(w.packed, w.scales, w.biases, gs, device=dev))
    return out


def copies_for(bytes_per_copy):
    return max(2, -(-2 * LLC_BYTES // bytes_per_copy))


def source_sha(paths):
    h = hashlib.sha256()
    for p in paths:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


# ---------------------------------------------------------------- the decode layer (the step)

LAYER = [  # name, N, K, kind
    ("q", 4096, 4096, "gemv"),
    ("k", 1024, 4096, "gemv"),
    ("v", 1024, 4096, "gemv"),
    ("o", 4096, 4096, "gemv"),
    ("gate", 14336, 4096, "gemv"),
    ("up", 14336, 4096, "gemv"),
    ("down", 4096, 14336, "silu_gate_resid"),
]
GS = 64
DOMINANT = ("gate", "up")  # the two 14336 x 4096 gemv launches of each step


def call_bytes(N, K, kind):
    return gemv_bytes(N, K, GS) if kind == "gemv" else gated_resid_bytes(N, K, GS)


def layer_bytes():
    return sum(call_bytes(N, K, kind) for _, N, K, kind in LAYER)


class DecodeLayers:
    def __init__(self, dev, n_layers):
        self.dev = dev
        self.layers = []
        for li in range(n_layers):
            d = {}
            for si, (name, N, K, kind) in enumerate(LAYER):
                rng = np.random.Generator(np.random.PCG64(synth.make_seed(1, si) + 7919 * li))
                w = synth.gen_weight(rng, N, K, GS)
                d[name] = Int8Weight.from_arrays(w.packed, w.scales, w.biases, GS, device=dev)
            self.layers.append(d)
        rng = np.random.Generator(np.random.PCG64(synth.make_seed(1, 99)))
        self.x = bits_dev(synth.gen_act(rng, 4096), dev)
        self.x_resid = bits_dev(synth.gen_act(rng, 4096), dev)
        self.out = {name: torch.empty(N, dtype=torch.bfloat16, device=dev) for name, N, _, _ in LAYER}

    def call(self, li, name, kind):
        L, o = self.layers[li], self.out
        if kind == "gemv":
            L[name].gemv(self.x, o[name])
        else:
            L[name].gemv_silu_gate_resid(o["gate"], o["up"], self.x_resid, o[name])

    def step(self, i, timings=None):
        li = i % len(self.layers)
        for name, _, _, kind in LAYER:
            if timings is None:
                self.call(li, name, kind)
            else:
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record()
                self.call(li, name, kind)
                b.record()
                timings.append((name, a, b))


def time_batches(fn, iters, reps=5):
    """Median over reps of (batch of `iters` calls) / iters, in seconds, via HIP events."""
    times = []
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for i in range(iters):
            fn(i)
        b.record()
        b.synchronize()
        times.append(a.elapsed_time(b) / 1e3 / iters)
    return float(np.median(times))


# ---------------------------------------------------------------- secondary measurements

def secondary(dev, quick):
    res = {}
    N, K, gs = 28672, 8192, 128  # 70B-shaped FFN: dequantize_to of the up/gate weight
    ws = make_weights(4000, N, K, gs, 2, dev)
    outs = [torch.empty((N, K), dtype=torch.bfloat16, device=dev) for _ in range(2)]
    for i in range(3):
        ws[i % 2].dequantize_to(outs[i % 2])
    t = time_batches(lambda i: ws[i % 2].dequantize_to(outs[i % 2]), 10)
    b = dequant_bytes(N, K, gs)
    res["dequantize_to_28672x8192_gs128"] = {"us": t * 1e6, "GB/s": b / t / 1e9, "frac_hbm": b / t / 1e9 / HBM_PEAK_GBS}
    del ws, outs
    torch.cuda.empty_cache()

    N, K, gs = 8192, 28672, 128  # 70B-shaped down projection, gated + residual
    ws = make_weights(4100, N, K, gs, copies_for(N * K), dev)
    rng = np.random.default_rng(5)
    g, u, r = (bits_dev(synth.gen_act(rng, n), dev) for n in (K, K, N))
    y = torch.empty(N, dtype=torch.bfloat16, device=dev)
    t = time_batches(lambda i: ws[i % len(ws)].gemv_silu_gate_resid(g, u, r, y), 30)
    b = gated_resid_bytes(N, K, gs)
    res["gemv_silu_gate_resid_8192x28672_gs128"] = {"us": t * 1e6, "GB/s": b / t / 1e9,
                                                   "frac_hbm": b / t / 1e9 / HBM_PEAK_GBS}
    del ws
    torch.cuda.empty_cache()

    for N, K in ((14336, 4096), (4096, 14336)):  # small-batch decode and prefill gemm
        for gs in ((64,) if quick else (32, 64, 128)):
            ws = make_weights(2000 + N + gs, N, K, gs, copies_for(N * K), dev)
            rng = np.random.default_rng(N + gs)
            for m in (2, 4, 8, 16):
                X = bits_dev(synth.gen_act(rng, (m, K)), dev)
                Y = torch.empty((m, N), dtype=torch.bfloat16, device=dev)
                t = time_batches(lambda i: ws[i % len(ws)].gemm(X, Y), 30)
                b = gemm_bytes(N, K, gs, m)
                res[f"gemm_m{m}_{N}x{K}_gs{gs}"] = {"us": t * 1e6, "GB/s": b / t / 1e9,
                                                    "frac_hbm": b / t / 1e9 / HBM_PEAK_GBS}
            if gs == 64:
                for m in (512, 2048):
                    X = bits_dev(synth.gen_act(rng, (m, K)), dev)
                    Y = torch.empty((m, N), dtype=torch.bfloat16, device=dev)
                    t = time_batches(lambda i: ws[i % len(ws)].gemm(X, Y), 10)
                    fl = 2.0 * m * N * K
                    res[f"gemm_m{m}_{N}x{K}_gs64"] = {"us": t * 1e6, "TFLOP/s": fl / t / 1e12,
                                                      "frac_mfma_bf16": fl / t / 1e12 / BF16_MFMA_PEAK_TFLOPS}
            del ws
            torch.cuda.empty_cache()
    return res


# ---------------------------------------------------------------- CPU oracle baseline

def cpu_baseline(budget_s=12.0):
    import oracle
    layers = []
    for si, (name, N, K, kind) in enumerate(LAYER):
        rng = np.random.Generator(np.random.PCG64(synth.make_seed(1, si)))
        layers.append((synth.gen_weight(rng, N, K, GS), kind))
    rng = np.random.Generator(np.random.PCG64(synth.make_seed(1, 99)))
    x = synth.gen_act(rng, 4096)
    r = synth.gen_act(rng, 4096)
    g = synth.gen_act(rng, 14336)
    u = synth.gen_act(rng, 14336)
    n = 0
    t0 = time.perf_counter()
    while True:
        for w, kind in layers:
            if kind == "gemv":
                oracle.gemv(w.packed, w.scales, w.biases, GS, x)
            else:
                oracle.gemv_silu_gate_resid(w.packed, w.scales, w.biases, GS, g, u, r)
        n += 1
        el = time.perf_counter() - t0
        if el >= budget_s or n >= 200:
            break
    return {"value": layer_bytes() * n / el / 1e9, "unit": "GB/s", "cores": oracle.max_threads(), "kind": "oracle",
            "sample": f"{n} decode-layer steps (the same 7 calls, shapes and byte count as the GPU step), "
                      f"{el:.1f} s"}


def traffic_record():
    """HBM bytes per launch of the dominant kernel from committed rocprofv3 counters, if still current."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    with open(TRAFFIC_FILE) as f:
        rec = json.load(f)
    if rec.get("kernel_source_sha256") != source_sha(GEMV_SOURCES):
        return None  # the kernel changed since the counters were taken
    return rec


# ---------------------------------------------------------------- main

def dominant_graph(dl, passes=16):
    """A HIP graph of `passes` rounds of the gate and up gemv over every rotated
    layer: the dominant kernel launched back to back, with no host launch
    latency between launches and the per-replay launch cost spread over many."""
    for li in range(len(dl.layers)):
        for name in DOMINANT:
            dl.call(li, name, "gemv")
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(passes):
            for li in range(len(dl.layers)):
                for name in DOMINANT:
                    dl.call(li, name, "gemv")
    g.replay()
    torch.cuda.synchronize()
    return g, passes * len(dl.layers) * len(DOMINANT)


def profile_only(dev, replays=2):
    """For rocprofv3: the dominant kernel exactly as timed region 2 runs it
    (graph replays of the gate/up gemv only), then a plain 256 MiB device copy
    that calibrates the FETCH_SIZE / WRITE_SIZE counters."""
    per_layer = sum(N * K for _, N, K, _ in LAYER)
    dl = DecodeLayers(dev, max(2, -(-2 * LLC_BYTES // per_layer)))
    g, per_replay = dominant_graph(dl)
    for _ in range(replays):
        g.replay()
    torch.cuda.synchronize()
    src = torch.empty(256 << 20, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"profile_only": True, "gemv_launches": per_replay * (replays + 1) + per_replay // 16,
                      "calibration_copy_bytes": src.numel()}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=300)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--full-secondary", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--eager", action="store_true", help="time eager launches instead of graph replays")
    ap.add_argument("--profile-only", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: this library has no multi-GPU path (run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    load_library()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.profile_only:
        profile_only(dev)
        return

    per_layer = sum(N * K for _, N, K, _ in LAYER)
    n_layers = max(2, -(-2 * LLC_BYTES // per_layer))
    dl = DecodeLayers(dev, n_layers)
    print(f"# decode layer: {len(LAYER)} calls, {layer_bytes() / 1e6:.1f} MB/step, {n_layers} layers rotated",
          file=sys.stderr, flush=True)
    for i in range(args.warmup):
        dl.step(i)
    torch.cuda.synchronize()

    # one HIP graph per layer: its seven launches, replayed as a unit
    graphs = []
    if not args.eager:
        for li in range(n_layers):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                dl.step(li)
            graphs.append(g)
        for g in graphs:
            g.replay()
        torch.cuda.synchronize()

    # ---- timed region 1: K steps (graph replays, or eager launches)
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record()
    for i in range(args.steps):
        if graphs:
            graphs[i % n_layers].replay()
        else:
            dl.step(i)
    end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    step_s = start.elapsed_time(end) / 1e3 / args.steps
    value = layer_bytes() / step_s / 1e9

    # ---- timed region 2: the dominant kernel alone, back to back (see
    # dominant_graph); HIP events on the launch stream around the replays.
    g_dom, dom_per_replay = dominant_graph(dl)
    reps = max(2, -(-2 * args.steps // dom_per_replay))
    s2, e2 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s2.record()
    for _ in range(reps):
        g_dom.replay()
    e2.record()
    torch.cuda.synchronize()
    avg_dom = s2.elapsed_time(e2) / 1e3 / (reps * dom_per_replay)

    # ---- per-call view (eager launches, HIP events around each; includes
    # host launch latency, reported for reference only)
    timings = []
    for i in range(min(args.steps, 30)):
        dl.step(i, timings)
    torch.cuda.synchronize()
    per_call = {}
    for name, a, b in timings:
        per_call.setdefault(name, []).append(a.elapsed_time(b) / 1e3)
    calls = {}
    for name, N, K, kind in LAYER:
        avg = float(np.mean(per_call[name]))
        b = call_bytes(N, K, kind)
        calls[name] = {"N": N, "K": K, "kind": kind, "avg_event_us": avg * 1e6, "GB/s": b / avg / 1e9}
    b_dom = gemv_bytes(14336, 4096, GS)
    traffic = traffic_record()
    roofline = {"bound": "hbm", "achieved": b_dom / avg_dom / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": b_dom / avg_dom / 1e9 / HBM_PEAK_GBS,
                "traffic": traffic["hbm_bytes_per_launch"] if traffic else None,
                "kernel": "k_gemv, 14336x4096 gs64 (gate/up)", "bytes_per_launch": b_dom,
                "avg_launch_us": avg_dom * 1e6, "launches": reps * dom_per_replay}

    result = {
        "metric": METRIC, "value": value, "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": step_s * 1e3, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": "llama3-8b-shaped decode layer: gemv q,k,v,o,gate,up + gemv_silu_gate_resid down, "
                               "m=1, group_size=64",
                   "bytes_per_step": layer_bytes(), "layers_rotated": n_layers, "frac_hbm_peak": value / HBM_PEAK_GBS,
                   "timing": "eager launches" if args.eager else "HIP graph per layer",
                   "wall_s": wall},
        "roofline": roofline,
        "calls": calls,
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline()
    if not args.no_secondary:
        del dl, graphs
        torch.cuda.empty_cache()
        result["secondary"] = secondary(dev, quick=not args.full_secondary)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
