"""Benchmark of the 8-bit affine weight-only linear layers on one MI355X.

A step is one Llama-3-8B-shaped decode layer at m = 1, group_size 64, in four
launches: gemv_multi over q [4096,4096], k and v [1024,4096] (one activation,
three weights), gemv on o [4096,4096], gemv_multi over gate and up
[14336,4096], then gemv_silu_gate_resid on down [4096,14336] fed by the gate
and up outputs.  Weights of several layers are cycled so that successive steps
stream different bytes and the 256 MB last-level cache cannot serve them.

value = algorithmic bytes per step (codes + scales + biases of every weight,
plus the activations each launch reads and writes) / measured time per step,
in GB/s, with each layer's launches replayed as a HIP graph.  The roofline
object reports the dominant kernel (the gate+up gemv_multi launch) from HIP
events around a batched, graph-replayed run of that launch alone.  Secondary
lines: the same layer as seven single-weight launches, the quantizer on an
8B gate/up weight, the expert-indexed gemv over 8 experts of that shape (top-2
routing, 1 and 4 tokens), the FP8 E4M3 gemv (per-row and 128 x 128 block
scales) on the 8B FFN shapes, dequantize_to and the gated GEMV of the 70B-shaped
FFN, the small-batch gemm (m = 2..16, and 32 and 64 at group size 64) and the
prefill gemm (m = 512, 2048) in TFLOP/s.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-secondary] [--no-cpu-baseline]
       python bench.py --profile-only     # dominant kernel + calibration copy, for rocprofv3
       python bench.py --profile-prefill  # the m = 2048 prefill gemm alone, for rocprofv3 counters
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

from weight_only_quantized_int8_amd import (Fp8Weight, Int8Weight, binding, gemv_multi, load_library,  # noqa: E402
                                           moe_gemv, synth)

HBM_PEAK_GBS = 8000.0
BF16_MFMA_PEAK_TFLOPS = 2500.0
LLC_BYTES = 256 << 20
METRIC = "int8 GEMV achieved HBM GB/s (% of peak) at m=1; prefill GEMM TFLOP/s"
# the device sources of the gate/up gemv kernel (its traffic record is void
# once either changes)
GEMV_SOURCES = [os.path.join(ROOT, "weight_only_quantized_int8_amd", "csrc", f)
                for f in ("gemv.hip", "common.h")]
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

WEIGHTS = [  # name, N, K
    ("q", 4096, 4096),
    ("k", 1024, 4096),
    ("v", 1024, 4096),
    ("o", 4096, 4096),
    ("gate", 14336, 4096),
    ("up", 14336, 4096),
    ("down", 4096, 14336),
]
SHAPE = {name: (N, K) for name, N, K in WEIGHTS}
GS = 64
# launches of one step: (launch, kind, weights)
FUSED = [
    ("qkv", "multi", ("q", "k", "v")),
    ("o", "gemv", ("o",)),
    ("gate_up", "multi", ("gate", "up")),
    ("down", "silu_gate_resid", ("down",)),
]
UNFUSED = [(n, "gemv", (n,)) for n in ("q", "k", "v", "o", "gate", "up")] + [("down", "silu_gate_resid", ("down",))]
DOMINANT = "gate_up"  # the 2 x 14336 x 4096 launch of each step


def launch_bytes(kind, names):
    """Algorithmic bytes of one launch: every weight once, the activation(s) read once, the outputs written."""
    K = SHAPE[names[0]][1]
    if kind == "silu_gate_resid":
        N = SHAPE[names[0]][0]
        return gated_resid_bytes(N, K, GS)
    return sum(N * K + 4 * N * K // GS + 2 * N for N, _ in (SHAPE[n] for n in names)) + 2 * K


def plan_bytes(plan):
    return sum(launch_bytes(kind, names) for _, kind, names in plan)


class DecodeLayers:
    def __init__(self, dev, n_layers):
        self.dev = dev
        self.layers = []
        for li in range(n_layers):
            d = {}
            for si, (name, N, K) in enumerate(WEIGHTS):
                rng = np.random.Generator(np.random.PCG64(synth.make_seed(1, si) + 7919 * li))
                w = synth.gen_weight(rng, N, K, GS)
                d[name] = Int8Weight.from_arrays(w.packed, w.scales, w.biases, GS, device=dev)
            self.layers.append(d)
        rng = np.random.Generator(np.random.PCG64(synth.make_seed(1, 99)))
        self.x = bits_dev(synth.gen_act(rng, 4096), dev)
        self.x_resid = bits_dev(synth.gen_act(rng, 4096), dev)
        self.out = {name: torch.empty(N, dtype=torch.bfloat16, device=dev) for name, N, _ in WEIGHTS}

    def launch(self, li, kind, names):
        L, o = self.layers[li], self.out
        if kind == "multi":
            gemv_multi([L[n] for n in names], self.x, [o[n] for n in names])
        elif kind == "gemv":
            L[names[0]].gemv(self.x, o[names[0]])
        else:
            L[names[0]].gemv_silu_gate_resid(o["gate"], o["up"], self.x_resid, o[names[0]])

    def step(self, i, plan, timings=None):
        li = i % len(self.layers)
        for name, kind, names in plan:
            if timings is None:
                self.launch(li, kind, names)
            else:
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record()
                self.launch(li, kind, names)
                b.record()
                timings.append((name, a, b))

    def graphs(self, plan):
        """One HIP graph per rotated layer holding that layer's launches."""
        out = []
        for li in range(len(self.layers)):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                self.step(li, plan)
            out.append(g)
        for g in out:
            g.replay()
        torch.cuda.synchronize()
        return out


def time_graph_steps(graphs, steps):
    """Seconds per step over `steps` replays (cycling the layers), HIP events on the replay stream."""
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for i in range(steps):
        graphs[i % len(graphs)].replay()
    end.record()
    torch.cuda.synchronize()
    return start.elapsed_time(end) / 1e3 / steps


def time_batches(fn, iters, reps=5):
    """Seconds per call: `iters` calls (fn(0) .. fn(iters-1), which rotate
    their inputs) captured in one HIP graph after a warm-up, the graph replayed
    `reps` times between two HIP events on the capturing stream; median over
    the replays.  Graph replay keeps host launch cost out of the kernel time."""
    for i in range(min(iters, 3)):
        fn(i)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(iters):
            fn(i)
    g.replay()
    torch.cuda.synchronize()
    times = []
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        g.replay()
        b.record()
        b.synchronize()
        times.append(a.elapsed_time(b) / 1e3 / iters)
    del g
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

    N, K, gs = 14336, 4096, 64  # quantize an 8B gate/up weight (BF16 -> codes, scales, biases)
    rng = np.random.Generator(np.random.PCG64(4200))
    wd = [bits_dev(synth.gen_dense_weight(rng, N, K), dev) for _ in range(copies_for(3 * N * K))]
    packed = torch.empty((N, K // 4), dtype=torch.int32, device=dev)
    sc = torch.empty((N, K // gs), dtype=torch.bfloat16, device=dev)
    bi = torch.empty((N, K // gs), dtype=torch.bfloat16, device=dev)
    def quant(i):  # the current stream at call time (the capturing one inside a graph)
        w_ = wd[i % len(wd)]
        binding.int8_quantize(w_.data_ptr(), N, K, gs, packed.data_ptr(), sc.data_ptr(), bi.data_ptr(),
                              torch.cuda.current_stream().cuda_stream)

    t = time_batches(quant, 10)
    b = 2 * N * K + N * K + 4 * N * K // gs
    res["quantize_14336x4096_gs64"] = {"us": t * 1e6, "GB/s": b / t / 1e9, "frac_hbm": b / t / 1e9 / HBM_PEAK_GBS}
    del wd, packed, sc, bi
    torch.cuda.empty_cache()

    # expert-indexed gemv: 8 experts of the 8B gate/up shape, top-2 routing.
    # One token: consecutive calls name disjoint expert pairs, so every call
    # streams its two experts from HBM.  Four tokens: random routing over two
    # copies of the stacked experts; bytes count each distinct expert once.
    E, N, K, gs = 8, 14336, 4096, 64
    stacks = make_weights(4300, E * N, K, gs, 2, dev)
    rng = np.random.Generator(np.random.PCG64(4301))
    x1 = bits_dev(synth.gen_act(rng, (1, 1, K)), dev)
    y1 = torch.empty((1, 2, N), dtype=torch.bfloat16, device=dev)
    pairs = [torch.tensor([[2 * i, 2 * i + 1]], dtype=torch.int32, device=dev) for i in range(4)]
    t = time_batches(lambda i: moe_gemv(stacks[0], E, x1, pairs[i % 4], y1), 40)
    b = 2 * (N * K + 4 * N * K // gs) + 2 * K + 2 * 2 * N + 4 * 2
    res["moe_gemv_8x14336x4096_gs64_top2_t1"] = {"us": t * 1e6, "GB/s": b / t / 1e9,
                                                 "frac_hbm": b / t / 1e9 / HBM_PEAK_GBS}
    T = 4
    x4 = bits_dev(synth.gen_act(rng, (T, 1, K)), dev)
    y4 = torch.empty((T, 2, N), dtype=torch.bfloat16, device=dev)
    id_sets = [synth.gen_ids(rng, T, 2, E) for _ in range(8)]
    distinct = float(np.mean([len(np.unique(s)) for s in id_sets]))
    ids4 = [torch.from_numpy(s.view(np.int32)).to(dev) for s in id_sets]
    t = time_batches(lambda i: moe_gemv(stacks[i % 2], E, x4, ids4[i % 8], y4), 40)
    b = distinct * (N * K + 4 * N * K // gs) + 2 * T * K + 2 * T * 2 * N + 4 * T * 2
    res["moe_gemv_8x14336x4096_gs64_top2_t4"] = {"us": t * 1e6, "GB/s": b / t / 1e9,
                                                 "frac_hbm": b / t / 1e9 / HBM_PEAK_GBS,
                                                 "distinct_experts": distinct}
    del stacks
    torch.cuda.empty_cache()

    # FP8 E4M3 weight gemv on the 8B gate/up and down shapes, per-row f32 and
    # 128 x 128 block BF16 scales
    for N, K in ((14336, 4096), (4096, 14336)):
        for name, fmt in (("row", binding.FP8_PER_ROW), ("block128_bf16", binding.FP8_BLOCK_BF16)):
            rng = np.random.Generator(np.random.PCG64(4400 + N))
            codes = torch.from_numpy(synth.gen_fp8_codes(rng, N, K)).to(dev)
            if fmt == binding.FP8_PER_ROW:
                sc = torch.from_numpy(synth.gen_fp8_scale(rng, N, bf16=False)).to(dev)
            else:
                sc = bits_dev(synth.gen_fp8_scale(rng, (-(-N // 128), -(-K // 128)), bf16=True), dev)
            ws = [Fp8Weight(codes.clone(), sc.clone(), fmt, 128) for _ in range(copies_for(N * K))]
            x = bits_dev(synth.gen_act(rng, K), dev)
            y = torch.empty(N, dtype=torch.bfloat16, device=dev)
            t = time_batches(lambda i: ws[i % len(ws)].gemv(x, y), 30)
            b = N * K + sc.numel() * sc.element_size() + 2 * K + 2 * N
            res[f"fp8_gemv_{name}_{N}x{K}"] = {"us": t * 1e6, "GB/s": b / t / 1e9,
                                                "frac_hbm": b / t / 1e9 / HBM_PEAK_GBS}
            del ws, codes, sc
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
                for m in (32, 64):  # batched decode: 16-row passes on the 4096-row weight
                    X = bits_dev(synth.gen_act(rng, (m, K)), dev)
                    Y = torch.empty((m, N), dtype=torch.bfloat16, device=dev)
                    t = time_batches(lambda i: ws[i % len(ws)].gemm(X, Y), 20)
                    b = gemm_bytes(N, K, gs, m)
                    res[f"gemm_m{m}_{N}x{K}_gs64"] = {"us": t * 1e6, "GB/s": b / t / 1e9,
                                                      "frac_hbm": b / t / 1e9 / HBM_PEAK_GBS,
                                                      "TFLOP/s": 2.0 * m * N * K / t / 1e12}
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
    """The oracle computing the same step (each weight's product, the gated down projection)."""
    import oracle
    ws = {}
    for si, (name, N, K) in enumerate(WEIGHTS):
        rng = np.random.Generator(np.random.PCG64(synth.make_seed(1, si)))
        ws[name] = synth.gen_weight(rng, N, K, GS)
    rng = np.random.Generator(np.random.PCG64(synth.make_seed(1, 99)))
    x = synth.gen_act(rng, 4096)
    r = synth.gen_act(rng, 4096)
    g = synth.gen_act(rng, 14336)
    u = synth.gen_act(rng, 14336)
    n = 0
    t0 = time.perf_counter()
    while True:
        for name in ("q", "k", "v", "o", "gate", "up"):
            w = ws[name]
            oracle.gemv(w.packed, w.scales, w.biases, GS, x)
        w = ws["down"]
        oracle.gemv_silu_gate_resid(w.packed, w.scales, w.biases, GS, g, u, r)
        n += 1
        el = time.perf_counter() - t0
        if el >= budget_s or n >= 200:
            break
    return {"value": plan_bytes(FUSED) * n / el / 1e9, "unit": "GB/s", "cores": oracle.max_threads(),
            "kind": "oracle",
            "sample": f"{n} decode-layer steps (the same products, shapes and byte count as the GPU step), "
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


def write_traffic_record(fetch_csv, write_csv):
    """Turn two rocprofv3 --pmc counter_collection.csv files of `bench.py
    --profile-only` (FETCH_SIZE, then WRITE_SIZE) into the traffic record:
    median KiB per dispatch of the dominant kernel, scaled by what the same
    counter reads for the 256 MiB calibration copy."""
    import csv
    import statistics

    def per_kernel(path):
        out = {}
        with open(path) as f:
            for row in csv.DictReader(f):
                out.setdefault((row["Kernel_Name"], row["Grid_Size"]), []).append(float(row["Counter_Value"]))
        return out

    f, w = per_kernel(fetch_csv), per_kernel(write_csv)
    dom = [k for k in f if "k_gemv_multi" in k[0]]
    cal = [k for k in f if "copyBuffer" in k[0] and max(f[k]) > 100000]
    if len(dom) != 1 or len(cal) != 1:
        raise SystemExit(f"expected one dominant kernel and one calibration copy, got {dom} / {cal}")
    dom, cal = dom[0], cal[0]
    copy_kib = (256 << 20) / 1024
    ff, wf = copy_kib / statistics.median(f[cal]), copy_kib / statistics.median(w[cal])
    fk, wk = statistics.median(f[dom]), statistics.median(w[dom])
    hbm = fk * 1024 * ff + wk * 1024 * wf
    alg = launch_bytes("multi", ("gate", "up"))
    short = re.search(r"(k_\w+<[^>]*>)", dom[0])
    rec = {"kernel": (short.group(1) if short else dom[0]) + " (gemv_multi: gate+up, 2 x 14336x4096, group_size 64)",
           "kernel_source_sha256": source_sha(GEMV_SOURCES),
           "kernel_sources": [os.path.relpath(p, ROOT) for p in GEMV_SOURCES],
           "dispatches": len(f[dom]),
           "fetch_size_kib_median": fk, "write_size_kib_median": wk,
           "calibration_copy_bytes": 256 << 20,
           "calibration_fetch_size_kib": statistics.median(f[cal]),
           "calibration_write_size_kib": statistics.median(w[cal]),
           "fetch_factor": ff, "write_factor": wf,
           "hbm_bytes_per_launch": round(hbm), "algorithmic_bytes_per_launch": alg,
           "ratio_to_algorithmic": hbm / alg}
    with open(TRAFFIC_FILE, "w") as fo:
        json.dump(rec, fo, indent=1)
    print(json.dumps(rec, indent=1))


# ---------------------------------------------------------------- main

def dominant_graph(dl, passes=16):
    """A HIP graph of `passes` rounds of the dominant launch over every rotated
    layer: back to back, no host launch latency between launches, and the
    per-replay launch cost spread over many launches."""
    kind, names = next((k, n) for nm, k, n in FUSED if nm == DOMINANT)
    for li in range(len(dl.layers)):
        dl.launch(li, kind, names)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(passes):
            for li in range(len(dl.layers)):
                dl.launch(li, kind, names)
    g.replay()
    torch.cuda.synchronize()
    return g, passes * len(dl.layers)


def n_rotated_layers():
    per_layer = sum(N * K for _, N, K in WEIGHTS)
    return max(2, -(-2 * LLC_BYTES // per_layer))


def profile_only(dev, replays=2):
    """For rocprofv3: the dominant launch exactly as timed region 2 runs it
    (graph replays), then a plain 256 MiB device copy that calibrates the
    FETCH_SIZE / WRITE_SIZE counters."""
    dl = DecodeLayers(dev, n_rotated_layers())
    g, per_replay = dominant_graph(dl)
    for _ in range(replays):
        g.replay()
    torch.cuda.synchronize()
    src = torch.empty(256 << 20, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"profile_only": True, "dominant_launches": per_replay * (replays + 1) + per_replay // 16,
                      "calibration_copy_bytes": src.numel()}), flush=True)


def profile_prefill(dev, launches=12):
    """For rocprofv3 counters of the prefill kernel: the m = 2048 gemm on the
    8B gate/up weight [14336, 4096] gs64, launched `launches` times (after a
    warm-up of the same launch) on two rotated weights."""
    N, K, gs, m = 14336, 4096, 64, 2048
    ws = make_weights(2000 + N + gs, N, K, gs, 2, dev)
    rng = np.random.default_rng(N + gs)
    X = bits_dev(synth.gen_act(rng, (m, K)), dev)
    Y = torch.empty((m, N), dtype=torch.bfloat16, device=dev)
    ws[0].gemm(X, Y)
    torch.cuda.synchronize()
    for i in range(launches):
        ws[i % 2].gemm(X, Y)
    torch.cuda.synchronize()
    print(json.dumps({"profile_prefill": True, "m": m, "N": N, "K": K, "launches": launches + 1,
                      "flops_per_launch": 2 * m * N * K}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=300)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--full-secondary", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--profile-only", action="store_true")
    ap.add_argument("--profile-prefill", action="store_true",
                    help="only the m = 2048 prefill gemm, for rocprofv3 counters")
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write the traffic record from two rocprofv3 --pmc runs of --profile-only, then exit")
    args = ap.parse_args()
    if args.traffic_from:
        write_traffic_record(*args.traffic_from)
        return
    if args.gpus != 1:
        print("bench.py measures one GPU: this library has no multi-GPU path (run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    load_library()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.profile_prefill:
        profile_prefill(dev)
        return
    if args.profile_only:
        profile_only(dev)
        return

    n_layers = n_rotated_layers()
    dl = DecodeLayers(dev, n_layers)
    step_bytes = plan_bytes(FUSED)
    print(f"# decode layer: {len(FUSED)} launches, {step_bytes / 1e6:.1f} MB/step, {n_layers} layers rotated",
          file=sys.stderr, flush=True)
    for i in range(args.warmup):
        dl.step(i, FUSED)
    torch.cuda.synchronize()

    # ---- timed region 1: K steps, each layer's launches replayed as one HIP graph
    graphs = dl.graphs(FUSED)
    t0 = time.perf_counter()
    step_s = time_graph_steps(graphs, args.steps)
    wall = time.perf_counter() - t0
    value = step_bytes / step_s / 1e9

    # ---- timed region 2: the dominant launch alone, back to back (see
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
    b_dom = launch_bytes("multi", ("gate", "up"))
    traffic = traffic_record()
    roofline = {"bound": "hbm", "achieved": b_dom / avg_dom / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": b_dom / avg_dom / 1e9 / HBM_PEAK_GBS,
                "traffic": traffic["hbm_bytes_per_launch"] if traffic else None,
                "kernel": "k_gemv_multi: gate+up, 2 x 14336x4096 gs64", "bytes_per_launch": b_dom,
                "avg_launch_us": avg_dom * 1e6, "launches": reps * dom_per_replay}

    # ---- per-launch view (eager launches, HIP events around each; includes
    # host launch latency, reported for reference only)
    timings = []
    for i in range(min(args.steps, 30)):
        dl.step(i, FUSED, timings)
    torch.cuda.synchronize()
    per_call = {}
    for name, a, b in timings:
        per_call.setdefault(name, []).append(a.elapsed_time(b) / 1e3)
    calls = {}
    for name, kind, names in FUSED:
        avg = float(np.mean(per_call[name]))
        b = launch_bytes(kind, names)
        calls[name] = {"weights": list(names), "kind": kind, "bytes": b, "avg_event_us": avg * 1e6,
                       "GB/s": b / avg / 1e9}

    # ---- the same layer as seven single-weight launches (one graph per layer)
    unfused_s = time_graph_steps(dl.graphs(UNFUSED), args.steps)
    unfused = {"launches": len(UNFUSED), "ms_per_step": unfused_s * 1e3,
               "GB/s": plan_bytes(UNFUSED) / unfused_s / 1e9, "bytes_per_step": plan_bytes(UNFUSED)}

    result = {
        "metric": METRIC, "value": value, "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": step_s * 1e3, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": "llama3-8b-shaped decode layer at m=1, group_size=64: gemv_multi(q,k,v), gemv(o), "
                               "gemv_multi(gate,up), gemv_silu_gate_resid(down)",
                   "bytes_per_step": step_bytes, "layers_rotated": n_layers, "frac_hbm_peak": value / HBM_PEAK_GBS,
                   "timing": "HIP graph per layer", "wall_s": wall},
        "roofline": roofline,
        "calls": calls,
        "unfused_step": unfused,
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline()
    if not args.no_secondary:
        del dl, graphs, g_dom
        torch.cuda.empty_cache()
        result["secondary"] = secondary(dev, quick=not args.full_secondary)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
