"""Benchmark of the 8-bit affine weight-only linear layers on one MI355X.

A step is one Llama-3-8B-shaped decode layer at m = 1, group_size 64, in four
launches: gemv_multi over q [4096,4096], k and v [1024,4096] (one activation,
three weights), gemv on o [4096,4096], gemv_multi over gate and up
[14336,4096], then gemv_silu_gate_resid on down [4096,14336] fed by the gate
and up outputs.  Weights of several layers are cycled so that successive steps
stream different bytes and the 256 MB last-level cache cannot serve them.

value = algorithmic bytes per step (codes + scales + biases of every weight,
plus the activations each launch reads and writes) / time per step, in GB/s:
the steps replayed as HIP graphs of up to 12 consecutive steps (so that the
host's cost of launching a graph does not sit between steps; the launches keep
their stream order), a HIP event after every graph, the median of 20 batches
of consecutive graphs.  The roofline object reports
the dominant kernel (the gate+up gemv_multi launch), the median over graph
replays of that launch alone.  Secondary lines, each the median of 20 graph
replays over rotated weights: every single-launch call of the decode
workloads (gemv on the gate, q/o and k/v shapes, gemv_silu_gate and
gemv_silu_gate_resid on the 8B and 70B down shapes), dequantize_to of the
70B-shaped weight, the own-built streaming read (at the byte counts of the
q/o, gate/up and 70B down weights), copy and expand (the achievable ceilings
beside the nominal 8 TB/s; each streaming line carries its fraction of the
matching ceiling), the quantizer, the expert-indexed gemv, the FP8 gemv, the
small-batch gemm and the prefill gemm in TFLOP/s.
cpu_baseline: the oracle on the host cores, at all cores and at one thread.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-secondary] [--no-cpu-baseline]
       python bench.py --profile NAME   # one launch alone + a calibration copy, for rocprofv3
       python bench.py --traffic-from FETCH.csv WRITE.csv --target NAME   # write profiles/traffic_NAME.json
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

    def graphs(self, plan, per=1):
        """HIP graphs of `per` consecutive steps each (the layers in rotation),
        one per starting layer: graph j runs steps j, j + 1, ..., j + per - 1
        (mod the layer count).  Several steps per graph keep the host's graph
        launch cost off the GPU's critical path; the launches inside keep
        their stream order, so every step still runs after the one before."""
        out = []
        for li in range(len(self.layers)):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for s in range(per):
                    self.step(li + s, plan)
            out.append(g)
        for g in out:
            g.replay()
        torch.cuda.synchronize()
        return out


def steps_per_graph(steps, most=12):
    """The largest count of steps per graph, at most `most`, that divides `steps`."""
    return max(d for d in range(1, most + 1) if steps % d == 0)


def replay_steps(graphs, per, steps, events=None):
    """Exactly `steps` steps as steps / per graph replays, continuing the layer
    rotation from one replay to the next; a HIP event after each replay."""
    for r in range(steps // per):
        graphs[(r * per) % len(graphs)].replay()
        if events is not None:
            events[r + 1].record()


def time_graph_steps(graphs, per, steps):
    """Seconds per step over `steps` steps replayed as graphs of `per` steps, HIP events on the replay stream."""
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    replay_steps(graphs, per, steps)
    end.record()
    torch.cuda.synchronize()
    return start.elapsed_time(end) / 1e3 / steps


def time_batches(fn, iters, reps=20):
    """Seconds per call: `iters` calls (fn(0) .. fn(iters-1), which rotate
    their inputs) captured in one HIP graph after a warm-up, the graph replayed
    `reps` times, a HIP event on the capturing stream after each replay; the
    median over the replays (batches).  Graph replay keeps host launch cost out
    of the kernel time."""
    for i in range(min(iters, 3)):
        fn(i)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(iters):
            fn(i)
    g.replay()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
    ev[0].record()
    for r in range(reps):
        g.replay()
        ev[r + 1].record()
    torch.cuda.synchronize()
    times = [ev[r].elapsed_time(ev[r + 1]) / 1e3 / iters for r in range(reps)]
    del g
    return float(np.median(times))


# ---------------------------------------------------------------- single launches (secondary lines and profiles)
#
# Each target is one call of the library, set up on rotated weights (enough
# copies that the 256 MB last-level cache cannot serve repeats), with its
# algorithmic bytes (or flops) per launch, the kernel that runs it and that
# kernel's device sources (a traffic record is void once they change).

CSRC = os.path.join(ROOT, "weight_only_quantized_int8_amd", "csrc")


def _src(*names):
    return [os.path.join(CSRC, n) for n in names] + [os.path.join(CSRC, "common.h")]


class Target:
    def __init__(self, name, kernel, sources, iters, bytes_=None, flops=None, note=""):
        self.name, self.kernel, self.sources, self.iters = name, kernel, sources, iters
        self.bytes, self.flops, self.note = bytes_, flops, note

    def setup(self, dev):  # -> callable(i) launching call i
        raise NotImplementedError


class GemvTarget(Target):
    def __init__(self, name, N, K, gs, kind, iters=30):
        b = gated_resid_bytes(N, K, gs) if kind == "silu_gate_resid" else \
            gemv_bytes(N, K, gs) + (2 * K if kind == "silu_gate" else 0)
        super().__init__(name, "k_gemv<", _src("gemv.hip"), iters, bytes_=b,
                         note=f"{kind} {N}x{K} gs{gs}")
        self.N, self.K, self.gs, self.kind = N, K, gs, kind

    def setup(self, dev):
        N, K, gs = self.N, self.K, self.gs
        ws = make_weights(5000 + N + K + gs, N, K, gs, copies_for(N * K), dev)
        rng = np.random.default_rng(N + K)
        g, u = bits_dev(synth.gen_act(rng, K), dev), bits_dev(synth.gen_act(rng, K), dev)
        r = bits_dev(synth.gen_act(rng, N), dev)
        y = torch.empty(N, dtype=torch.bfloat16, device=dev)
        if self.kind == "gemv":
            return lambda i: ws[i % len(ws)].gemv(g, y)
        if self.kind == "silu_gate":
            return lambda i: ws[i % len(ws)].gemv_silu_gate(g, u, y)
        return lambda i: ws[i % len(ws)].gemv_silu_gate_resid(g, u, r, y)


class GateUpTarget(Target):
    """The decode step's dominant launch: gemv_multi over gate and up."""

    def __init__(self):
        super().__init__("gate_up", "k_gemv_multi", _src("gemv.hip"), 48,
                         bytes_=launch_bytes("multi", ("gate", "up")), note="gemv_multi 2 x 14336x4096 gs64")

    def setup(self, dev):
        N, K = 14336, 4096
        pairs = [make_weights(5100 + 2 * c, N, K, GS, 1, dev) + make_weights(5101 + 2 * c, N, K, GS, 1, dev)
                 for c in range(copies_for(2 * N * K))]
        x = bits_dev(synth.gen_act(np.random.default_rng(5), K), dev)
        ys = [torch.empty(N, dtype=torch.bfloat16, device=dev) for _ in range(2)]
        return lambda i: gemv_multi(pairs[i % len(pairs)], x, ys)


class DequantTarget(Target):
    def __init__(self, N=28672, K=8192, gs=128):
        super().__init__("dequant", "k_dequant", _src("dequant.hip"), 10, bytes_=dequant_bytes(N, K, gs),
                         note=f"dequantize_to {N}x{K} gs{gs}")
        self.N, self.K, self.gs = N, K, gs

    def setup(self, dev):
        N, K, gs = self.N, self.K, self.gs
        ws = make_weights(4000, N, K, gs, 2, dev)
        outs = [torch.empty((N, K), dtype=torch.bfloat16, device=dev) for _ in range(2)]
        return lambda i: ws[i % 2].dequantize_to(outs[i % 2])


class QuantizeTarget(Target):
    """int8_quantize of an 8B gate/up-shaped BF16 weight (codes, scales, biases)."""

    def __init__(self, N=14336, K=4096, gs=64):
        super().__init__("quantize", "k_quantize", _src("quantize.hip"), 10,
                         bytes_=2 * N * K + N * K + 4 * N * K // gs, note=f"quantize {N}x{K} gs{gs}")
        self.N, self.K, self.gs = N, K, gs

    def setup(self, dev):
        N, K, gs = self.N, self.K, self.gs
        rng = np.random.Generator(np.random.PCG64(4200))
        wd = [bits_dev(synth.gen_dense_weight(rng, N, K), dev) for _ in range(copies_for(3 * N * K))]
        packed = torch.empty((N, K // 4), dtype=torch.int32, device=dev)
        sc = torch.empty((N, K // gs), dtype=torch.bfloat16, device=dev)
        bi = torch.empty((N, K // gs), dtype=torch.bfloat16, device=dev)

        def quant(i):  # the current stream at call time (the capturing one inside a graph)
            w_ = wd[i % len(wd)]
            binding.int8_quantize(w_.data_ptr(), N, K, gs, packed.data_ptr(), sc.data_ptr(), bi.data_ptr(),
                                  torch.cuda.current_stream().cuda_stream)
        return quant


class GemmTarget(Target):
    def __init__(self, name, m, N, K, gs, kernel, iters, source=None):
        fl = 2 * m * N * K
        source = source or ("gemm_prefill.hip" if m > 16 else "gemm_smallm.hip")
        super().__init__(name, kernel, _src(source), iters,
                         bytes_=gemm_bytes(N, K, gs, m), flops=fl, note=f"gemm m={m} {N}x{K} gs{gs}")
        self.m, self.N, self.K, self.gs = m, N, K, gs

    def setup(self, dev):
        m, N, K, gs = self.m, self.N, self.K, self.gs
        ws = make_weights(2000 + N + gs, N, K, gs, copies_for(N * K) if m <= 128 else 2, dev)
        X = bits_dev(synth.gen_act(np.random.default_rng(N + gs + m), (m, K)), dev)
        Y = torch.empty((m, N), dtype=torch.bfloat16, device=dev)
        return lambda i: ws[i % len(ws)].gemm(X, Y)


class StreamReadTarget(Target):
    """The own-built streaming read over as many bytes as one weight's codes
    (by default the 8B gate/up weight's)."""

    def __init__(self, name="stream_read", nbytes=14336 * 4096):
        super().__init__(name, "k_stream_read", _src("measure.hip"), 30, bytes_=nbytes,
                         note=f"plain streaming read of {nbytes} bytes")
        self.n = nbytes

    def setup(self, dev):
        bufs = [torch.empty(self.n, dtype=torch.uint8, device=dev) for _ in range(copies_for(self.n))]
        for b in bufs:
            b.fill_(1)
        sink = torch.zeros(4, dtype=torch.int32, device=dev)
        return lambda i: binding.int8w_stream_read(bufs[i % len(bufs)].data_ptr(), self.n, sink.data_ptr(),
                                                   torch.cuda.current_stream().cuda_stream)


class StreamCopyTarget(Target):
    def __init__(self, nbytes=256 << 20):
        super().__init__("stream_copy", "k_stream_copy", _src("measure.hip"), 10, bytes_=2 * nbytes,
                         note=f"plain streaming copy of {nbytes} bytes (read + write)")
        self.n = nbytes

    def setup(self, dev):
        src = [torch.ones(self.n, dtype=torch.uint8, device=dev) for _ in range(2)]
        dst = [torch.empty(self.n, dtype=torch.uint8, device=dev) for _ in range(2)]
        return lambda i: binding.int8w_stream_copy(src[i % 2].data_ptr(), dst[i % 2].data_ptr(), self.n,
                                                   torch.cuda.current_stream().cuda_stream)


class StreamExpandTarget(Target):
    """The own-built streaming expand: every byte widened to 16 bits (one byte
    read, two written: dequantize_to's mix)."""

    def __init__(self, nbytes=128 << 20):
        super().__init__("stream_expand", "k_stream_expand", _src("measure.hip"), 10, bytes_=3 * nbytes,
                         note=f"plain streaming expand of {nbytes} bytes to {2 * nbytes} (read + 2 x write)")
        self.n = nbytes

    def setup(self, dev):
        src = [torch.ones(self.n, dtype=torch.uint8, device=dev) for _ in range(copies_for(self.n))]
        dst = [torch.empty(2 * self.n, dtype=torch.uint8, device=dev) for _ in range(2)]
        return lambda i: binding.int8w_stream_expand(src[i % len(src)].data_ptr(), dst[i % 2].data_ptr(), self.n,
                                                     torch.cuda.current_stream().cuda_stream)


class Fp8Target(Target):
    """FP8 E4M3 gemv with 128 x 128 BF16 block scales (the Fp8Weight page)."""

    def __init__(self, name, N, K, iters=30):
        nb = (-(-N // 128)) * (-(-K // 128))
        super().__init__(name, "k_fp8_gemv", _src("fp8_gemv.hip"), iters, bytes_=N * K + 2 * nb + 2 * K + 2 * N,
                         note=f"fp8 gemv {N}x{K} 128x128 BF16 block scales")
        self.N, self.K = N, K

    def setup(self, dev):
        N, K = self.N, self.K
        rng = np.random.Generator(np.random.PCG64(4400 + N))
        codes = torch.from_numpy(synth.gen_fp8_codes(rng, N, K)).to(dev)
        sc = bits_dev(synth.gen_fp8_scale(rng, (-(-N // 128), -(-K // 128)), bf16=True), dev)
        ws = [Fp8Weight(codes.clone(), sc.clone(), binding.FP8_BLOCK_BF16, 128) for _ in range(copies_for(N * K))]
        x = bits_dev(synth.gen_act(rng, K), dev)
        y = torch.empty(N, dtype=torch.bfloat16, device=dev)
        return lambda i: ws[i % len(ws)].gemv(x, y)


TARGETS = {t.name: t for t in [
    GateUpTarget(),
    GemvTarget("gate", 14336, 4096, 64, "gemv"),
    GemvTarget("qo", 4096, 4096, 64, "gemv"),
    GemvTarget("kv", 1024, 4096, 64, "gemv"),
    GemvTarget("silu_gate", 4096, 14336, 64, "silu_gate"),
    GemvTarget("down", 4096, 14336, 64, "silu_gate_resid"),
    GemvTarget("down70b", 8192, 28672, 128, "silu_gate_resid"),
    DequantTarget(),
    QuantizeTarget(),
    Fp8Target("fp8_block_4096x14336", 4096, 14336),
    GemmTarget("rows2_70b", 2, 8192, 28672, 128, "k_gemv_rows_lds", 30, source="gemv.hip"),
    GemmTarget("smallm16", 16, 4096, 14336, 64, "k_gemm_smallm", 30),
    GemmTarget("prefill512", 512, 4096, 14336, 64, "k_gemm_prefill", 10),
    GemmTarget("prefill2048", 2048, 14336, 4096, 64, "k_gemm_prefill", 10),
    StreamReadTarget(),
    StreamReadTarget("stream_read_q", 4096 * 4096),
    StreamReadTarget("stream_read_70b", 8192 * 28672),
    StreamCopyTarget(),
    StreamExpandTarget(),
]}

# the own-built ceiling each streaming line is compared with: a plain read of
# about the same byte count for the gemv lines, the expand for dequantize_to
CEILING_OF = {"gate": "stream_read", "silu_gate": "stream_read", "down": "stream_read", "qo": "stream_read_q",
              "kv": "stream_read_q", "down70b": "stream_read_70b", "dequant": "stream_expand"}


def traffic_file(name):
    return os.path.join(ROOT, "profiles", f"traffic_{name}.json")


def traffic_record(name):
    """HBM bytes per launch of a target from committed rocprofv3 counters, if still current."""
    path = traffic_file(name)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_source_sha256") != source_sha(TARGETS[name].sources):
        return None  # the kernel changed since the counters were taken
    return rec


def measure_target(t, dev):
    fn = t.setup(dev)
    s = time_batches(fn, t.iters)
    out = {"us": s * 1e6, "call": t.note}
    if t.bytes is not None:
        out["GB/s"] = t.bytes / s / 1e9
        out["frac_hbm"] = t.bytes / s / 1e9 / HBM_PEAK_GBS
    if t.flops is not None:
        out["TFLOP/s"] = t.flops / s / 1e12
        out["frac_mfma_bf16"] = t.flops / s / 1e12 / BF16_MFMA_PEAK_TFLOPS
    rec = traffic_record(t.name)
    if rec:
        out["hbm_traffic_ratio"] = rec["ratio_to_algorithmic"]
    del fn
    torch.cuda.empty_cache()
    return out


# ---------------------------------------------------------------- secondary measurements

def secondary(dev, quick):
    res = {}
    # the single-launch calls of the decode workloads, the calibration streams,
    # dequantize_to of the 70B-shaped weight, and the profiled gemm shapes
    for name in ("gate", "qo", "kv", "silu_gate", "down", "down70b", "dequant", "stream_read", "stream_read_q",
                 "stream_read_70b", "stream_copy", "stream_expand"):
        t = TARGETS[name]
        res[name] = measure_target(t, dev)
        print(f"# {name}: {res[name]['us']:.2f} us", file=sys.stderr, flush=True)
    for name, ceil in CEILING_OF.items():
        res[name]["ceiling"] = ceil
        res[name]["frac_of_ceiling"] = res[name]["GB/s"] / res[ceil]["GB/s"]

    # quantize an 8B gate/up weight (BF16 -> codes, scales, biases); its own-built
    # ceiling is the copy (it reads two bytes for each one it writes)
    q = measure_target(TARGETS["quantize"], dev)
    q["ceiling"] = "stream_copy"
    q["frac_of_ceiling"] = q["GB/s"] / res["stream_copy"]["GB/s"]
    res["quantize_14336x4096_gs64"] = q

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
                for m in (32, 64):  # batched decode: 32-row passes on the 4096-row weight
                    X = bits_dev(synth.gen_act(rng, (m, K)), dev)
                    Y = torch.empty((m, N), dtype=torch.bfloat16, device=dev)
                    t = time_batches(lambda i: ws[i % len(ws)].gemm(X, Y), 20)
                    b = gemm_bytes(N, K, gs, m)
                    res[f"gemm_m{m}_{N}x{K}_gs64"] = {"us": t * 1e6, "GB/s": b / t / 1e9,
                                                      "frac_hbm": b / t / 1e9 / HBM_PEAK_GBS,
                                                      "TFLOP/s": 2.0 * m * N * K / t / 1e12}
                # the library's dense BF16 GEMM (torch.matmul, hipBLASLt) on the
                # same activations and the dequantized weight: a practical
                # ceiling for the matrix cores under this load, measured
                # beside the fused kernel (it reads 2 bytes per weight and
                # does no dequantization)
                wdq = [torch.empty((N, K), dtype=torch.bfloat16, device=dev) for _ in range(2)]
                for j in range(2):
                    ws[j].dequantize_to(wdq[j])
                for m in (512, 2048):
                    X = bits_dev(synth.gen_act(rng, (m, K)), dev)
                    Y = torch.empty((m, N), dtype=torch.bfloat16, device=dev)
                    t = time_batches(lambda i: ws[i % len(ws)].gemm(X, Y), 10)
                    tl = time_batches(lambda i: torch.matmul(X, wdq[i % 2].t(), out=Y), 10)
                    fl = 2.0 * m * N * K
                    res[f"gemm_m{m}_{N}x{K}_gs64"] = {"us": t * 1e6, "TFLOP/s": fl / t / 1e12,
                                                      "frac_mfma_bf16": fl / t / 1e12 / BF16_MFMA_PEAK_TFLOPS,
                                                      "library_bf16_us": tl * 1e6,
                                                      "library_bf16_TFLOP/s": fl / tl / 1e12,
                                                      "frac_of_library_bf16": tl / t}
                del wdq
            del ws
            torch.cuda.empty_cache()
    # two rows on long in_features where X's rows are kept in LDS (group size
    # 32 at 14336, and the 70B-shaped down projection)
    for N, K, gs in ((4096, 14336, 32), (8192, 28672, 128)):
        ws = make_weights(2200 + N + gs, N, K, gs, copies_for(N * K), dev)
        X = bits_dev(synth.gen_act(np.random.default_rng(2201 + N), (2, K)), dev)
        Y = torch.empty((2, N), dtype=torch.bfloat16, device=dev)
        t = time_batches(lambda i: ws[i % len(ws)].gemm(X, Y), 30)
        b = gemm_bytes(N, K, gs, 2)
        res[f"gemm_m2_{N}x{K}_gs{gs}"] = {"us": t * 1e6, "GB/s": b / t / 1e9, "frac_hbm": b / t / 1e9 / HBM_PEAK_GBS}
        del ws
        torch.cuda.empty_cache()
    # a weight whose one round of 256 x 128 tiles walks all of K: m = 32 goes
    # through one 32-row small-m pass
    N, K, gs, m = 18944, 3584, 64, 32
    ws = make_weights(2100, N, K, gs, copies_for(N * K), dev)
    X = bits_dev(synth.gen_act(np.random.default_rng(2101), (m, K)), dev)
    Y = torch.empty((m, N), dtype=torch.bfloat16, device=dev)
    t = time_batches(lambda i: ws[i % len(ws)].gemm(X, Y), 20)
    b = gemm_bytes(N, K, gs, m)
    res[f"gemm_m{m}_{N}x{K}_gs64"] = {"us": t * 1e6, "GB/s": b / t / 1e9, "frac_hbm": b / t / 1e9 / HBM_PEAK_GBS,
                                      "TFLOP/s": 2.0 * m * N * K / t / 1e12}
    del ws
    torch.cuda.empty_cache()
    return res


# ---------------------------------------------------------------- CPU oracle baseline

def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _decode_step_rate(budget_s, max_steps):
    """The oracle computing the decode step (each weight's product, the gated
    down projection) repeatedly for about budget_s seconds: (GB/s, steps, s)."""
    import oracle
    ws = {}
    for si, (name, N, K) in enumerate(WEIGHTS):
        rng = np.random.Generator(np.random.PCG64(synth.make_seed(1, si)))
        ws[name] = synth.gen_weight(rng, N, K, GS)
    rng = np.random.Generator(np.random.PCG64(synth.make_seed(1, 99)))
    x, r = synth.gen_act(rng, 4096), synth.gen_act(rng, 4096)
    g, u = synth.gen_act(rng, 14336), synth.gen_act(rng, 14336)
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
        if el >= budget_s or n >= max_steps:
            break
    return plan_bytes(FUSED) * n / el / 1e9, n, el


def cpu_baseline():
    """The oracle, as it is, on the host cores: the decode step at all cores
    (the reported value) and at one thread, then bounded samples of the
    prefill gemm and of the 70B-shaped dequantize_to at all cores."""
    import oracle
    cores = oracle.max_threads()
    v, n, el = _decode_step_rate(8.0, 200)
    out = {"value": v, "unit": "GB/s", "cores": cores, "kind": "oracle",
           "sample": f"{n} decode-layer steps (the same products, shapes and byte count as the GPU step), "
                     f"{el:.1f} s on {cores} threads",
           "cpu_model": cpu_model()}
    oracle.set_threads(1)
    try:
        v1, n1, el1 = _decode_step_rate(5.0, 50)
    finally:
        oracle.set_threads(cores)
    out["one_thread"] = {"value": v1, "unit": "GB/s", "cores": 1,
                         "sample": f"{n1} decode-layer steps, {el1:.1f} s"}
    # prefill: 128 rows of the m = 512 workload on the 8B gate/up weight
    rng = np.random.Generator(np.random.PCG64(7100))
    w = synth.gen_weight(rng, 14336, 4096, GS)
    X = synth.gen_act(rng, (128, 4096))
    t0 = time.perf_counter()
    oracle.gemm(w.packed, w.scales, w.biases, GS, X)
    el = time.perf_counter() - t0
    out["prefill_gemm"] = {"value": 2.0 * 128 * 14336 * 4096 / el / 1e9, "unit": "GFLOP/s", "cores": cores,
                           "sample": f"gemm on 128 rows of X against the 14336x4096 gs64 weight, {el:.1f} s"}
    # dequantize_to: 8192 rows of the 28672 x 8192 gs128 weight, three times
    w = synth.gen_weight(rng, 8192, 8192, 128)
    t0 = time.perf_counter()
    for _ in range(3):
        oracle.dequantize_to(w.packed, w.scales, w.biases, 128)
    el = time.perf_counter() - t0
    out["dequantize_to"] = {"value": 3 * dequant_bytes(8192, 8192, 128) / el / 1e9, "unit": "GB/s", "cores": cores,
                            "sample": f"dequantize_to of 8192 rows of the 28672x8192 gs128 weight, 3 times, "
                                      f"{el:.2f} s"}
    return out


def write_traffic_record(name, fetch_csv, write_csv):
    """Turn two rocprofv3 --pmc counter_collection.csv files of `bench.py
    --profile NAME` (FETCH_SIZE, then WRITE_SIZE) into the target's traffic
    record: median KiB per dispatch of its kernel, scaled by what the same
    counter reads for the 256 MiB calibration copy."""
    import csv
    import statistics

    t = TARGETS[name]

    def per_kernel(path):
        out = {}
        with open(path) as f:
            for row in csv.DictReader(f):
                out.setdefault((row["Kernel_Name"], row["Grid_Size"]), []).append(float(row["Counter_Value"]))
        return out

    f, w = per_kernel(fetch_csv), per_kernel(write_csv)
    dom = [k for k in f if t.kernel in k[0]]
    cal = [k for k in f if "copyBuffer" in k[0] and max(f[k]) > 100000]
    if len(dom) != 1 or len(cal) != 1:
        raise SystemExit(f"expected one {t.kernel} kernel and one calibration copy, got {dom} / {cal}")
    dom, cal = dom[0], cal[0]
    copy_kib = (256 << 20) / 1024
    # the calibration copies' own dispatches: other copies of the run (a
    # target's rotated buffers) can share the copy kernel and its grid size,
    # and move far fewer bytes (a 256 MiB copy reads about 128 MiB and writes
    # 256 MiB in the counters' units)
    fcal = [v for v in f[cal] if v > 0.35 * copy_kib]
    wcal = [v for v in w.get(cal, []) if v > 0.7 * copy_kib]
    if not fcal or not wcal:
        raise SystemExit("no calibration copy dispatch in the counter files")
    ff, wf = copy_kib / statistics.median(fcal), copy_kib / statistics.median(wcal)
    fk, wk = statistics.median(f[dom]), statistics.median(w[dom])
    hbm = fk * 1024 * ff + wk * 1024 * wf
    short = re.search(r"(k_\w+<[^>]*>|k_\w+)", dom[0])
    rec = {"kernel": (short.group(1) if short else dom[0]) + f" ({t.note})",
           "kernel_source_sha256": source_sha(t.sources),
           "kernel_sources": [os.path.relpath(p, ROOT) for p in t.sources],
           "dispatches": len(f[dom]),
           "fetch_size_kib_median": fk, "write_size_kib_median": wk,
           "calibration_copy_bytes": 256 << 20,
           "calibration_fetch_size_kib": statistics.median(fcal),
           "calibration_write_size_kib": statistics.median(wcal),
           "fetch_factor": ff, "write_factor": wf,
           "hbm_bytes_per_launch": round(hbm), "algorithmic_bytes_per_launch": t.bytes,
           "ratio_to_algorithmic": hbm / t.bytes}
    with open(traffic_file(name), "w") as fo:
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


def calibration_copy(dev):
    """Five plain 256 MiB device copies: what FETCH_SIZE / WRITE_SIZE read for
    a known byte count scales the counters of the profiled kernel."""
    src = torch.empty(256 << 20, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    return src.numel()


def profile_target(dev, name, replays=3):
    """For rocprofv3: one target's launch alone, as bench.py times it (a HIP
    graph of its rotated calls, replayed), then the calibration copy."""
    t = TARGETS[name]
    if name == "gate_up":  # exactly the roofline measurement's graph
        dl = DecodeLayers(dev, n_rotated_layers())
        g, per_replay = dominant_graph(dl)
    else:
        fn = t.setup(dev)
        for i in range(min(t.iters, 3)):
            fn(i)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(t.iters):
                fn(i)
        g.replay()
        per_replay = t.iters
    for _ in range(replays):
        g.replay()
    torch.cuda.synchronize()
    nb = calibration_copy(dev)
    print(json.dumps({"profile": name, "kernel": t.kernel, "call": t.note, "launches_timed": per_replay * replays,
                      "algorithmic_bytes": t.bytes, "flops": t.flops, "calibration_copy_bytes": nb}), flush=True)


def batch_medians(events, steps_per_event, n_batches):
    """Seconds per step: the events bracket consecutive steps; they are split
    into n_batches consecutive batches, and the median over the batches is
    returned with the mean over all of them."""
    per = [events[i].elapsed_time(events[i + 1]) / 1e3 for i in range(len(events) - 1)]
    nb = max(1, min(n_batches, len(per)))
    bounds = np.linspace(0, len(per), nb + 1).round().astype(int)
    b = [sum(per[bounds[j]:bounds[j + 1]]) / ((bounds[j + 1] - bounds[j]) * steps_per_event) for j in range(nb)]
    return float(np.median(b)), sum(per) / (len(per) * steps_per_event), nb


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=300)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--full-secondary", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--profile", choices=sorted(TARGETS), help="one launch alone, for rocprofv3")
    ap.add_argument("--profile-only", action="store_true", help="same as --profile gate_up")
    ap.add_argument("--profile-prefill", action="store_true", help="same as --profile prefill2048")
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write profiles/traffic_<target>.json from two rocprofv3 --pmc runs of --profile, then exit")
    ap.add_argument("--target", default="gate_up", choices=sorted(TARGETS), help="the target of --traffic-from")
    args = ap.parse_args()
    if args.traffic_from:
        write_traffic_record(args.target, *args.traffic_from)
        return
    if args.gpus != 1:
        print("bench.py measures one GPU: this library has no multi-GPU path (run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    load_library()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    prof = args.profile or ("gate_up" if args.profile_only else "prefill2048" if args.profile_prefill else None)
    if prof:
        profile_target(dev, prof)
        return

    n_layers = n_rotated_layers()
    dl = DecodeLayers(dev, n_layers)
    step_bytes = plan_bytes(FUSED)
    print(f"# decode layer: {len(FUSED)} launches, {step_bytes / 1e6:.1f} MB/step, {n_layers} layers rotated",
          file=sys.stderr, flush=True)
    for i in range(args.warmup):
        dl.step(i, FUSED)
    torch.cuda.synchronize()

    # ---- timed region 1: exactly K steps, replayed as HIP graphs of `per`
    # consecutive steps (per divides K); a HIP event after every replay, the
    # replays split into (up to) 20 consecutive batches, value from the median
    # batch
    per = steps_per_graph(args.steps)
    graphs = dl.graphs(FUSED, per)
    n_rep = args.steps // per
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(n_rep + 1)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev[0].record()
    replay_steps(graphs, per, args.steps, ev)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    step_s, step_mean_s, n_batches = batch_medians(ev, per, 20)
    value = step_bytes / step_s / 1e9
    # the same steps with one graph per step: the host's graph launch cost
    # then sits between consecutive steps (reported for reference)
    one_per_graph_s = time_graph_steps(dl.graphs(FUSED, 1), 1, args.steps)

    # ---- timed region 2: the dominant launch alone, back to back (see
    # dominant_graph); a HIP event on the launch stream after every replay,
    # median over at least 20 replays
    g_dom, dom_per_replay = dominant_graph(dl)
    reps = max(20, -(-2 * args.steps // dom_per_replay))
    ev2 = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
    ev2[0].record()
    for r in range(reps):
        g_dom.replay()
        ev2[r + 1].record()
    torch.cuda.synchronize()
    avg_dom, mean_dom, _ = batch_medians(ev2, dom_per_replay, reps)
    b_dom = launch_bytes("multi", ("gate", "up"))
    traffic = traffic_record("gate_up")
    roofline = {"bound": "hbm", "achieved": b_dom / avg_dom / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": b_dom / avg_dom / 1e9 / HBM_PEAK_GBS,
                "traffic": traffic["hbm_bytes_per_launch"] if traffic else None,
                "kernel": "k_gemv_multi: the step's gate+up launch (int8_gemv_multi), 2 x 14336x4096 gs64",
                "bytes_per_launch": b_dom, "avg_launch_us": avg_dom * 1e6, "mean_launch_us": mean_dom * 1e6,
                "launches": reps * dom_per_replay, "batches": reps,
                "timing": "median over graph replays of 48 launches, HIP events on the launch stream"}

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
        calls[name] = {"weights": list(names), "kind": kind, "bytes": b, "avg_eager_event_us": avg * 1e6,
                       "GB/s": b / avg / 1e9}

    # ---- the same layer as seven single-weight launches (graphs of `per` steps)
    unfused_s = time_graph_steps(dl.graphs(UNFUSED, per), per, args.steps)
    unfused = {"launches": len(UNFUSED), "ms_per_step": unfused_s * 1e3,
               "GB/s": plan_bytes(UNFUSED) / unfused_s / 1e9, "bytes_per_step": plan_bytes(UNFUSED)}

    result = {
        "metric": METRIC, "value": value, "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": step_s * 1e3, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": "llama3-8b-shaped decode layer at m=1, group_size=64: gemv_multi(q,k,v), gemv(o), "
                               "gemv_multi(gate,up), gemv_silu_gate_resid(down)",
                   "bytes_per_step": step_bytes, "layers_rotated": n_layers, "frac_hbm_peak": value / HBM_PEAK_GBS,
                   "timing": f"HIP graphs of {per} consecutive steps, HIP event after every graph, "
                             f"median of {n_batches} batches",
                   "steps_per_graph": per, "ms_per_step_one_graph_per_step": one_per_graph_s * 1e3,
                   "mean_ms_per_step": step_mean_s * 1e3, "wall_s": wall},
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
