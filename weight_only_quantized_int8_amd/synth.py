"""Seeded synthetic inputs for the 8-bit affine weight-only linear layers.

This module draws random numbers and rounds them to BF16 with torch's own CPU
conversion; it holds none of the layers' arithmetic (no unpacking, no affine
dequantization, no products).  Both the CPU oracle's tests and the GPU path's
tests and benchmark take their inputs from here, so the two sides see the same
bytes.

Value distributions (the decode/prefill workloads of these layers):
  codes   uint8 uniform on [0, 255], packed 4 per uint32, code k in byte k%4;
  scales  BF16 of fp32 uniform[0.002, 0.01];
  biases  BF16 of fp32 (-128 * scale_bf16 * (1 + U(-0.05, 0.05)));
  x, gate, up, x_resid: BF16 of fp32 N(0, 1);
  dense BF16 weights (the quantizer's input): BF16 of fp32 N(0, 0.02^2), with
  one row in 64 scaled by 8 (outlier rows) and one value in 512 by 16
  (outlier values).
  FP8 E4M3 weights: E4M3 (torch's float8_e4m3fn conversion) of fp32
  N(0, 96^2) clipped to +-448, so that the codes span the format's range;
  per-row scales f32 uniform[1e-4, 4e-4]; block scales the same, as BF16 or
  f32.
  routing ids: each token names topk distinct experts, uniformly.
Generator: NumPy PCG64, seed = 1000 * workload_index + shape_index, draws in
the fixed order codes, scales, bias jitter, then activations.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np
import torch


def to_bf16_bits(values_f32: np.ndarray) -> np.ndarray:
    """fp32 -> BF16 bit patterns (uint16) via torch's CPU round-to-nearest-even."""
    t = torch.from_numpy(np.ascontiguousarray(values_f32, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


@dataclass
class WeightArrays:
    packed: np.ndarray   # uint32 [N, K/4]
    scales: np.ndarray   # uint16 (BF16 bits) [N, K/gs]
    biases: np.ndarray   # uint16 (BF16 bits) [N, K/gs]
    out_features: int
    in_features: int
    group_size: int


def make_seed(workload_index: int, shape_index: int) -> int:
    return 1000 * int(workload_index) + int(shape_index)


def gen_weight(rng: np.random.Generator, N: int, K: int, group_size: int) -> WeightArrays:
    if K % 4 or K % group_size:
        raise ValueError("in_features must be a multiple of 4 and of group_size")
    G = K // group_size
    codes = rng.integers(0, 256, size=(N, K), dtype=np.uint8)
    packed = np.ascontiguousarray(codes).view("<u4").reshape(N, K // 4).astype(np.uint32, copy=False)
    s32 = rng.uniform(0.002, 0.01, size=(N, G)).astype(np.float32)
    scales = to_bf16_bits(s32)
    jitter = rng.uniform(-0.05, 0.05, size=(N, G)).astype(np.float32)
    s_back = torch.from_numpy(scales.view(np.int16)).view(torch.bfloat16).float().numpy()
    b32 = (np.float32(-128.0) * s_back * (np.float32(1.0) + jitter)).astype(np.float32)
    biases = to_bf16_bits(b32)
    return WeightArrays(packed, scales, biases, N, K, group_size)


def gen_act(rng: np.random.Generator, shape) -> np.ndarray:
    """BF16 bits of N(0,1) samples."""
    return to_bf16_bits(rng.standard_normal(size=shape).astype(np.float32))


def gen_case(workload_index: int, shape_index: int, N: int, K: int, group_size: int,
             act_shapes: dict[str, tuple]) -> tuple[WeightArrays, dict[str, np.ndarray]]:
    """One weight plus named activations, in the fixed draw order."""
    rng = np.random.Generator(np.random.PCG64(make_seed(workload_index, shape_index)))
    w = gen_weight(rng, N, K, group_size)
    acts = {name: gen_act(rng, shape) for name, shape in act_shapes.items()}
    return w, acts


def gen_dense_weight(rng: np.random.Generator, N: int, K: int) -> np.ndarray:
    """BF16 bit patterns [N, K] of a dense weight with outlier rows and values."""
    w = rng.standard_normal((N, K)).astype(np.float32) * np.float32(0.02)
    rows = rng.random(N) < 1.0 / 64
    w[rows] *= np.float32(8.0)
    spikes = rng.random((N, K)) < 1.0 / 512
    w[spikes] *= np.float32(16.0)
    return to_bf16_bits(w)


def gen_ids(rng: np.random.Generator, tokens: int, topk: int, num_experts: int) -> np.ndarray:
    """Synthetic routing: each token names topk distinct experts, uniformly at
    random (what a top-k router yields), as uint32 [tokens, topk]."""
    if topk > num_experts:
        raise ValueError("topk exceeds the number of experts")
    out = np.empty((tokens, topk), np.uint32)
    for t in range(tokens):
        out[t] = rng.permutation(num_experts)[:topk]
    return out


def gen_fp8_codes(rng: np.random.Generator, N: int, K: int) -> np.ndarray:
    """E4M3 bytes [N, K]: fp32 N(0, 96^2) clipped to +-448, converted by torch."""
    v = np.clip(rng.standard_normal((N, K)).astype(np.float32) * np.float32(96.0), -448.0, 448.0)
    return torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy().copy()


def gen_fp8_scale(rng: np.random.Generator, shape, bf16: bool) -> np.ndarray:
    """Scales f32 uniform[1e-4, 4e-4]: float32, or BF16 bit patterns."""
    s = rng.uniform(1e-4, 4e-4, size=shape).astype(np.float32)
    return to_bf16_bits(s) if bf16 else s
