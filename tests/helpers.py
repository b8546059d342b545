"""Shared test helpers: uploading seeded inputs, reading BF16 results back, comparing with the oracle."""
from __future__ import annotations

import numpy as np
import torch

import oracle
from weight_only_quantized_int8_amd import synth


def bits_to_dev(bits: np.ndarray, device="cuda") -> torch.Tensor:
    """uint16 BF16 bit patterns -> bfloat16 tensor on the GPU."""
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(device)


def dev_to_bits(t: torch.Tensor) -> np.ndarray:
    """bfloat16 tensor -> uint16 bit patterns on the host."""
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def make_weight(seed: int, N: int, K: int, gs: int):
    rng = np.random.Generator(np.random.PCG64(seed))
    return synth.gen_weight(rng, N, K, gs), rng


def upload(w: synth.WeightArrays):
    from weight_only_quantized_int8_amd import Int8Weight
    return Int8Weight.from_arrays(w.packed, w.scales, w.biases, w.group_size)


def assert_close(y_bits: np.ndarray, y_ref: np.ndarray, A: np.ndarray, what: str) -> None:
    """The acceptance rule for products: |y - y_ref| <= 8e-3 |y_ref| + 2e-3 A, finite."""
    ok = oracle.within_tolerance(y_bits, y_ref, A)
    if not ok.all():
        idx = np.flatnonzero(~ok.ravel())
        i = idx[0]
        y = oracle.bf16_to_f32(y_bits.ravel()[i])
        raise AssertionError(
            f"{what}: {idx.size} of {ok.size} outputs out of tolerance; first at flat index {i}: "
            f"gpu {float(y)!r} ref {y_ref.ravel()[i]!r} A {A.ravel()[i]!r}")
