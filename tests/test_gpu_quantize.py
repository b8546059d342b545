"""GPU parity of int8_quantize (BF16 weight -> codes, scales, biases) against the oracle.

The quantizer follows the rustdoc page of the DynQuantizedStorage trait,
method quantize (the plain affine min/max reading stated in include/int8w.h).
Codes, scales and biases are integers and BF16 bit patterns decided in fp32 on
both sides, so the comparison is bit-exact.
"""
import numpy as np
import pytest
import torch

import oracle
from helpers import bits_to_dev, dev_to_bits
from weight_only_quantized_int8_amd import Int8Weight, binding, synth

pytestmark = pytest.mark.gpu


def log(msg):
    print(msg, flush=True)


def gpu_quantize(w_bits, gs):
    W = Int8Weight.quantize(bits_to_dev(w_bits), gs)
    torch.cuda.synchronize()
    packed = W.packed.cpu().numpy().view(np.uint32)
    return packed, dev_to_bits(W.scales), dev_to_bits(W.biases), W


@pytest.mark.parametrize("N,K,gs", [
    (256, 512, 64),
    (14336, 4096, 64),     # an 8B gate/up weight
    (4096, 14336, 128),
    (33, 96, 32),
    (7, 4128, 32),         # last 1 KiB item partial
    (1, 32, 32),
    (3000, 1280, 128),
])
def test_quantize_bit_exact(N, K, gs):
    log(f"quantize N={N} K={K} gs={gs}")
    rng = np.random.Generator(np.random.PCG64(70_000 + N + K + gs))
    w = synth.gen_dense_weight(rng, N, K)
    p_ref, s_ref, b_ref = oracle.quantize(w, gs)
    p, s, b, _ = gpu_quantize(w, gs)
    assert np.array_equal(s, s_ref)
    assert np.array_equal(b, b_ref)
    assert np.array_equal(p, p_ref)


def test_quantize_special_groups():
    log("quantize special groups")
    N, K, gs = 8, 256, 64
    rng = np.random.Generator(np.random.PCG64(70_100))
    w = synth.gen_dense_weight(rng, N, K)
    w[0, :] = 0                  # all +0
    w[1, :64] = 0x8000           # all -0
    w[1, 64:128] = 0x8000
    w[1, 64:96] = 0              # mixed zeros
    w[2, :64] = 0x3FC0           # constant 1.5
    w[3, :64] = np.where(np.arange(64) % 2 == 0, 0x4F00, 0xCF00)  # +-2^31: span overflows nothing, large scale
    w[4, 128:192] = 0x3F80       # constant, then one outlier
    w[4, 150] = 0x4580
    w[5, :] = np.arange(256, dtype=np.uint16) + 0x3F80  # a run of consecutive BF16 values
    p_ref, s_ref, b_ref = oracle.quantize(w, gs)
    p, s, b, _ = gpu_quantize(w, gs)
    assert np.array_equal(s, s_ref) and np.array_equal(b, b_ref) and np.array_equal(p, p_ref)
    assert (b_ref[0] == 0).all() and (b_ref[1, :2] == 0).all()  # zero minimum is +0


@pytest.mark.parametrize("gs", [32, 64, 128])
def test_quantize_signed_zero_groups(gs):
    # all-zero groups in every order of -0 and +0, and groups whose maximum is
    # a zero: scale and bias follow the oracle bit for bit (a zero extreme is
    # +0 on both sides, so the lane order of the GPU min/max does not matter)
    log(f"quantize signed-zero groups gs={gs}")
    N, K = 12, 4 * gs
    rng = np.random.Generator(np.random.PCG64(70_400 + gs))
    w = synth.gen_dense_weight(rng, N, K)
    pz, nz = np.uint16(0x0000), np.uint16(0x8000)
    for n in range(N):
        for g in range(K // gs):
            sl = slice(g * gs, (g + 1) * gs)
            kind = (n + g) % 6
            if kind == 0:
                w[n, sl] = nz; w[n, g * gs] = pz                    # one +0 first, then -0
            elif kind == 1:
                w[n, sl] = pz; w[n, g * gs] = nz                    # one -0 first, then +0
            elif kind == 2:
                w[n, sl] = np.where(rng.random(gs) < 0.5, nz, pz)   # random signs
            elif kind == 3:
                w[n, sl] = nz                                       # all -0
            elif kind == 4:
                w[n, sl] = np.where(rng.random(gs) < 0.5, nz, pz)   # maximum a zero,
                w[n, g * gs + int(rng.integers(gs))] = 0xBF80       # minimum -1
    p_ref, s_ref, b_ref = oracle.quantize(w, gs)
    p, s, b, _ = gpu_quantize(w, gs)
    assert np.array_equal(s, s_ref) and np.array_equal(b, b_ref) and np.array_equal(p, p_ref)
    zero_groups = np.array([[(n + g) % 6 < 4 for g in range(K // gs)] for n in range(N)])
    assert (s_ref[zero_groups] == 0).all() and (b_ref[zero_groups] == 0).all()


def test_quantize_then_dequantize_round_trip_matches_oracle():
    log("quantize -> dequantize_to round trip")
    N, K, gs = 1024, 2048, 64
    rng = np.random.Generator(np.random.PCG64(70_200))
    w = synth.gen_dense_weight(rng, N, K)
    p_ref, s_ref, b_ref = oracle.quantize(w, gs)
    _, _, _, W = gpu_quantize(w, gs)
    dq = W.dequantize_to()
    torch.cuda.synchronize()
    assert np.array_equal(dev_to_bits(dq).reshape(N, K), oracle.dequantize_to(p_ref, s_ref, b_ref, gs))


def test_quantize_writes_only_its_outputs():
    log("quantize guard bytes")
    N, K, gs = 37, 160, 32
    rng = np.random.Generator(np.random.PCG64(70_300))
    w = bits_to_dev(synth.gen_dense_weight(rng, N, K))
    G = K // gs
    packed = torch.full((N * K // 4 + 16,), -7, dtype=torch.int32, device="cuda")
    scales = torch.full((N * G + 16,), 3.0, dtype=torch.bfloat16, device="cuda")
    biases = torch.full((N * G + 16,), 5.0, dtype=torch.bfloat16, device="cuda")
    rc = binding.int8_quantize(w.data_ptr(), N, K, gs, packed.data_ptr(), scales.data_ptr(), biases.data_ptr(),
                               torch.cuda.current_stream().cuda_stream)
    assert rc == binding.INT8W_OK
    torch.cuda.synchronize()
    assert (packed[N * K // 4:].cpu() == -7).all()
    assert (scales[N * G:].float().cpu() == 3.0).all() and (biases[N * G:].float().cpu() == 5.0).all()


def test_quantize_exact_ties_take_the_division_path():
    # every value after the first two of each group is exactly halfway between
    # two codes (scale 1/16): the kernel's reciprocal shortcut must defer to
    # the IEEE division and round to even, like the oracle
    log("quantize exact ties")
    k = np.arange(62)
    grp = np.concatenate([[0.0, 255 / 16], (2 * k + 1) / 32.0]).astype(np.float32)
    rng = np.random.Generator(np.random.PCG64(70_300))
    N, K, gs = 64, 1024, 64
    w = synth.gen_dense_weight(rng, N, K)
    tie_bits = oracle.f32_to_bf16(grp)
    for n in range(0, N, 3):
        for g in range(n % 4, K // gs, 4):
            w[n, g * gs:(g + 1) * gs] = rng.permutation(tie_bits)
    p_ref, s_ref, b_ref = oracle.quantize(w, gs)
    p, s, b, _ = gpu_quantize(w, gs)
    assert np.array_equal(s, s_ref) and np.array_equal(b, b_ref)
    assert np.array_equal(p, p_ref)
