"""GPU parity of int8w_fp8_gemv (FP8 E4M3 weight, y = W x) against the oracle.

The call follows the rustdoc page "Fp8Weight": [n, k] E4M3 bytes with a
per-row f32 scale, per-block BF16 or f32 scales [ceil(n/BS), ceil(k/BS)], or
one global scale (readings stated in include/int8w.h).  Products meet
|y - y_ref| <= 8e-3 |y_ref| + 2e-3 sum_k |w x|; the decode of every code is
checked bit for bit.
"""
import numpy as np
import pytest
import torch

import oracle
from helpers import assert_close, bits_to_dev, dev_to_bits
from weight_only_quantized_int8_amd import Fp8Weight, synth
from weight_only_quantized_int8_amd.binding import FP8_BLOCK_BF16, FP8_BLOCK_F32, FP8_PER_ROW, FP8_SINGLE

pytestmark = pytest.mark.gpu

FORMATS = {"row": FP8_PER_ROW, "block_bf16": FP8_BLOCK_BF16, "block_f32": FP8_BLOCK_F32, "single": FP8_SINGLE}


def log(msg):
    print(msg, flush=True)


def make(rng, N, K, fmt, bs):
    codes = synth.gen_fp8_codes(rng, N, K)
    if fmt == FP8_PER_ROW:
        scale = synth.gen_fp8_scale(rng, N, bf16=False)
    elif fmt in (FP8_BLOCK_BF16, FP8_BLOCK_F32):
        scale = synth.gen_fp8_scale(rng, (-(-N // bs), -(-K // bs)), bf16=fmt == FP8_BLOCK_BF16)
    else:
        scale = None
    return codes, scale


def upload(codes, scale, fmt, bs, single=2.5e-4):
    w = torch.from_numpy(codes).cuda()
    s = None
    if scale is not None:
        s = (bits_to_dev(scale) if fmt == FP8_BLOCK_BF16 else torch.from_numpy(scale).cuda())
    return Fp8Weight(w, s, fmt, bs, single)


@pytest.mark.parametrize("fmt", list(FORMATS))
@pytest.mark.parametrize("N,K,bs", [
    (256, 512, 128),       # small
    (14336, 4096, 128),    # 8B gate/up shape
    (4096, 14336, 128),    # 8B down shape (16-wave workgroups, two rows side by side)
    (300, 1040, 64),       # ragged k (tail segment), n not a multiple of the block
    (77, 4112, 256),
    (5, 36864, 1024),      # several K-tiles
    (1000, 3072, 128),     # register-resident form, three segments
    (600, 2048, 64),       # two segments, several row blocks per wave
    (65, 1024, 128),       # one segment, ragged rows
    (40, 20000, 64),       # two K-tiles, the last segment partial, block scales loaded per item
    (3000, 8192, 512),     # LDS form with one row at a time, several row blocks
])
def test_fp8_gemv_matches_oracle(fmt, N, K, bs):
    log(f"fp8_gemv {fmt} N={N} K={K} bs={bs}")
    f = FORMATS[fmt]
    rng = np.random.Generator(np.random.PCG64(90_000 + N + K + bs + f))
    codes, scale = make(rng, N, K, f, bs)
    x = synth.gen_act(rng, K)
    W = upload(codes, scale, f, bs)
    y = dev_to_bits(W.gemv(bits_to_dev(x)))
    y_ref, A = oracle.fp8_gemv(codes, scale, f, x, bs, single_scale=2.5e-4)
    assert_close(y, y_ref, A, f"fp8_gemv {fmt} {N}x{K}")


def test_fp8_decode_of_every_code_is_exact():
    # row i holds code i in column 0 and zeros elsewhere; x = e_0, scale 1:
    # y[i] is the decoded code (every E4M3 value is exact in BF16)
    log("fp8 decode of all 256 codes")
    N, K = 256, 64
    codes = np.zeros((N, K), np.uint8)
    codes[:, 0] = np.arange(256, dtype=np.uint8)
    x = np.zeros(K, np.uint16)
    x[0] = 0x3F80  # 1.0
    W = upload(codes, np.ones(N, np.float32), FP8_PER_ROW, 128)
    y = dev_to_bits(W.gemv(bits_to_dev(x)))
    ref = oracle.e4m3_to_f64(np.arange(256, dtype=np.uint8))
    nan = np.isnan(ref)
    assert nan.sum() == 2
    assert np.isnan(oracle.bf16_to_f32(y[nan])).all()
    want = oracle.f32_to_bf16(ref[~nan].astype(np.float32))
    want[want == 0x8000] = 0  # -0 * 1 summed from +0 is +0, on both sides
    assert np.array_equal(y[~nan], want)


def test_fp8_gemv_writes_exactly_n_outputs():
    log("fp8_gemv output extent")
    N, K, bs = 333, 2048, 128
    rng = np.random.Generator(np.random.PCG64(90_500))
    codes, scale = make(rng, N, K, FP8_BLOCK_BF16, bs)
    x = synth.gen_act(rng, K)
    W = upload(codes, scale, FP8_BLOCK_BF16, bs)
    buf = torch.full((N + 64,), 1234.0, dtype=torch.bfloat16, device="cuda")
    W.gemv(bits_to_dev(x), buf[:N])
    torch.cuda.synchronize()
    assert (buf[N:] == 1234.0).all()
    y_ref, A = oracle.fp8_gemv(codes, scale, FP8_BLOCK_BF16, x, bs)
    assert_close(dev_to_bits(buf[:N]), y_ref, A, "fp8_gemv in a larger buffer")
