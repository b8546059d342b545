"""GPU parity of int8_moe_gemv (expert-indexed products) against the oracle.

The call follows the DynQuantizedStorage trait page, provided method
indexed_moe_forward, read as stated in include/int8w.h: stacked experts,
x [tokens, 1 or topk, K], ids [tokens, topk] on the device, y [tokens, topk,
N], NaN (0x7FC0) for an id with no expert.  Products meet the gemv bound
|y - y_ref| <= 8e-3 |y_ref| + 2e-3 sum_k |w x|; NaN slots are compared bit
for bit.
"""
import numpy as np
import pytest
import torch

import oracle
from helpers import assert_close, bits_to_dev, dev_to_bits, upload
from weight_only_quantized_int8_amd import Int8Weight, moe_gemv, synth

pytestmark = pytest.mark.gpu

NAN_BF16 = 0x7FC0


def log(msg):
    print(msg, flush=True)


def run_case(seed, E, N, K, gs, T, topk, per_slot_rows, ids=None):
    rng = np.random.Generator(np.random.PCG64(seed))
    w = synth.gen_weight(rng, E * N, K, gs)
    if ids is None:
        ids = synth.gen_ids(rng, T, topk, E)
    x = synth.gen_act(rng, (T, topk if per_slot_rows else 1, K))
    W = upload(w)
    ids_d = torch.from_numpy(ids.view(np.int32)).cuda()
    y = moe_gemv(W, E, bits_to_dev(x), ids_d)
    torch.cuda.synchronize()
    return w, W, x, ids, dev_to_bits(y)


@pytest.mark.parametrize("E,N,K,gs,T,topk,per_slot", [
    (4, 96, 512, 64, 1, 2, False),       # the small shape, one token
    (8, 300, 1056, 32, 3, 2, True),      # ragged K (tail segment), own rows per slot
    (6, 77, 4128, 32, 5, 3, False),      # ragged K past one segment, odd N
    (8, 1024, 4096, 64, 4, 2, False),
    (3, 200, 16384, 128, 2, 2, True),    # 16-wave workgroups
    (2, 4096, 16384, 128, 1, 2, False),  # 16-wave workgroups, two rows side by side
    (2, 300, 20480, 64, 1, 2, False),    # one tile with per-item scales (K over 16384)
    (16, 64, 1024, 32, 16, 4, True),     # many slots, few rows each
])
def test_moe_gemv_matches_oracle(E, N, K, gs, T, topk, per_slot):
    log(f"moe_gemv E={E} N={N} K={K} gs={gs} T={T} topk={topk} per_slot={per_slot}")
    w, _, x, ids, y = run_case(80_000 + E * 7 + N + K + T, E, N, K, gs, T, topk, per_slot)
    y_ref, A = oracle.moe_gemv(w.packed, w.scales, w.biases, gs, E, x, ids)
    assert y.shape == (T, topk, N)
    assert_close(y, y_ref, A, f"moe_gemv E={E} N={N} K={K}")


def test_moe_gemv_repeated_experts_and_ids_without_expert():
    log("moe_gemv repeated and invalid ids")
    E, N, K, gs, T, topk = 4, 160, 2048, 64, 4, 3
    ids = np.array([[1, 1, 3], [4, 0, 0xFFFFFFFF], [2, 2, 2], [3, 0, 1]], np.uint32)
    w, _, x, ids, y = run_case(80_500, E, N, K, gs, T, topk, False, ids=ids)
    y_ref, A = oracle.moe_gemv(w.packed, w.scales, w.biases, gs, E, x, ids)
    bad = ids >= E
    assert (y[bad] == NAN_BF16).all()
    assert_close(y[~bad], y_ref[~bad], A[~bad], "moe_gemv valid slots")
    # one expert named twice with the same input row gives the same outputs
    assert np.array_equal(y[0, 0], y[0, 1]) and np.array_equal(y[2, 0], y[2, 2])


def test_moe_gemv_writes_exactly_the_slots():
    log("moe_gemv output extent")
    E, N, K, gs, T, topk = 4, 100, 1024, 32, 3, 2
    rng = np.random.Generator(np.random.PCG64(80_600))
    w = synth.gen_weight(rng, E * N, K, gs)
    ids = synth.gen_ids(rng, T, topk, E)
    x = synth.gen_act(rng, (T, 1, K))
    W = upload(w)
    buf = torch.full((T * topk * N + 64,), 1234.0, dtype=torch.bfloat16, device="cuda")
    y = buf[:T * topk * N].view(T, topk, N)
    moe_gemv(W, E, bits_to_dev(x), torch.from_numpy(ids.view(np.int32)).cuda(), y)
    torch.cuda.synchronize()
    assert (buf[T * topk * N:] == 1234.0).all()
    y_ref, A = oracle.moe_gemv(w.packed, w.scales, w.biases, gs, E, x, ids)
    assert_close(dev_to_bits(y), y_ref, A, "moe_gemv in a larger buffer")


def test_moe_gemv_equals_gemv_of_the_selected_expert():
    # one token, two experts of the 8B gate/up shape: each slot's rows are the
    # gemv of that expert's slice, with the same tile split, so bit-identical
    log("moe_gemv 8 x [14336, 4096] top-2 vs gemv")
    E, N, K, gs = 8, 14336, 4096, 64
    w, W, x, ids, y = run_case(80_700, E, N, K, gs, 1, 2, False)
    xd = bits_to_dev(x.reshape(K))
    for j in range(2):
        e = int(ids[0, j])
        sl = slice(e * N, (e + 1) * N)
        We = Int8Weight(W.packed[sl], W.scales[sl], W.biases[sl], gs)
        ye = dev_to_bits(We.gemv(xd))
        assert np.array_equal(y[0, j], ye), j
    y_ref, A = oracle.moe_gemv(w.packed, w.scales, w.biases, gs, E, x, ids)
    assert_close(y, y_ref, A, "moe_gemv 8 x [14336, 4096] top-2")


@pytest.mark.parametrize("E,N,K,gs,T,topk,per_slot", [
    (2, 640, 4096, 64, 6, 2, False),   # every token names both experts: 6 slots each, two passes of 4
    (8, 512, 2048, 32, 5, 3, True),    # own input rows per slot
    (64, 96, 1024, 128, 16, 8, False), # many experts, many slots
])
def test_moe_gemv_several_tokens_each_slot_equals_gemv_of_its_expert(E, N, K, gs, T, topk, per_slot):
    # the expert-grouped form streams each named expert once for all its
    # slots; every slot's outputs are still bit-identical to int8_gemv of its
    # expert on its input row (same per-row arithmetic), and within tolerance
    log(f"moe_gemv grouped E={E} N={N} K={K} gs={gs} T={T} topk={topk} per_slot={per_slot}")
    w, W, x, ids, y = run_case(81_000 + E + N + K + T, E, N, K, gs, T, topk, per_slot)
    y_ref, A = oracle.moe_gemv(w.packed, w.scales, w.biases, gs, E, x, ids)
    assert_close(y, y_ref, A, f"moe_gemv grouped E={E} T={T}")
    for t in range(T):
        for j in range(topk):
            e = int(ids[t, j])
            sl = slice(e * N, (e + 1) * N)
            We = Int8Weight(W.packed[sl], W.scales[sl], W.biases[sl], gs)
            xe = bits_to_dev(np.ascontiguousarray(x[t, j if per_slot else 0]))
            assert np.array_equal(y[t, j], dev_to_bits(We.gemv(xe))), (t, j)
