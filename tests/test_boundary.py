"""The C-ABI boundary on the CPU: the library loads, exports what include/int8w.h
declares, and rejects every invalid call before launching anything.

No test here passes a call that validates (it would launch a kernel); each
one checks a status code and the last-error text.  Rules follow the rustdoc
page "MlxInt8Weight", method load (2-D U32 weight, BF16 scales/biases of
shape [out_features, in_features/group_size], group_size divides
in_features) plus the library's own alignment and aliasing rules.
"""
import os
import re

import pytest

from weight_only_quantized_int8_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_functions(header="int8w.h"):
    text = open(os.path.join(ROOT, "include", header)).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(int8w?_\w+)\s*\(", text, flags=re.M)))


def all_header_functions():
    return sorted(set().union(*(header_functions(h) for h in sorted(os.listdir(os.path.join(ROOT, "include")))
                                if h.endswith(".h"))))


def test_header_declares_the_entry_points():
    assert header_functions() == sorted(B.EXPORTED)
    assert header_functions("int8w_measure.h") == sorted(B.EXPORTED_MEASURE)


def test_library_exports_every_declared_symbol():
    lib = B.load_library()
    names = all_header_functions()
    assert len(names) == len(B.EXPORTED) + len(B.EXPORTED_MEASURE)
    for name in names:
        assert hasattr(lib, name), name
    nm = os.popen(f"nm -D --defined-only {B.library_path()}").read()
    for name in names:
        assert re.search(rf"\bT {name}$", nm, flags=re.M), f"{name} is not an exported text symbol"


@pytest.mark.parametrize("call,code,text", [
    (lambda: B.int8w_stream_read(0, 1024, A16, 0), B.INT8W_ERR_NULL, "src is NULL"),
    (lambda: B.int8w_stream_read(A16, 1000, A16, 0), B.INT8W_ERR_SHAPE, "multiple of 1024"),
    (lambda: B.int8w_stream_read(A16, 0, A16, 0), B.INT8W_ERR_SHAPE, "multiple of 1024"),
    (lambda: B.int8w_stream_read(A16 + 8, 1024, A16, 0), B.INT8W_ERR_ALIGN, "src is not 16-byte"),
    (lambda: B.int8w_stream_read(A16, 1024, 0, 0), B.INT8W_ERR_NULL, "sink is NULL"),
    (lambda: B.int8w_stream_copy(A16, 0, 1024, 0), B.INT8W_ERR_NULL, "dst is NULL"),
    (lambda: B.int8w_stream_copy(A16, A16 + 512, 1024, 0), B.INT8W_ERR_ALIAS, "overlaps"),
    (lambda: B.int8w_stream_copy(A16, 2 * A16 + 4, 1024, 0), B.INT8W_ERR_ALIGN, "dst is not 16-byte"),
    (lambda: B.int8w_stream_expand(A16, 0, 1024, 0), B.INT8W_ERR_NULL, "dst is NULL"),
    # the expand writes 2 * bytes: a dst 1024 bytes below src overlaps it
    (lambda: B.int8w_stream_expand(A16 + 1024, A16, 1024, 0), B.INT8W_ERR_ALIAS, "overlaps"),
    (lambda: B.int8w_stream_expand(A16, A16 + 2048 + 8, 1024, 0), B.INT8W_ERR_ALIGN, "dst is not 16-byte"),
    (lambda: B.int8w_stream_expand(A16, A16 + 4096, 1000, 0), B.INT8W_ERR_SHAPE, "multiple of 1024"),
])
def test_calibration_streams_reject_invalid_calls(call, code, text):
    rc, msg = err(call())
    assert rc == code and text in msg, (rc, msg)


def test_storage_bytes():
    assert B.storage_bytes(14336, 4096, 64) == 14336 * 4096 + 4 * 14336 * 64
    assert B.storage_bytes(8192, 28672, 128) == 8192 * 28672 + 4 * 8192 * 224
    assert B.storage_bytes(4, 64, 48) == 0
    assert B.storage_bytes(0, 64, 32) == 0


A16 = 1 << 20  # fake, 16-byte aligned "device" addresses: never dereferenced by these tests


def desc(N=64, K=256, gs=64, packed=A16, scales=2 * A16, biases=3 * A16):
    return B.WeightDesc(packed, scales, biases, N, K, gs)


def err(rc):
    assert rc != B.INT8W_OK
    return rc, B.load_library().int8w_last_error().decode()


@pytest.mark.parametrize("kw,code,text", [
    (dict(packed=0), B.INT8W_ERR_NULL, "missing a tensor"),
    (dict(scales=0), B.INT8W_ERR_NULL, "missing a tensor"),
    (dict(biases=0), B.INT8W_ERR_NULL, "missing a tensor"),
    (dict(N=0), B.INT8W_ERR_SHAPE, "zero dimension"),
    (dict(K=0), B.INT8W_ERR_SHAPE, "zero dimension"),
    (dict(gs=0), B.INT8W_ERR_SHAPE, "zero dimension"),
    (dict(K=96, gs=64), B.INT8W_ERR_SHAPE, "does not divide"),
    (dict(K=48, gs=48), B.INT8W_ERR_UNSUPPORTED, "not supported"),
    (dict(K=256, gs=256), B.INT8W_ERR_UNSUPPORTED, "not supported"),
    (dict(K=32, gs=16), B.INT8W_ERR_UNSUPPORTED, "not supported"),
    (dict(packed=A16 + 4), B.INT8W_ERR_ALIGN, "packed"),
    (dict(scales=2 * A16 + 1), B.INT8W_ERR_ALIGN, "scales/biases"),
    (dict(N=1 << 20, K=1 << 20, gs=64), B.INT8W_ERR_SHAPE, "too large"),
])
def test_validate_rejects(kw, code, text):
    rc, msg = err(B.int8w_validate(desc(**kw)))
    assert rc == code and text in msg
    # every entry point applies the same weight checks before anything else
    for call in (lambda d: B.int8_dequantize_to(d, 4 * A16, 0),
                 lambda d: B.int8_gemv(d, 4 * A16, 5 * A16, 0),
                 lambda d: B.int8_gemv_silu_gate(d, 4 * A16, 5 * A16, 6 * A16, 0),
                 lambda d: B.int8_gemv_silu_gate_resid(d, 4 * A16, 5 * A16, 6 * A16, 7 * A16, 0),
                 lambda d: B.int8_gemm(d, 4 * A16, 5 * A16, 3, 0)):
        assert err(call(desc(**kw)))[0] == code


def test_validate_accepts_and_clears_error():
    B.int8w_validate(desc(gs=48, K=96))
    assert B.int8w_validate(desc()) == B.INT8W_OK
    assert B.load_library().int8w_last_error() == b""
    for gs in (32, 64, 128):
        assert B.int8w_validate(desc(K=4 * gs, gs=gs)) == B.INT8W_OK


def test_null_activation_and_output_pointers():
    d = desc()
    assert err(B.int8_dequantize_to(d, 0, 0))[0] == B.INT8W_ERR_NULL
    assert err(B.int8_gemv(d, 0, 5 * A16, 0))[0] == B.INT8W_ERR_NULL
    assert err(B.int8_gemv(d, 4 * A16, 0, 0))[0] == B.INT8W_ERR_NULL
    assert err(B.int8_gemv_silu_gate(d, 0, 5 * A16, 6 * A16, 0))[0] == B.INT8W_ERR_NULL
    assert err(B.int8_gemv_silu_gate(d, 4 * A16, 0, 6 * A16, 0))[0] == B.INT8W_ERR_NULL
    assert err(B.int8_gemv_silu_gate_resid(d, 4 * A16, 5 * A16, 0, 7 * A16, 0))[0] == B.INT8W_ERR_NULL
    assert err(B.int8_gemm(d, 0, 5 * A16, 2, 0))[0] == B.INT8W_ERR_NULL


def test_alignment_of_activations_and_outputs():
    d = desc()
    assert err(B.int8_dequantize_to(d, 4 * A16 + 2, 0))[0] == B.INT8W_ERR_ALIGN
    assert err(B.int8_gemv(d, 4 * A16 + 8, 5 * A16, 0))[0] == B.INT8W_ERR_ALIGN
    assert err(B.int8_gemv(d, 4 * A16, 5 * A16 + 1, 0))[0] == B.INT8W_ERR_ALIGN
    assert err(B.int8_gemv_silu_gate(d, 4 * A16 + 4, 5 * A16, 6 * A16, 0))[0] == B.INT8W_ERR_ALIGN
    assert err(B.int8_gemv_silu_gate_resid(d, 4 * A16, 5 * A16, 6 * A16 + 1, 7 * A16, 0))[0] == B.INT8W_ERR_ALIGN
    assert err(B.int8_gemm(d, 4 * A16 + 2, 5 * A16, 2, 0))[0] == B.INT8W_ERR_ALIGN


def test_outputs_may_not_overlap_inputs():
    N, K, gs = 64, 256, 64
    d = desc(N, K, gs)
    # y inside packed, scales, biases
    for base in (A16 + 64, 2 * A16 + 2, 3 * A16 + 126):
        assert err(B.int8_gemv(d, 4 * A16, base, 0))[0] == B.INT8W_ERR_ALIAS
    # y overlapping x by one element at either end
    assert err(B.int8_gemv(d, 4 * A16, 4 * A16 + 2 * K - 2, 0))[0] == B.INT8W_ERR_ALIAS
    assert err(B.int8_gemv(d, 4 * A16 + 16, 4 * A16 + 16 - 2 * N + 2, 0))[0] == B.INT8W_ERR_ALIAS
    # dequantize_to output over the codes
    assert err(B.int8_dequantize_to(d, A16, 0))[0] == B.INT8W_ERR_ALIAS
    # gated: y over gate or up; y partially over x_resid
    assert err(B.int8_gemv_silu_gate(d, 4 * A16, 5 * A16, 4 * A16 + 32, 0))[0] == B.INT8W_ERR_ALIAS
    assert err(B.int8_gemv_silu_gate(d, 4 * A16, 5 * A16, 5 * A16, 0))[0] == B.INT8W_ERR_ALIAS
    rc, msg = err(B.int8_gemv_silu_gate_resid(d, 4 * A16, 5 * A16, 6 * A16, 6 * A16 + 2, 0))
    assert rc == B.INT8W_ERR_ALIAS and "x_resid" in msg
    # gemm: Y over X
    assert err(B.int8_gemm(d, 4 * A16, 4 * A16 + 2 * K * 3 - 2, 3, 0))[0] == B.INT8W_ERR_ALIAS
    # adjacent but not overlapping is only refused for another reason (none here) -> would launch; not called


def test_gemm_m_zero_is_a_no_op():
    assert B.int8_gemm(desc(), 0, 0, 0, 0) == B.INT8W_OK


def test_gemm_tiled_width_limit():
    # a 256-row X tile of in_features = 2^23 would need 4 GiB of 32-bit offsets
    rc, msg = err(B.int8_gemm(desc(N=64, K=1 << 23, gs=64), 4 * A16, 1 << 40, 17, 0))
    assert rc == B.INT8W_ERR_SHAPE and "in_features" in msg


def test_gemm_rows_times_width_limit():
    rc, msg = err(B.int8_gemm(desc(N=64, K=1 << 16, gs=64), 4 * A16, 1 << 40, 1 << 17, 0))
    assert rc == B.INT8W_ERR_SHAPE and "rows" in msg


def test_wrapper_applies_load_rules_on_tensors():
    torch = pytest.importorskip("torch")
    p = torch.zeros((4, 16), dtype=torch.int32)
    s = torch.zeros((4, 2), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="2-D 32-bit"):
        B.Int8Weight(p.float(), s, s, 32)
    with pytest.raises(ValueError, match="2-D 32-bit"):
        B.Int8Weight(p.reshape(-1), s, s, 32)
    with pytest.raises(ValueError, match="bfloat16"):
        B.Int8Weight(p, s.float(), s, 32)
    with pytest.raises(ValueError, match=r"\[4, 2\]"):
        B.Int8Weight(p, s[:, :1], s[:, :1], 32)
    with pytest.raises(ValueError, match="does not divide"):
        B.Int8Weight(p, s, s, 48)
    with pytest.raises(ValueError, match="one GPU"):
        B.Int8Weight(p, s, s, 32)  # CPU tensors are refused before any call


def test_gemv_multi_rejects():
    q, k = desc(N=64, K=256, gs=64), desc(N=16, K=256, gs=64, packed=8 * A16, scales=9 * A16, biases=10 * A16)
    x, y0, y1 = 4 * A16, 5 * A16, 6 * A16
    rc, msg = err(B.int8_gemv_multi([], x, [], 0))
    assert rc == B.INT8W_ERR_SHAPE and "count 0" in msg
    five = [desc(packed=(20 + 3 * i) * A16, scales=(21 + 3 * i) * A16, biases=(22 + 3 * i) * A16) for i in range(5)]
    rc, msg = err(B.int8_gemv_multi(five, x, [(40 + i) * A16 for i in range(5)], 0))
    assert rc == B.INT8W_ERR_SHAPE and "count 5" in msg
    # every weight is validated; in_features and group_size must agree
    assert err(B.int8_gemv_multi([q, desc(N=0)], x, [y0, y1], 0))[0] == B.INT8W_ERR_SHAPE
    rc, msg = err(B.int8_gemv_multi([q, desc(N=16, K=512, packed=8 * A16, scales=9 * A16, biases=10 * A16)],
                                    x, [y0, y1], 0))
    assert rc == B.INT8W_ERR_SHAPE and "in_features" in msg
    rc, msg = err(B.int8_gemv_multi([q, desc(N=16, K=256, gs=32, packed=8 * A16, scales=9 * A16, biases=10 * A16)],
                                    x, [y0, y1], 0))
    assert rc == B.INT8W_ERR_SHAPE and "group_size" in msg
    # pointers
    assert err(B.int8_gemv_multi([q, k], 0, [y0, y1], 0))[0] == B.INT8W_ERR_NULL
    assert err(B.int8_gemv_multi([q, k], x, [y0, 0], 0))[0] == B.INT8W_ERR_NULL
    assert err(B.int8_gemv_multi([q, k], x + 2, [y0, y1], 0))[0] == B.INT8W_ERR_ALIGN
    assert err(B.int8_gemv_multi([q, k], x, [y0, y1 + 1], 0))[0] == B.INT8W_ERR_ALIGN
    # outputs: not over x, not over any weight, not over each other
    assert err(B.int8_gemv_multi([q, k], x, [y0, x + 64], 0))[0] == B.INT8W_ERR_ALIAS
    assert err(B.int8_gemv_multi([q, k], x, [y0, 8 * A16 + 16], 0))[0] == B.INT8W_ERR_ALIAS
    assert err(B.int8_gemv_multi([q, k], x, [y0, 2 * A16], 0))[0] == B.INT8W_ERR_ALIAS
    rc, msg = err(B.int8_gemv_multi([q, k], x, [y0, y0 + 2 * 64 - 2], 0))
    assert rc == B.INT8W_ERR_ALIAS and "y[0] and y[1]" in msg


def test_quantize_rejects():
    w, pk, sc, bi = 4 * A16, A16, 2 * A16, 3 * A16
    assert err(B.int8_quantize(0, 64, 256, 64, pk, sc, bi, 0))[0] == B.INT8W_ERR_NULL
    assert err(B.int8_quantize(w, 64, 256, 64, 0, sc, bi, 0))[0] == B.INT8W_ERR_NULL
    assert err(B.int8_quantize(w, 0, 256, 64, pk, sc, bi, 0))[0] == B.INT8W_ERR_SHAPE
    assert err(B.int8_quantize(w, 64, 96, 64, pk, sc, bi, 0))[0] == B.INT8W_ERR_SHAPE
    assert err(B.int8_quantize(w, 64, 96, 48, pk, sc, bi, 0))[0] == B.INT8W_ERR_UNSUPPORTED
    assert err(B.int8_quantize(w + 2, 64, 256, 64, pk, sc, bi, 0))[0] == B.INT8W_ERR_ALIGN
    assert err(B.int8_quantize(w, 64, 256, 64, pk + 8, sc, bi, 0))[0] == B.INT8W_ERR_ALIGN
    # outputs over the input or over each other
    rc, msg = err(B.int8_quantize(w, 64, 256, 64, w + 1024, sc, bi, 0))
    assert rc == B.INT8W_ERR_ALIAS and "packed" in msg
    rc, msg = err(B.int8_quantize(w, 64, 256, 64, pk, sc, sc + 64, 0))
    assert rc == B.INT8W_ERR_ALIAS and "scales" in msg and "biases" in msg


def test_moe_gemv_rejects():
    w = desc(N=64, K=256, gs=64)  # 4 experts of [16, 256] stacked
    x, ids, y = 4 * A16, 5 * A16, 6 * A16
    assert B.int8_moe_gemv(w, 4, x, 1, ids, 0, 2, y, 0) == B.INT8W_OK  # no slots: nothing to do
    assert B.int8_moe_gemv(w, 4, x, 1, ids, 3, 0, y, 0) == B.INT8W_OK
    rc, msg = err(B.int8_moe_gemv(w, 0, x, 1, ids, 1, 2, y, 0))
    assert rc == B.INT8W_ERR_SHAPE and "experts" in msg
    assert err(B.int8_moe_gemv(w, 3, x, 1, ids, 1, 2, y, 0))[0] == B.INT8W_ERR_SHAPE
    assert err(B.int8_moe_gemv(desc(N=0), 4, x, 1, ids, 1, 2, y, 0))[0] == B.INT8W_ERR_SHAPE
    rc, msg = err(B.int8_moe_gemv(w, 4, x, 1, ids, 40000, 2, y, 0))
    assert rc == B.INT8W_ERR_SHAPE and "slots" in msg
    rc, msg = err(B.int8_moe_gemv(w, 4, x, 3, ids, 1, 2, y, 0))
    assert rc == B.INT8W_ERR_SHAPE and "x_rows" in msg
    for args in ((0, ids, y), (x, 0, y), (x, ids, 0)):
        assert err(B.int8_moe_gemv(w, 4, args[0], 1, args[1], 1, 2, args[2], 0))[0] == B.INT8W_ERR_NULL
    assert err(B.int8_moe_gemv(w, 4, x + 8, 1, ids, 1, 2, y, 0))[0] == B.INT8W_ERR_ALIGN
    assert err(B.int8_moe_gemv(w, 4, x, 1, ids + 2, 1, 2, y, 0))[0] == B.INT8W_ERR_ALIGN
    assert err(B.int8_moe_gemv(w, 4, x, 1, ids, 1, 2, y + 1, 0))[0] == B.INT8W_ERR_ALIGN
    # y [tokens, topk, N] over x [tokens, x_rows, K], over ids, over the experts
    rc, msg = err(B.int8_moe_gemv(w, 4, x, 2, ids, 3, 2, x + 6 * 256 * 2 - 2, 0))
    assert rc == B.INT8W_ERR_ALIAS and "input x" in msg
    rc, msg = err(B.int8_moe_gemv(w, 4, x, 1, ids, 3, 2, ids + 20, 0))
    assert rc == B.INT8W_ERR_ALIAS and "ids" in msg
    rc, msg = err(B.int8_moe_gemv(w, 4, x, 1, ids, 1, 2, 3 * A16 + 64, 0))
    assert rc == B.INT8W_ERR_ALIAS and "biases" in msg


def fp8desc(n=64, k=256, fmt=B.FP8_PER_ROW, weight=A16, scale=2 * A16, bs=128, single=1.0):
    return B.Fp8WeightDesc(weight, scale, n, k, fmt, bs, single)


def test_fp8_gemv_rejects():
    x, y = 4 * A16, 5 * A16
    rc, msg = err(B.int8w_fp8_gemv(fp8desc(weight=0), x, y, 0))
    assert rc == B.INT8W_ERR_NULL
    assert err(B.int8w_fp8_gemv(fp8desc(n=0), x, y, 0))[0] == B.INT8W_ERR_SHAPE
    rc, msg = err(B.int8w_fp8_gemv(fp8desc(k=200), x, y, 0))
    assert rc == B.INT8W_ERR_SHAPE and "multiple of 16" in msg
    rc, msg = err(B.int8w_fp8_gemv(fp8desc(fmt=7), x, y, 0))
    assert rc == B.INT8W_ERR_UNSUPPORTED and "scale_format" in msg
    for bs in (0, 32, 96, 2048):
        rc, msg = err(B.int8w_fp8_gemv(fp8desc(fmt=B.FP8_BLOCK_BF16, bs=bs), x, y, 0))
        assert rc == B.INT8W_ERR_UNSUPPORTED and "block_size" in msg
    # the tag decides what the scale must be
    assert err(B.int8w_fp8_gemv(fp8desc(scale=0), x, y, 0))[0] == B.INT8W_ERR_NULL
    assert err(B.int8w_fp8_gemv(fp8desc(fmt=B.FP8_BLOCK_F32, scale=0), x, y, 0))[0] == B.INT8W_ERR_NULL
    rc, msg = err(B.int8w_fp8_gemv(fp8desc(fmt=B.FP8_SINGLE), x, y, 0))
    assert rc == B.INT8W_ERR_SHAPE and "NULL" in msg
    assert err(B.int8w_fp8_gemv(fp8desc(scale=2 * A16 + 2), x, y, 0))[0] == B.INT8W_ERR_ALIGN
    assert err(B.int8w_fp8_gemv(fp8desc(fmt=B.FP8_BLOCK_F32, scale=2 * A16 + 2), x, y, 0))[0] == B.INT8W_ERR_ALIGN
    assert err(B.int8w_fp8_gemv(fp8desc(weight=A16 + 8), x, y, 0))[0] == B.INT8W_ERR_ALIGN
    assert err(B.int8w_fp8_gemv(fp8desc(), x + 8, y, 0))[0] == B.INT8W_ERR_ALIGN
    assert err(B.int8w_fp8_gemv(fp8desc(), x, y + 1, 0))[0] == B.INT8W_ERR_ALIGN
    assert err(B.int8w_fp8_gemv(fp8desc(), 0, y, 0))[0] == B.INT8W_ERR_NULL
    # y over the weight, the scale (its extent depends on the layout) or x
    rc, msg = err(B.int8w_fp8_gemv(fp8desc(), x, A16 + 64 * 256 - 2, 0))
    assert rc == B.INT8W_ERR_ALIAS and "weight" in msg
    rc, msg = err(B.int8w_fp8_gemv(fp8desc(), x, 2 * A16 + 64 * 4 - 2, 0))
    assert rc == B.INT8W_ERR_ALIAS and "scale" in msg
    rc, msg = err(B.int8w_fp8_gemv(fp8desc(fmt=B.FP8_BLOCK_BF16, n=300, k=528), x, 2 * A16 + 3 * 5 * 2 - 2, 0))
    assert rc == B.INT8W_ERR_ALIAS and "scale" in msg
    rc, msg = err(B.int8w_fp8_gemv(fp8desc(), x, x + 2 * 255, 0))
    assert rc == B.INT8W_ERR_ALIAS and "input x" in msg


def test_gemm_workspace_rules():
    d = desc(N=4096, K=14336, gs=64)
    need = B.int8_gemm_workspace_bytes(d, 512)
    assert need >= 4 * 64 * 4 * 32768  # m = 512 on a 4096-row weight: 4 parts of 64 tiles
    assert B.int8_gemm_workspace_bytes(d, 16) == 0 and B.int8_gemm_workspace_bytes(d, 2048) == 0
    X, Y, WS = 8 * A16, 64 * A16, 512 * A16
    rc, msg = err(B.int8_gemm_ws(d, X, Y, 512, 0, 0, 0))
    assert rc == B.INT8W_ERR_NULL and "workspace" in msg
    rc, msg = err(B.int8_gemm_ws(d, X, Y, 512, WS + 16, need, 0))
    assert rc == B.INT8W_ERR_ALIGN and "workspace" in msg
    rc, msg = err(B.int8_gemm_ws(d, X, Y, 512, WS, need - 1, 0))
    assert rc == B.INT8W_ERR_SHAPE and "needs" in msg
    rc, msg = err(B.int8_gemm_ws(d, X, Y, 512, X, need, 0))
    assert rc == B.INT8W_ERR_ALIAS and "workspace" in msg
