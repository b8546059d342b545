"""CPU oracle for 8-bit affine group-quantized weight-only linear layers.

TEST INFRASTRUCTURE ONLY.  Only the test-suite, the smoke check and the CPU
baseline leg of the benchmark may import this package.  The library under test
never does, and this package imports nothing from it.

The arithmetic lives in ``int8w_oracle.c`` (plain C, fp32 dequant, fp64 sums);
this module only marshals NumPy arrays through ctypes.  Each function follows
the rustdoc page "MlxInt8Weight" (metrale_gpu_runtime::mlx_int8): the struct
description ("8-bit affine", no Drop), the packed/scales/biases field sections
and the methods dequantize_to, gemv, gemv_silu_gate, gemv_silu_gate_resid and
gemm.  ``quantize`` (BF16 weight -> codes, scales, biases) follows the rustdoc
page of the DynQuantizedStorage trait, method quantize, which gives no formula:
its reading (affine min/max in fp32) is stated in ``int8w_oracle.c``.
``moe_gemv`` (expert-indexed products) follows the same trait page, provided
method indexed_moe_forward, which gives only a signature; its reading (stacked
experts, per-slot ids, NaN for an id with no expert) is stated in
``int8w_oracle.c``.  ``fp8_gemv`` follows the rustdoc page "Fp8Weight" (E4M3
bytes with per-row, per-block or single scales); its readings are stated in
``int8w_oracle.c``.  Readings the MlxInt8Weight page leaves open (byte order,
signedness, precision, rounding, silu) are stated in ``int8w_oracle.c``'s
header.

Pins: every function is checked against something other than itself in
``tests/test_oracle_pins.py`` (library routines, exact rational arithmetic,
closed forms and hand-computed examples).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "int8w_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle_int8w.so")

CFLAGS = ["-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp", "-fPIC", "-shared", "-std=c99"]


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (no fast-math, no FMA contraction)."""
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        tmp = _LIB_PATH + ".tmp"
        subprocess.run(["gcc", *CFLAGS, _SRC, "-o", tmp, "-lm"], check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


_lib = None


def _load():
    global _lib
    if _lib is None:
        build(force=False)
        lib = ctypes.CDLL(_LIB_PATH)
        p = ctypes.c_void_p
        i64 = ctypes.c_int64
        lib.orc_bf16_to_f32.argtypes = [ctypes.c_uint16]
        lib.orc_bf16_to_f32.restype = ctypes.c_float
        lib.orc_f32_to_bf16_rne.argtypes = [ctypes.c_float]
        lib.orc_f32_to_bf16_rne.restype = ctypes.c_uint16
        lib.orc_f32_to_bf16_rne_array.argtypes = [p, p, i64]
        lib.orc_unpack.argtypes = [p, i64, p]
        lib.orc_weight_f32.argtypes = [p, p, p, i64, i64, i64, p]
        lib.orc_dequantize_to.argtypes = [p, p, p, i64, i64, i64, p]
        lib.orc_matmul_act_f64.argtypes = [p, p, p, i64, i64, i64, p, i64, p, p]
        lib.orc_gemm.argtypes = [p, p, p, i64, i64, i64, p, i64, p, p]
        lib.orc_gemv.argtypes = [p, p, p, i64, i64, i64, p, p, p]
        lib.orc_silu_gate_act.argtypes = [p, p, i64, p]
        lib.orc_gemv_silu_gate.argtypes = [p, p, p, i64, i64, i64, p, p, p, p]
        lib.orc_gemv_silu_gate_resid.argtypes = [p, p, p, i64, i64, i64, p, p, p, p, p]
        lib.orc_quantize.argtypes = [p, i64, i64, i64, p, p, p]
        lib.orc_e4m3_to_f64.argtypes = [ctypes.c_uint8]
        lib.orc_e4m3_to_f64.restype = ctypes.c_double
        lib.orc_fp8_gemv.argtypes = [p, p, i64, i64, ctypes.c_int, i64, ctypes.c_double, p, p, p]
        lib.orc_moe_gemv.argtypes = [p, p, p, i64, i64, i64, i64, p, i64, p, i64, i64, p, p]
        lib.orc_max_threads.restype = ctypes.c_int
        lib.orc_set_threads.argtypes = [ctypes.c_int]
        lib.orc_set_threads.restype = None
        _lib = lib
    return _lib


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype) -> np.ndarray:
    a = np.ascontiguousarray(a)
    if a.dtype != dtype:
        a = a.view(dtype) if a.dtype.itemsize == np.dtype(dtype).itemsize else a.astype(dtype)
    return a


def _weight(packed, scales, biases, group_size):
    packed = _c(packed, np.uint32)
    scales = _c(scales, np.uint16)
    biases = _c(biases, np.uint16)
    N, kw = packed.shape
    K = 4 * kw
    gs = int(group_size)
    if gs <= 0 or K % gs:
        raise ValueError(f"group_size {gs} does not divide in_features {K}")
    if scales.shape != (N, K // gs) or biases.shape != (N, K // gs):
        raise ValueError("scales/biases must be [out_features, in_features/group_size]")
    return packed, scales, biases, N, K, gs


def max_threads() -> int:
    return int(_load().orc_max_threads())


def set_threads(n: int) -> None:
    """OpenMP threads for the oracle's row loops (results are the same for any count)."""
    _load().orc_set_threads(int(n))


def bf16_to_f32(bits) -> np.ndarray:
    """BF16 bit patterns -> float32 (exact widening)."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def f32_to_bf16(values) -> np.ndarray:
    """float32 -> BF16 bit patterns, round to nearest, ties to even."""
    f = np.ascontiguousarray(values, dtype=np.float32)
    out = np.empty(f.shape, dtype=np.uint16)
    _load().orc_f32_to_bf16_rne_array(_ptr(f), _ptr(out), f.size)
    return out


def unpack(packed) -> np.ndarray:
    """uint32 words -> uint8 codes, code 4*i+j = byte j of word i (LSB first)."""
    p = _c(packed, np.uint32)
    codes = np.empty(p.shape[:-1] + (p.shape[-1] * 4,), dtype=np.uint8)
    _load().orc_unpack(_ptr(p), p.size, _ptr(codes))
    return codes


def weight_f32(packed, scales, biases, group_size) -> np.ndarray:
    """fp32 affine weights [N, K]: q*scale + bias per group."""
    packed, scales, biases, N, K, gs = _weight(packed, scales, biases, group_size)
    w = np.empty((N, K), dtype=np.float32)
    _load().orc_weight_f32(_ptr(packed), _ptr(scales), _ptr(biases), N, K, gs, _ptr(w))
    return w


def dequantize_to(packed, scales, biases, group_size) -> np.ndarray:
    """The full dequantized weight as BF16 bit patterns [N, K]."""
    packed, scales, biases, N, K, gs = _weight(packed, scales, biases, group_size)
    out = np.empty((N, K), dtype=np.uint16)
    _load().orc_dequantize_to(_ptr(packed), _ptr(scales), _ptr(biases), N, K, gs, _ptr(out))
    return out


def matmul_act(packed, scales, biases, group_size, act_f64):
    """Y[i,n] = sum_k w[n,k] a[i,k] for fp64 activations a [m,K]; returns (Y, A)."""
    packed, scales, biases, N, K, gs = _weight(packed, scales, biases, group_size)
    a = np.ascontiguousarray(act_f64, dtype=np.float64)
    if a.ndim == 1:
        a = a[None, :]
    m = a.shape[0]
    if a.shape[1] != K:
        raise ValueError("activation width must equal in_features")
    Y = np.empty((m, N), dtype=np.float64)
    A = np.empty((m, N), dtype=np.float64)
    _load().orc_matmul_act_f64(_ptr(packed), _ptr(scales), _ptr(biases), N, K, gs, _ptr(a), m, _ptr(Y), _ptr(A))
    return Y, A


def gemm(packed, scales, biases, group_size, X):
    """Y = X W^T for BF16 X [m, K]; returns fp64 (Y [m,N], A [m,N])."""
    packed, scales, biases, N, K, gs = _weight(packed, scales, biases, group_size)
    X = _c(X, np.uint16)
    if X.ndim == 1:
        X = X[None, :]
    m = X.shape[0]
    if X.shape[1] != K:
        raise ValueError("X must be [m, in_features]")
    Y = np.empty((m, N), dtype=np.float64)
    A = np.empty((m, N), dtype=np.float64)
    _load().orc_gemm(_ptr(packed), _ptr(scales), _ptr(biases), N, K, gs, _ptr(X), m, _ptr(Y), _ptr(A))
    return Y, A


def gemv(packed, scales, biases, group_size, x):
    """y = W x for BF16 x [K]; returns fp64 (y [N], A [N])."""
    Y, A = gemm(packed, scales, biases, group_size, np.asarray(x).reshape(1, -1))
    return Y[0], A[0]


def silu_gate_act(gate, up) -> np.ndarray:
    """fp64 silu(gate) * up for BF16 gate, up [K]."""
    g = _c(gate, np.uint16).ravel()
    u = _c(up, np.uint16).ravel()
    if g.size != u.size:
        raise ValueError("gate and up must have the same length")
    a = np.empty(g.size, dtype=np.float64)
    _load().orc_silu_gate_act(_ptr(g), _ptr(u), g.size, _ptr(a))
    return a


def gemv_silu_gate(packed, scales, biases, group_size, gate, up):
    """y = W (silu(gate) * up); returns fp64 (y [N], A [N])."""
    packed, scales, biases, N, K, gs = _weight(packed, scales, biases, group_size)
    g = _c(gate, np.uint16).ravel()
    u = _c(up, np.uint16).ravel()
    if g.size != K or u.size != K:
        raise ValueError("gate/up must be [in_features]")
    y = np.empty(N, dtype=np.float64)
    A = np.empty(N, dtype=np.float64)
    _load().orc_gemv_silu_gate(_ptr(packed), _ptr(scales), _ptr(biases), N, K, gs, _ptr(g), _ptr(u), _ptr(y), _ptr(A))
    return y, A


def gemv_silu_gate_resid(packed, scales, biases, group_size, gate, up, x_resid):
    """y[n] = x_resid[n] + sum_k W[n,k] silu(gate[k]) up[k]; returns fp64 (y, A)."""
    packed, scales, biases, N, K, gs = _weight(packed, scales, biases, group_size)
    g = _c(gate, np.uint16).ravel()
    u = _c(up, np.uint16).ravel()
    r = _c(x_resid, np.uint16).ravel()
    if g.size != K or u.size != K or r.size != N:
        raise ValueError("gate/up must be [in_features], x_resid [out_features]")
    y = np.empty(N, dtype=np.float64)
    A = np.empty(N, dtype=np.float64)
    _load().orc_gemv_silu_gate_resid(_ptr(packed), _ptr(scales), _ptr(biases), N, K, gs, _ptr(g), _ptr(u), _ptr(r),
                                     _ptr(y), _ptr(A))
    return y, A


def quantize(w_bits, group_size):
    """BF16 weight [N, K] (bit patterns) -> (packed uint32 [N, K/4], scales, biases BF16 bits [N, K/gs]).

    The plain affine min/max quantizer (see orc_quantize for the exact steps)."""
    w = _c(w_bits, np.uint16)
    if w.ndim != 2:
        raise ValueError("weight must be 2-D [out_features, in_features]")
    N, K = w.shape
    gs = int(group_size)
    if gs <= 0 or K % gs or K % 4:
        raise ValueError(f"group_size {gs} must divide in_features {K} (a multiple of 4)")
    packed = np.zeros((N, K // 4), np.uint32)
    scales = np.zeros((N, K // gs), np.uint16)
    biases = np.zeros((N, K // gs), np.uint16)
    _load().orc_quantize(_ptr(w), N, K, gs, _ptr(packed), _ptr(scales), _ptr(biases))
    return packed, scales, biases


def moe_gemv(packed, scales, biases, group_size, num_experts, x, ids):
    """Expert-indexed products (see orc_moe_gemv for the reading).

    packed [E*N, K/4], scales/biases [E*N, K/gs] hold E = num_experts stacked
    experts; x is BF16 [T, S, K] with S = 1 or topk; ids is uint32 [T, topk].
    Returns fp64 (y [T, topk, N], A [T, topk, N]); a slot whose id is not below
    E gets NaN outputs (A = 0)."""
    packed, scales, biases, EN, K, gs = _weight(packed, scales, biases, group_size)
    E = int(num_experts)
    if E <= 0 or EN % E:
        raise ValueError(f"{EN} stacked rows are not a whole number of {E} experts")
    N = EN // E
    ids = _c(ids, np.uint32)
    if ids.ndim != 2:
        raise ValueError("ids must be [tokens, topk]")
    T, topk = ids.shape
    x = _c(x, np.uint16)
    if x.ndim != 3 or x.shape[0] != T or x.shape[2] != K or x.shape[1] not in (1, topk):
        raise ValueError("x must be [tokens, 1 or topk, in_features]")
    S = x.shape[1]
    y = np.empty((T, topk, N), dtype=np.float64)
    A = np.empty((T, topk, N), dtype=np.float64)
    _load().orc_moe_gemv(_ptr(packed), _ptr(scales), _ptr(biases), E, N, K, gs, _ptr(x), S, _ptr(ids), T, topk,
                         _ptr(y), _ptr(A))
    return y, A


FP8_PER_ROW, FP8_BLOCK_BF16, FP8_BLOCK_F32, FP8_SINGLE = 0, 1, 2, 3


def e4m3_to_f64(codes) -> np.ndarray:
    """E4M3 bytes -> fp64 values (NaN for 0x7F / 0xFF); see orc_e4m3_to_f64."""
    c = np.ascontiguousarray(codes, dtype=np.uint8)
    lib = _load()
    table = np.array([lib.orc_e4m3_to_f64(i) for i in range(256)], dtype=np.float64)
    return table[c]


def fp8_gemv(weight, scale, scale_format, x, block_size=128, single_scale=1.0):
    """y = W x for an FP8 E4M3 weight [N, K] (uint8 bytes) with one of the
    three scale layouts of the rustdoc page "Fp8Weight"; returns fp64 (y, A).

    scale: float32 [N] (FP8_PER_ROW), BF16 bit patterns [ceil(N/BS), ceil(K/BS)]
    (FP8_BLOCK_BF16), float32 of that shape (FP8_BLOCK_F32), or None with
    single_scale (FP8_SINGLE)."""
    w = _c(weight, np.uint8)
    if w.ndim != 2:
        raise ValueError("weight must be [N, K] bytes")
    N, K = w.shape
    bs = int(block_size)
    fmt = int(scale_format)
    nb, kb = -(-N // bs), -(-K // bs)
    if fmt == FP8_PER_ROW:
        sc = _c(scale, np.float32).reshape(-1)
        if sc.size != N:
            raise ValueError("per-row scale must be [N] f32")
    elif fmt in (FP8_BLOCK_BF16, FP8_BLOCK_F32):
        sc = _c(scale, np.uint16 if fmt == FP8_BLOCK_BF16 else np.float32)
        if sc.shape != (nb, kb):
            raise ValueError(f"block scale must be [{nb}, {kb}]")
    elif fmt == FP8_SINGLE:
        sc = np.zeros(1, np.float32)
    else:
        raise ValueError(f"unknown scale format {fmt}")
    x = _c(x, np.uint16).reshape(-1)
    if x.size != K:
        raise ValueError("x must be [K]")
    y = np.empty(N, dtype=np.float64)
    A = np.empty(N, dtype=np.float64)
    _load().orc_fp8_gemv(_ptr(w), _ptr(sc), N, K, fmt, bs, float(np.float32(single_scale)), _ptr(x), _ptr(y), _ptr(A))
    return y, A


def within_tolerance(y_bf16_bits, y_ref, A, rel: float = 8e-3, absA: float = 2e-3) -> np.ndarray:
    """Acceptance for products: |y - y_ref| <= rel*|y_ref| + absA*A, and y finite."""
    y = bf16_to_f32(y_bf16_bits).astype(np.float64)
    ok = np.isfinite(y) & (np.abs(y - y_ref) <= rel * np.abs(y_ref) + absA * A)
    return ok
