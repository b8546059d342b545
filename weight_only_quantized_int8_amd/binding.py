"""Thin ctypes binding of libint8w.so (include/int8w.h).

Argument marshalling only: every computation runs in the library's HIP
kernels.  PyTorch provides device memory and the current stream.  If the
library has not been built, loading it raises -- there is no fallback.

The checks in :class:`Int8Weight` follow the rustdoc page "MlxInt8Weight",
method load: the weight must be a 2-D 32-bit tensor, scales and biases BF16
of shape [out_features, in_features / group_size], and group_size must divide
in_features.
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_PKG, "libint8w.so")

INT8W_OK = 0
INT8W_ERR_NULL = -1
INT8W_ERR_SHAPE = -2
INT8W_ERR_UNSUPPORTED = -3
INT8W_ERR_ALIGN = -4
INT8W_ERR_ALIAS = -5
INT8W_ERR_HIP = -6
ERROR_NAMES = {
    INT8W_ERR_NULL: "INT8W_ERR_NULL",
    INT8W_ERR_SHAPE: "INT8W_ERR_SHAPE",
    INT8W_ERR_UNSUPPORTED: "INT8W_ERR_UNSUPPORTED",
    INT8W_ERR_ALIGN: "INT8W_ERR_ALIGN",
    INT8W_ERR_ALIAS: "INT8W_ERR_ALIAS",
    INT8W_ERR_HIP: "INT8W_ERR_HIP",
}

EXPORTED = (
    "int8w_validate", "int8w_storage_bytes", "int8_dequantize_to", "int8_gemv", "int8_gemv_silu_gate",
    "int8_gemv_silu_gate_resid", "int8_gemm", "int8_gemv_multi", "int8_quantize", "int8_moe_gemv",
    "int8w_fp8_gemv", "int8w_last_error", "int8_gemm_workspace_bytes", "int8_gemm_ws", "int8_gemm_noalloc",
)
# calibration streams declared in include/int8w_measure.h
EXPORTED_MEASURE = ("int8w_stream_read", "int8w_stream_copy", "int8w_stream_expand")
FP8_PER_ROW, FP8_BLOCK_BF16, FP8_BLOCK_F32, FP8_SINGLE = 0, 1, 2, 3  # INT8W_FP8_*
MAX_MULTI = 4  # INT8W_MAX_MULTI
MAX_MOE_SLOTS = 65536  # INT8W_MAX_MOE_SLOTS


class Int8wError(RuntimeError):
    def __init__(self, code: int, message: str):
        super().__init__(f"{ERROR_NAMES.get(code, code)}: {message}")
        self.code = code
        self.message = message


class WeightDesc(ctypes.Structure):
    """Mirror of ``int8w_weight`` (include/int8w.h)."""
    _fields_ = [
        ("packed", ctypes.c_void_p),
        ("scales", ctypes.c_void_p),
        ("biases", ctypes.c_void_p),
        ("out_features", ctypes.c_uint32),
        ("in_features", ctypes.c_uint32),
        ("group_size", ctypes.c_uint32),
    ]


class Fp8WeightDesc(ctypes.Structure):
    """Mirror of ``int8w_fp8_weight`` (include/int8w.h)."""
    _fields_ = [
        ("weight", ctypes.c_void_p),
        ("scale", ctypes.c_void_p),
        ("n", ctypes.c_uint32),
        ("k", ctypes.c_uint32),
        ("scale_format", ctypes.c_uint32),
        ("block_size", ctypes.c_uint32),
        ("single_scale", ctypes.c_float),
    ]


_lib = None


def library_path() -> str:
    return _LIB_PATH


def load_library() -> ctypes.CDLL:
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(
            f"{_LIB_PATH} is not built; run `python -m weight_only_quantized_int8_amd.build` "
            "(the HIP library is required: there is no CPU fallback)")
    lib = ctypes.CDLL(_LIB_PATH)
    P = ctypes.c_void_p
    W = ctypes.POINTER(WeightDesc)
    u64 = ctypes.c_uint64
    lib.int8w_validate.argtypes = [W]
    lib.int8w_validate.restype = ctypes.c_int
    lib.int8w_storage_bytes.argtypes = [ctypes.c_uint32, ctypes.c_uint32, ctypes.c_uint32]
    lib.int8w_storage_bytes.restype = ctypes.c_uint64
    lib.int8_dequantize_to.argtypes = [W, P, u64]
    lib.int8_dequantize_to.restype = ctypes.c_int
    lib.int8_gemv.argtypes = [W, P, P, u64]
    lib.int8_gemv.restype = ctypes.c_int
    lib.int8_gemv_silu_gate.argtypes = [W, P, P, P, u64]
    lib.int8_gemv_silu_gate.restype = ctypes.c_int
    lib.int8_gemv_silu_gate_resid.argtypes = [W, P, P, P, P, u64]
    lib.int8_gemv_silu_gate_resid.restype = ctypes.c_int
    lib.int8_gemm.argtypes = [W, P, P, ctypes.c_uint32, u64]
    lib.int8_gemm.restype = ctypes.c_int
    lib.int8_gemv_multi.argtypes = [W, ctypes.c_uint32, P, ctypes.POINTER(P), u64]
    lib.int8_gemv_multi.restype = ctypes.c_int
    u32 = ctypes.c_uint32
    lib.int8_quantize.argtypes = [P, u32, u32, u32, P, P, P, u64]
    lib.int8_quantize.restype = ctypes.c_int
    lib.int8_moe_gemv.argtypes = [W, u32, P, u32, P, u32, u32, P, u64]
    lib.int8_moe_gemv.restype = ctypes.c_int
    lib.int8w_fp8_gemv.argtypes = [ctypes.POINTER(Fp8WeightDesc), P, P, u64]
    lib.int8w_fp8_gemv.restype = ctypes.c_int
    lib.int8_gemm_workspace_bytes.argtypes = [W, ctypes.c_uint32]
    lib.int8_gemm_workspace_bytes.restype = ctypes.c_uint64
    lib.int8_gemm_ws.argtypes = [W, P, P, ctypes.c_uint32, P, u64, u64]
    lib.int8_gemm_ws.restype = ctypes.c_int
    lib.int8_gemm_noalloc.argtypes = [W, P, P, ctypes.c_uint32, u64]
    lib.int8_gemm_noalloc.restype = ctypes.c_int
    lib.int8w_stream_read.argtypes = [P, u64, P, u64]
    lib.int8w_stream_read.restype = ctypes.c_int
    lib.int8w_stream_copy.argtypes = [P, P, u64, u64]
    lib.int8w_stream_copy.restype = ctypes.c_int
    lib.int8w_stream_expand.argtypes = [P, P, u64, u64]
    lib.int8w_stream_expand.restype = ctypes.c_int
    lib.int8w_last_error.argtypes = []
    lib.int8w_last_error.restype = ctypes.c_char_p
    _lib = lib
    return lib


def _check(rc: int) -> None:
    if rc != INT8W_OK:
        msg = load_library().int8w_last_error().decode(errors="replace")
        raise Int8wError(rc, msg)


def storage_bytes(out_features: int, in_features: int, group_size: int) -> int:
    return int(load_library().int8w_storage_bytes(out_features, in_features, group_size))


# ---- raw C-ABI calls (device addresses as ints, stream as int) --------------------------------

def int8w_validate(desc: WeightDesc) -> int:
    return load_library().int8w_validate(ctypes.byref(desc))


def int8_dequantize_to(desc: WeightDesc, out: int, stream: int) -> int:
    return load_library().int8_dequantize_to(ctypes.byref(desc), out, stream)


def int8_gemv(desc: WeightDesc, x: int, y: int, stream: int) -> int:
    return load_library().int8_gemv(ctypes.byref(desc), x, y, stream)


def int8_gemv_silu_gate(desc: WeightDesc, gate: int, up: int, y: int, stream: int) -> int:
    return load_library().int8_gemv_silu_gate(ctypes.byref(desc), gate, up, y, stream)


def int8_gemv_silu_gate_resid(desc: WeightDesc, gate: int, up: int, x_resid: int, y: int, stream: int) -> int:
    return load_library().int8_gemv_silu_gate_resid(ctypes.byref(desc), gate, up, x_resid, y, stream)


def int8_gemm(desc: WeightDesc, x: int, y: int, m: int, stream: int) -> int:
    return load_library().int8_gemm(ctypes.byref(desc), x, y, m, stream)


def int8_quantize(w: int, out_features: int, in_features: int, group_size: int, packed: int, scales: int,
                  biases: int, stream: int) -> int:
    return load_library().int8_quantize(w, out_features, in_features, group_size, packed, scales, biases, stream)


def int8_moe_gemv(desc: WeightDesc, num_experts: int, x: int, x_rows: int, ids: int, tokens: int, topk: int,
                  y: int, stream: int) -> int:
    return load_library().int8_moe_gemv(ctypes.byref(desc), num_experts, x, x_rows, ids, tokens, topk, y, stream)


def int8w_fp8_gemv(desc: Fp8WeightDesc, x: int, y: int, stream: int) -> int:
    return load_library().int8w_fp8_gemv(ctypes.byref(desc), x, y, stream)


def int8_gemm_workspace_bytes(desc: WeightDesc, m: int) -> int:
    return int(load_library().int8_gemm_workspace_bytes(ctypes.byref(desc), m))


def int8_gemm_ws(desc: WeightDesc, x: int, y: int, m: int, ws: int, ws_bytes: int, stream: int) -> int:
    return load_library().int8_gemm_ws(ctypes.byref(desc), x, y, m, ws, ws_bytes, stream)


def int8_gemm_noalloc(desc: WeightDesc, x: int, y: int, m: int, stream: int) -> int:
    return load_library().int8_gemm_noalloc(ctypes.byref(desc), x, y, m, stream)


NOALLOC_SCRATCH_BYTES = 64 << 20  # INT8W_NOALLOC_SCRATCH_BYTES


def int8w_stream_read(src: int, nbytes: int, sink: int, stream: int) -> int:
    return load_library().int8w_stream_read(src, nbytes, sink, stream)


def int8w_stream_copy(src: int, dst: int, nbytes: int, stream: int) -> int:
    return load_library().int8w_stream_copy(src, dst, nbytes, stream)


def int8w_stream_expand(src: int, dst: int, nbytes: int, stream: int) -> int:
    return load_library().int8w_stream_expand(src, dst, nbytes, stream)


def int8_gemv_multi(descs, x: int, ys, stream: int) -> int:
    """descs: sequence of WeightDesc; ys: sequence of device addresses (same length)."""
    n = len(descs)
    arr = (WeightDesc * max(n, 1))(*descs)
    yarr = (ctypes.c_void_p * max(n, 1))(*ys)
    return load_library().int8_gemv_multi(arr, n, x, yarr, stream)


# ---- tensor-level wrapper -----------------------------------------------------------------------

def _stream_of(device: torch.device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _need_bf16(t: torch.Tensor, name: str, numel: int, device: torch.device) -> None:
    if t.dtype != torch.bfloat16:
        raise TypeError(f"{name} must be bfloat16, got {t.dtype}")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, weight on {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.numel() < numel:
        raise ValueError(f"{name} holds {t.numel()} elements, needs {numel}")


class Int8Weight:
    """One 8-bit affine group-quantized weight on the GPU (borrowed tensors).

    packed:  int32/uint32 [out_features, in_features/4] (code k in byte k%4 of word k/4)
    scales:  bfloat16 [out_features, in_features/group_size]
    biases:  bfloat16 [out_features, in_features/group_size]
    The tensors stay owned by the caller (this object keeps references).
    """

    def __init__(self, packed: torch.Tensor, scales: torch.Tensor, biases: torch.Tensor, group_size: int):
        if packed.dim() != 2 or packed.dtype not in (torch.int32, torch.uint32):
            raise ValueError("weight must be a 2-D 32-bit (U32) tensor")
        if scales.dtype != torch.bfloat16 or biases.dtype != torch.bfloat16:
            raise ValueError("scales and biases must be bfloat16")
        N, kw = packed.shape
        K = 4 * kw
        gs = int(group_size)
        if gs <= 0 or K % gs:
            raise ValueError(f"group_size {gs} does not divide in_features {K}")
        G = K // gs
        if tuple(scales.shape) != (N, G) or tuple(biases.shape) != (N, G):
            raise ValueError(f"scales/biases must be [{N}, {G}] = [out_features, in_features/group_size]")
        for t, name in ((packed, "packed"), (scales, "scales"), (biases, "biases")):
            if not t.is_contiguous():
                raise ValueError(f"{name} must be contiguous")
        if not (packed.device == scales.device == biases.device) or packed.device.type != "cuda":
            raise ValueError("packed, scales and biases must be on one GPU")
        self.packed, self.scales, self.biases = packed, scales, biases
        self.out_features, self.in_features, self.group_size = N, K, gs
        self.device = packed.device
        self.desc = WeightDesc(packed.data_ptr(), scales.data_ptr(), biases.data_ptr(), N, K, gs)
        _check(int8w_validate(self.desc))

    @classmethod
    def quantize(cls, w: torch.Tensor, group_size: int) -> "Int8Weight":
        """Encode a BF16 weight [out_features, in_features] on the GPU (int8_quantize)."""
        if w.dtype != torch.bfloat16 or w.dim() != 2 or not w.is_contiguous() or w.device.type != "cuda":
            raise ValueError("w must be a contiguous 2-D bfloat16 GPU tensor")
        N, K = w.shape
        gs = int(group_size)
        if gs <= 0 or K % gs or K % 4:
            raise ValueError(f"group_size {gs} must divide in_features {K} (a multiple of 4)")
        packed = torch.empty((N, K // 4), dtype=torch.int32, device=w.device)
        scales = torch.empty((N, K // gs), dtype=torch.bfloat16, device=w.device)
        biases = torch.empty((N, K // gs), dtype=torch.bfloat16, device=w.device)
        _check(int8_quantize(w.data_ptr(), N, K, gs, packed.data_ptr(), scales.data_ptr(), biases.data_ptr(),
                             _stream_of(w.device)))
        return cls(packed, scales, biases, gs)

    @classmethod
    def from_arrays(cls, packed, scales_bits, biases_bits, group_size: int, device="cuda") -> "Int8Weight":
        """Upload NumPy arrays (uint32 words, uint16 BF16 bit patterns)."""
        import numpy as np
        p = torch.from_numpy(np.ascontiguousarray(packed).view(np.int32)).to(device)
        s = torch.from_numpy(np.ascontiguousarray(scales_bits).view(np.int16)).view(torch.bfloat16).to(device)
        b = torch.from_numpy(np.ascontiguousarray(biases_bits).view(np.int16)).view(torch.bfloat16).to(device)
        return cls(p, s, b, group_size)

    def storage_bytes(self) -> int:
        return storage_bytes(self.out_features, self.in_features, self.group_size)

    def dequantize_to(self, out: torch.Tensor | None = None) -> torch.Tensor:
        N, K = self.out_features, self.in_features
        if out is None:
            out = torch.empty((N, K), dtype=torch.bfloat16, device=self.device)
        _need_bf16(out, "out", N * K, self.device)
        _check(int8_dequantize_to(self.desc, out.data_ptr(), _stream_of(self.device)))
        return out

    def gemv(self, x: torch.Tensor, y: torch.Tensor | None = None) -> torch.Tensor:
        _need_bf16(x, "x", self.in_features, self.device)
        if y is None:
            y = torch.empty(self.out_features, dtype=torch.bfloat16, device=self.device)
        _need_bf16(y, "y", self.out_features, self.device)
        _check(int8_gemv(self.desc, x.data_ptr(), y.data_ptr(), _stream_of(self.device)))
        return y

    def gemv_silu_gate(self, gate: torch.Tensor, up: torch.Tensor, y: torch.Tensor | None = None) -> torch.Tensor:
        _need_bf16(gate, "gate", self.in_features, self.device)
        _need_bf16(up, "up", self.in_features, self.device)
        if y is None:
            y = torch.empty(self.out_features, dtype=torch.bfloat16, device=self.device)
        _need_bf16(y, "y", self.out_features, self.device)
        _check(int8_gemv_silu_gate(self.desc, gate.data_ptr(), up.data_ptr(), y.data_ptr(), _stream_of(self.device)))
        return y

    def gemv_silu_gate_resid(self, gate: torch.Tensor, up: torch.Tensor, x_resid: torch.Tensor,
                             y: torch.Tensor | None = None) -> torch.Tensor:
        _need_bf16(gate, "gate", self.in_features, self.device)
        _need_bf16(up, "up", self.in_features, self.device)
        _need_bf16(x_resid, "x_resid", self.out_features, self.device)
        if y is None:
            y = torch.empty(self.out_features, dtype=torch.bfloat16, device=self.device)
        _need_bf16(y, "y", self.out_features, self.device)
        _check(int8_gemv_silu_gate_resid(self.desc, gate.data_ptr(), up.data_ptr(), x_resid.data_ptr(),
                                         y.data_ptr(), _stream_of(self.device)))
        return y

    def gemm(self, x: torch.Tensor, y: torch.Tensor | None = None, split_k: bool = True) -> torch.Tensor:
        """Y = X W^T.  With split_k (the default) a call whose grid has too few
        tiles runs int8_gemm_ws on a cached per-device workspace (int8_gemm_noalloc
        when that would have to grow during graph capture); otherwise int8_gemm."""
        if x.dim() != 2 or x.shape[1] != self.in_features:
            raise ValueError(f"X must be [m, {self.in_features}]")
        m = x.shape[0]
        _need_bf16(x, "X", m * self.in_features, self.device)
        if y is None:
            y = torch.empty((m, self.out_features), dtype=torch.bfloat16, device=self.device)
        _need_bf16(y, "Y", m * self.out_features, self.device)
        need = int8_gemm_workspace_bytes(self.desc, m) if split_k and m > 16 else 0
        stream = _stream_of(self.device)
        ws = _workspace(self.device, need) if need else None
        if ws is not None:
            _check(int8_gemm_ws(self.desc, x.data_ptr(), y.data_ptr(), m, ws.data_ptr(), ws.numel(), stream))
        elif need and need <= NOALLOC_SCRATCH_BYTES:
            # under graph capture, where the cached workspace may not grow: the
            # library's static scratch, same kernels and bits
            _check(int8_gemm_noalloc(self.desc, x.data_ptr(), y.data_ptr(), m, stream))
        else:
            _check(int8_gemm(self.desc, x.data_ptr(), y.data_ptr(), m, stream))
        return y


# One gemm workspace per device (scratch for split-K partials), grown on
# demand.  Calls that use it are ordered on the caller's stream; overlapping
# calls on several streams of one device would share it and race.
_workspaces: dict = {}


def _workspace(device: torch.device, nbytes: int):
    """The device's cached workspace of at least nbytes, grown if needed; None
    when it would have to grow while the current stream is being captured into
    a graph (an allocation made then would come from the graph's pool)."""
    key = device.index if device.index is not None else torch.cuda.current_device()
    ws = _workspaces.get(key)
    if ws is None or ws.numel() < nbytes:
        if torch.cuda.is_current_stream_capturing():
            return None
        ws = torch.empty(max(nbytes, 64 << 20), dtype=torch.uint8, device=device)
        _workspaces[key] = ws
    return ws


def gemv_multi(weights, x: torch.Tensor, ys=None):
    """y_i = W_i x for up to four Int8Weight sharing in_features and group_size, in one launch."""
    weights = list(weights)
    if not weights:
        raise ValueError("gemv_multi needs at least one weight")
    dev = weights[0].device
    _need_bf16(x, "x", weights[0].in_features, dev)
    if ys is None:
        ys = [torch.empty(w.out_features, dtype=torch.bfloat16, device=dev) for w in weights]
    ys = list(ys)
    if len(ys) != len(weights):
        raise ValueError("gemv_multi: one output per weight")
    for w, y in zip(weights, ys):
        if w.device != dev:
            raise ValueError("gemv_multi: weights on different devices")
        _need_bf16(y, "y", w.out_features, dev)
    _check(int8_gemv_multi([w.desc for w in weights], x.data_ptr(), [y.data_ptr() for y in ys], _stream_of(dev)))
    return ys


def moe_gemv(experts: Int8Weight, num_experts: int, x: torch.Tensor, ids: torch.Tensor, y=None):
    """Expert-indexed gemv (int8_moe_gemv).

    experts: E = num_experts experts of [N, K] stacked along rows (out_features = E*N)
    x:       bfloat16 [tokens, 1 or topk, K]
    ids:     int32/uint32 [tokens, topk] on the GPU (expert of each slot)
    returns  bfloat16 [tokens, topk, N]; a slot whose id is not below E is NaN
    """
    dev = experts.device
    E = int(num_experts)
    if E <= 0 or experts.out_features % E:
        raise ValueError(f"{experts.out_features} rows are not a whole number of {E} experts")
    N, K = experts.out_features // E, experts.in_features
    if ids.dim() != 2 or ids.dtype not in (torch.int32, torch.uint32) or ids.device != dev or not ids.is_contiguous():
        raise ValueError("ids must be a contiguous 32-bit [tokens, topk] tensor on the weight's GPU")
    T, topk = ids.shape
    if x.dim() != 3 or x.shape[0] != T or x.shape[2] != K or x.shape[1] not in (1, topk):
        raise ValueError(f"x must be [{T}, 1 or {topk}, {K}]")
    _need_bf16(x, "x", x.numel(), dev)
    if y is None:
        y = torch.empty((T, topk, N), dtype=torch.bfloat16, device=dev)
    _need_bf16(y, "y", T * topk * N, dev)
    _check(int8_moe_gemv(experts.desc, E, x.data_ptr(), x.shape[1], ids.data_ptr(), T, topk, y.data_ptr(),
                         _stream_of(dev)))
    return y


class Fp8Weight:
    """An FP8 E4M3 weight on the GPU (borrowed tensors), after the rustdoc page "Fp8Weight".

    weight: uint8 [n, k] E4M3 bytes (k a multiple of 16)
    scale:  float32 [n] (FP8_PER_ROW); bfloat16 or float32 [ceil(n/BS), ceil(k/BS)]
            (FP8_BLOCK_BF16 / FP8_BLOCK_F32); None (FP8_SINGLE, with single_scale)
    """

    def __init__(self, weight: torch.Tensor, scale, scale_format: int, block_size: int = 128,
                 single_scale: float = 1.0):
        if weight.dim() != 2 or weight.dtype != torch.uint8 or not weight.is_contiguous():
            raise ValueError("weight must be a contiguous 2-D uint8 tensor of E4M3 bytes")
        if weight.device.type != "cuda":
            raise ValueError("weight must be on a GPU")
        n, k = weight.shape
        fmt = int(scale_format)
        if fmt == FP8_SINGLE:
            if scale is not None:
                raise ValueError("FP8_SINGLE takes no scale tensor")
        else:
            want = {FP8_PER_ROW: torch.float32, FP8_BLOCK_BF16: torch.bfloat16, FP8_BLOCK_F32: torch.float32}.get(fmt)
            if want is None:
                raise ValueError(f"unknown scale format {fmt}")
            if scale is None or scale.dtype != want or scale.device != weight.device or not scale.is_contiguous():
                raise ValueError(f"scale must be a contiguous {want} tensor on the weight's GPU")
            bs = int(block_size)
            shape = (n,) if fmt == FP8_PER_ROW else (-(-n // bs), -(-k // bs))
            if tuple(scale.shape) != shape:
                raise ValueError(f"scale must have shape {shape}")
        self.weight, self.scale = weight, scale
        self.n, self.k, self.scale_format = n, k, fmt
        self.device = weight.device
        self.desc = Fp8WeightDesc(weight.data_ptr(), scale.data_ptr() if scale is not None else None, n, k, fmt,
                                  int(block_size), float(single_scale))

    def gemv(self, x: torch.Tensor, y: torch.Tensor | None = None) -> torch.Tensor:
        _need_bf16(x, "x", self.k, self.device)
        if y is None:
            y = torch.empty(self.n, dtype=torch.bfloat16, device=self.device)
        _need_bf16(y, "y", self.n, self.device)
        _check(int8w_fp8_gemv(self.desc, x.data_ptr(), y.data_ptr(), _stream_of(self.device)))
        return y
