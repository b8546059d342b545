"""MI355X-native 8-bit affine group-quantized weight-only linear layers.

The layers follow the rustdoc page "MlxInt8Weight" (metrale_gpu_runtime::
mlx_int8): a weight is packed uint32 words [out_features, in_features/4] of
uint8 codes with per-group BF16 scales and biases [out_features,
in_features/group_size], and w = q*scale + bias.  Every operation runs in
hand-written HIP kernels for gfx950, reached through the C-ABI library
``libint8w.so`` (declared in include/int8w.h); this package only marshals
arguments.  There is no CPU fallback: calls fail when the library is missing.
"""
from .binding import (Fp8Weight, Int8Weight, Int8wError, gemv_multi, library_path, load_library,  # noqa: F401
                      moe_gemv, storage_bytes)
