// launch.h -- internal host-side launchers of the gfx950 kernels (not part of
// the public C-ABI).  Arguments are already validated by capi.cpp; each
// launcher only sizes the grid and enqueues on `stream`.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "int8w.h"

namespace int8w {

struct WeightView {
  const uint32_t *packed;
  const uint16_t *scales;
  const uint16_t *biases;
  uint32_t N, K, gs;
};

// Number of compute units of the current device (cached per device).
int device_cu_count();

hipError_t launch_dequant(const WeightView &w, uint16_t *out, hipStream_t stream);

enum GemvEpilogue { kEpiNone = 0, kEpiSiluGate = 1, kEpiSiluGateResid = 2 };

// y = W a, with a = x (kEpiNone) or silu(gate)*up; plus x_resid for kEpiSiluGateResid.
// gemm with 2 <= m <= 4 rows of X on in_features 1024..4096 (a multiple of
// 1024): the register-resident gemv with several rows (gemv.hip).
bool gemv_rows_supported(uint32_t K, uint32_t m);
hipError_t launch_gemv_rows(const WeightView &w, const uint16_t *X, uint16_t *Y, uint32_t m, hipStream_t stream);
// gemm with m = 2 rows on in_features above 4096 (a multiple of 1024, up to
// 32768) where the small-m kernel is weakest (group size 32, or in_features
// above 16384): the same arithmetic with X's rows in LDS.
bool gemv_rows_lds_supported(uint32_t K, uint32_t gs, uint32_t m);
hipError_t launch_gemv_rows_lds(const WeightView &w, const uint16_t *X, uint16_t *Y, uint32_t m, hipStream_t stream);
hipError_t launch_gemv(const WeightView &w, GemvEpilogue epi, const uint16_t *x_or_gate,
                       const uint16_t *up, const uint16_t *x_resid, uint16_t *y, hipStream_t stream);

// y_i = W_i x for count (1..4) weights with the same K and group size, in one
// launch (each weight's rows streamed by its own share of the waves).
hipError_t launch_gemv_multi(const WeightView *w, uint16_t *const *y, uint32_t count, const uint16_t *x,
                             hipStream_t stream);

// Expert-indexed gemv: w holds E experts of [w.N / E, K] stacked along rows;
// y[p, :] = W_ids[p] x_row(p) for the tokens * topk slots p (x_row(p) is the
// token's row, or the slot's own when x_rows == topk).  ids are read on the
// device; a slot whose id is not below E gets NaN outputs.
hipError_t launch_moe_gemv(const WeightView &w, uint32_t E, const uint16_t *x, uint32_t x_rows, const uint32_t *ids,
                           uint32_t tokens, uint32_t topk, uint16_t *y, hipStream_t stream);

// y = W x for an FP8 E4M3 weight [N, K] (bytes, K a multiple of 16) with a
// per-row f32 scale [N], per-block BF16 or f32 scales [ceil(N/BS),
// ceil(K/BS)] (BS a power of two, 64..1024) or one global scale.
enum Fp8ScaleKind { kFp8PerRow = 0, kFp8BlockBf16 = 1, kFp8BlockF32 = 2, kFp8Single = 3 };
hipError_t launch_fp8_gemv(const uint8_t *codes, const void *scale, Fp8ScaleKind kind, uint32_t block_size,
                           float single, uint32_t N, uint32_t K, const uint16_t *x, uint16_t *y, hipStream_t stream);

// BF16 weight [N, K] -> codes (packed), scales, biases [N, K/gs] (affine min/max).
hipError_t launch_quantize(const uint16_t *w, uint32_t N, uint32_t K, uint32_t gs, uint32_t *packed, uint16_t *scales,
                           uint16_t *biases, hipStream_t stream);

// Y[m, N] = X[m, K] W^T for 2 <= m <= 16 (matrix cores, per-group rescale).
// Only for shapes where smallm_supported(K, gs) (the per-row scale/bias stage
// fits the LDS); others go to launch_gemm_prefill.
bool smallm_supported(uint32_t K, uint32_t gs);
hipError_t launch_gemm_smallm(const WeightView &w, const uint16_t *X, uint16_t *Y, uint32_t m,
                              hipStream_t stream);

// Y[m, N] = X[m, K] W^T for large m (weight tiles dequantized to BF16 in LDS).
// With a workspace (ws != nullptr, at least gemm_prefill_workspace_bytes; no
// initial value) a grid with too few tiles splits K over several work items
// per tile, whose fp32 partials a second launch adds in a fixed order;
// ws == nullptr never splits.
uint64_t gemm_prefill_workspace_bytes(const WeightView &w, uint32_t m);
hipError_t launch_gemm_prefill(const WeightView &w, const uint16_t *X, uint16_t *Y, uint32_t m, void *ws,
                               hipStream_t stream);

// The small-m kernel with two 16-row X tiles per pass (2 <= m <= 32), where
// smallm32_supported(K, gs) (its buffers and scale/bias rows fit the LDS).
bool smallm32_supported(uint32_t N, uint32_t K, uint32_t gs);
hipError_t launch_gemm_smallm32(const WeightView &w, const uint16_t *X, uint16_t *Y, uint32_t m,
                                hipStream_t stream);

// For 16 < m <= 128: the rows per small-m pass (32, or 16 where only the
// one-tile kernel fits) if passes over slices of X are expected to beat the
// tiled kernel (a grid of few tiles, each walking all of K; split over K
// when can_split), else 0.
uint32_t gemm_smallm_slice_rows(const WeightView &w, uint32_t m, bool can_split);

// Calibration streams (not part of the layer path): read `bytes` once, copy
// them, or widen each to 16 bits (2 * bytes written); bytes a multiple of 1024.
hipError_t launch_stream_read(const void *src, uint64_t bytes, uint32_t *sink, hipStream_t stream);
hipError_t launch_stream_copy(const void *src, void *dst, uint64_t bytes, hipStream_t stream);
hipError_t launch_stream_expand(const void *src, void *dst, uint64_t bytes, hipStream_t stream);

// ---- C-ABI internals shared by capi.cpp and noalloc.hip
// Records the calling thread's last error message and returns code.
int report_error(int code, const char *fmt, ...);
// int8_gemm / int8_gemm_ws: ws == nullptr never splits K.
int gemm_common(const int8w_weight *w, const uint16_t *x, uint16_t *y, uint32_t m, void *ws,
                uint64_t ws_bytes, uint64_t stream);

}  // namespace int8w
