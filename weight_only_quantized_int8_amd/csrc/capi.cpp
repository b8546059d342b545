// capi.cpp -- the C-ABI of libint8w (declared in include/int8w.h).
//
// Host-side only: argument validation (the rules the rustdoc page
// "MlxInt8Weight" gives for its load method, plus alignment, aliasing and
// size checks), choice of kernel by the number of input rows, and launch on
// the caller's stream.  Nothing here allocates or frees device memory.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>

#include "int8w.h"
#include "int8w_measure.h"
#include "launch.h"

namespace int8w {

namespace {

thread_local char g_last_error[512] = "";

int fail(int code, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
  va_end(ap);
  return code;
}

int ok() {
  g_last_error[0] = '\0';
  return INT8W_OK;
}

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

struct Range {
  const char *name;
  uintptr_t lo, hi;  // [lo, hi)
};

Range range(const char *name, const void *p, uint64_t bytes) {
  uintptr_t lo = reinterpret_cast<uintptr_t>(p);
  return Range{name, lo, lo + (uintptr_t)bytes};
}

bool overlaps(const Range &a, const Range &b) { return a.lo < b.hi && b.lo < a.hi; }

// Output `out` must not overlap any of the inputs.
int check_alias(const Range &out, const Range *ins, int n_ins) {
  for (int i = 0; i < n_ins; ++i)
    if (ins[i].hi > ins[i].lo && overlaps(out, ins[i]))
      return fail(INT8W_ERR_ALIAS, "output %s overlaps input %s", out.name, ins[i].name);
  return INT8W_OK;
}

int validate(const int8w_weight *w) {
  if (!w) return fail(INT8W_ERR_NULL, "weight descriptor is NULL");
  if (!w->packed || !w->scales || !w->biases)
    return fail(INT8W_ERR_NULL, "weight is missing a tensor (packed, scales or biases is NULL)");
  if (w->out_features == 0 || w->in_features == 0 || w->group_size == 0)
    return fail(INT8W_ERR_SHAPE, "zero dimension (out_features=%u in_features=%u group_size=%u)",
                w->out_features, w->in_features, w->group_size);
  if (w->in_features % w->group_size != 0)
    return fail(INT8W_ERR_SHAPE, "group_size %u does not divide in_features %u", w->group_size, w->in_features);
  if (w->in_features % 4 != 0)
    return fail(INT8W_ERR_SHAPE, "in_features %u is not a whole number of 4-code words", w->in_features);
  if (w->group_size != 32 && w->group_size != 64 && w->group_size != 128)
    return fail(INT8W_ERR_UNSUPPORTED, "group_size %u not supported (32, 64 or 128)", w->group_size);
  // Code runs are indexed with 32-bit integers, and per-wave buffer windows
  // (a few rows) must stay below 2^31 bytes.
  if ((uint64_t)w->out_features * (w->in_features / 16u) > 0x7FFFFFFFull || w->in_features > (1u << 24))
    return fail(INT8W_ERR_SHAPE, "weight too large (%u x %u codes)", w->out_features, w->in_features);
  if (!aligned(w->packed, 16)) return fail(INT8W_ERR_ALIGN, "packed is not 16-byte aligned");
  if (!aligned(w->scales, 2) || !aligned(w->biases, 2))
    return fail(INT8W_ERR_ALIGN, "scales/biases are not 2-byte aligned");
  return INT8W_OK;
}

WeightView view(const int8w_weight *w) {
  return WeightView{w->packed, w->scales, w->biases, w->out_features, w->in_features, w->group_size};
}

void weight_ranges(const int8w_weight *w, Range *r) {
  const uint64_t N = w->out_features, K = w->in_features, G = K / w->group_size;
  r[0] = range("packed", w->packed, N * K);
  r[1] = range("scales", w->scales, N * G * 2);
  r[2] = range("biases", w->biases, N * G * 2);
}

int finish_launch(hipError_t e, hipStream_t stream) {
  if (e != hipSuccess) return fail(INT8W_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
  static const bool sync_check = [] {
    const char *v = getenv("INT8W_SYNC_CHECK");
    return v && v[0] && v[0] != '0';
  }();
  if (sync_check) {
    e = hipStreamSynchronize(stream);
    if (e != hipSuccess) return fail(INT8W_ERR_HIP, "kernel execution failed: %s", hipGetErrorString(e));
  }
  return ok();
}

hipStream_t as_stream(uint64_t s) { return reinterpret_cast<hipStream_t>(static_cast<uintptr_t>(s)); }

}  // namespace

int device_cu_count() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

}  // namespace int8w

using namespace int8w;

extern "C" {

int int8w_validate(const int8w_weight *w) {
  int rc = validate(w);
  return rc == INT8W_OK ? ok() : rc;
}

uint64_t int8w_storage_bytes(uint32_t out_features, uint32_t in_features, uint32_t group_size) {
  if (out_features == 0 || in_features == 0 || group_size == 0 || in_features % group_size) return 0;
  const uint64_t N = out_features, K = in_features;
  return N * K + 4ull * N * (K / group_size);
}

int int8_dequantize_to(const int8w_weight *w, uint16_t *out, uint64_t stream) {
  int rc = validate(w);
  if (rc) return rc;
  if (!out) return fail(INT8W_ERR_NULL, "out is NULL");
  if (!aligned(out, 16)) return fail(INT8W_ERR_ALIGN, "out is not 16-byte aligned");
  Range ins[3];
  weight_ranges(w, ins);
  rc = check_alias(range("out", out, (uint64_t)w->out_features * w->in_features * 2), ins, 3);
  if (rc) return rc;
  (void)hipGetLastError();
  return finish_launch(launch_dequant(view(w), out, as_stream(stream)), as_stream(stream));
}

int int8_gemv(const int8w_weight *w, const uint16_t *x, uint16_t *y, uint64_t stream) {
  int rc = validate(w);
  if (rc) return rc;
  if (!x || !y) return fail(INT8W_ERR_NULL, "x or y is NULL");
  if (!aligned(x, 16)) return fail(INT8W_ERR_ALIGN, "x is not 16-byte aligned");
  if (!aligned(y, 2)) return fail(INT8W_ERR_ALIGN, "y is not 2-byte aligned");
  Range ins[4];
  weight_ranges(w, ins);
  ins[3] = range("x", x, (uint64_t)w->in_features * 2);
  rc = check_alias(range("y", y, (uint64_t)w->out_features * 2), ins, 4);
  if (rc) return rc;
  (void)hipGetLastError();
  return finish_launch(launch_gemv(view(w), kEpiNone, x, nullptr, nullptr, y, as_stream(stream)),
                       as_stream(stream));
}

int int8_quantize(const uint16_t *w, uint32_t out_features, uint32_t in_features, uint32_t group_size,
                  uint32_t *packed, uint16_t *scales, uint16_t *biases, uint64_t stream) {
  const int8w_weight out = {packed, scales, biases, out_features, in_features, group_size};
  int rc = validate(&out);
  if (rc) return rc;
  if (!w) return fail(INT8W_ERR_NULL, "w is NULL");
  if (!aligned(w, 16)) return fail(INT8W_ERR_ALIGN, "w is not 16-byte aligned");
  Range outs[3];
  weight_ranges(&out, outs);
  const Range in = range("w", w, (uint64_t)out_features * in_features * 2);
  for (int i = 0; i < 3; ++i) {
    if (overlaps(outs[i], in)) return fail(INT8W_ERR_ALIAS, "output %s overlaps input w", outs[i].name);
    for (int j = 0; j < i; ++j)
      if (overlaps(outs[i], outs[j])) return fail(INT8W_ERR_ALIAS, "outputs %s and %s overlap", outs[j].name, outs[i].name);
  }
  (void)hipGetLastError();
  return finish_launch(launch_quantize(w, out_features, in_features, group_size, packed, scales, biases,
                                       as_stream(stream)),
                       as_stream(stream));
}

int int8_gemv_multi(const int8w_weight *w, uint32_t count, const uint16_t *x, uint16_t *const *y,
                    uint64_t stream) {
  if (!w || !y || !x) return fail(INT8W_ERR_NULL, "weights, x or y is NULL");
  if (count == 0 || count > INT8W_MAX_MULTI)
    return fail(INT8W_ERR_SHAPE, "count %u outside 1..%d", count, INT8W_MAX_MULTI);
  WeightView views[INT8W_MAX_MULTI];
  Range ins[3 * INT8W_MAX_MULTI + 1];
  for (uint32_t i = 0; i < count; ++i) {
    int rc = validate(&w[i]);
    if (rc) return rc;
    if (w[i].in_features != w[0].in_features || w[i].group_size != w[0].group_size)
      return fail(INT8W_ERR_SHAPE, "weight %u has in_features %u / group_size %u, weight 0 has %u / %u", i,
                  w[i].in_features, w[i].group_size, w[0].in_features, w[0].group_size);
    if (!y[i]) return fail(INT8W_ERR_NULL, "y[%u] is NULL", i);
    if (!aligned(y[i], 2)) return fail(INT8W_ERR_ALIGN, "y[%u] is not 2-byte aligned", i);
    weight_ranges(&w[i], ins + 3 * i);
    views[i] = view(&w[i]);
  }
  if (!aligned(x, 16)) return fail(INT8W_ERR_ALIGN, "x is not 16-byte aligned");
  ins[3 * count] = range("x", x, (uint64_t)w[0].in_features * 2);
  for (uint32_t i = 0; i < count; ++i) {
    const Range yi = range("y", y[i], (uint64_t)w[i].out_features * 2);
    int rc = check_alias(yi, ins, 3 * (int)count + 1);
    if (rc) return rc;
    for (uint32_t j = 0; j < i; ++j)
      if (overlaps(yi, range("y", y[j], (uint64_t)w[j].out_features * 2)))
        return fail(INT8W_ERR_ALIAS, "outputs y[%u] and y[%u] overlap", j, i);
  }
  (void)hipGetLastError();
  return finish_launch(launch_gemv_multi(views, y, count, x, as_stream(stream)), as_stream(stream));
}

int int8_moe_gemv(const int8w_weight *experts, uint32_t num_experts, const uint16_t *x, uint32_t x_rows,
                  const uint32_t *ids, uint32_t tokens, uint32_t topk, uint16_t *y, uint64_t stream) {
  int rc = validate(experts);
  if (rc) return rc;
  if (num_experts == 0 || experts->out_features % num_experts != 0)
    return fail(INT8W_ERR_SHAPE, "%u stacked rows are not a whole number of %u experts", experts->out_features,
                num_experts);
  const uint64_t slots = (uint64_t)tokens * topk;
  if (slots > INT8W_MAX_MOE_SLOTS)
    return fail(INT8W_ERR_SHAPE, "tokens*topk = %llu exceeds %d slots", (unsigned long long)slots,
                INT8W_MAX_MOE_SLOTS);
  if (slots == 0) return ok();
  if (x_rows != 1 && x_rows != topk) return fail(INT8W_ERR_SHAPE, "x_rows %u is neither 1 nor topk %u", x_rows, topk);
  if (!x || !ids || !y) return fail(INT8W_ERR_NULL, "x, ids or y is NULL");
  if (!aligned(x, 16)) return fail(INT8W_ERR_ALIGN, "x is not 16-byte aligned");
  if (!aligned(ids, 4)) return fail(INT8W_ERR_ALIGN, "ids is not 4-byte aligned");
  if (!aligned(y, 2)) return fail(INT8W_ERR_ALIGN, "y is not 2-byte aligned");
  const uint64_t N = experts->out_features / num_experts, K = experts->in_features;
  Range ins[5];
  weight_ranges(experts, ins);
  ins[3] = range("x", x, (uint64_t)tokens * x_rows * K * 2);
  ins[4] = range("ids", ids, slots * 4);
  rc = check_alias(range("y", y, slots * N * 2), ins, 5);
  if (rc) return rc;
  (void)hipGetLastError();
  return finish_launch(launch_moe_gemv(view(experts), num_experts, x, x_rows, ids, tokens, topk, y,
                                       as_stream(stream)),
                       as_stream(stream));
}

int int8w_fp8_gemv(const int8w_fp8_weight *w, const uint16_t *x, uint16_t *y, uint64_t stream) {
  if (!w) return fail(INT8W_ERR_NULL, "weight descriptor is NULL");
  if (!w->weight) return fail(INT8W_ERR_NULL, "weight is NULL");
  if (w->n == 0 || w->k == 0) return fail(INT8W_ERR_SHAPE, "zero dimension (n=%u k=%u)", w->n, w->k);
  if (w->k % 16 != 0) return fail(INT8W_ERR_SHAPE, "k %u is not a multiple of 16", w->k);
  if ((uint64_t)w->n * (w->k / 16u) > 0x7FFFFFFFull || w->k > (1u << 24))
    return fail(INT8W_ERR_SHAPE, "weight too large (%u x %u codes)", w->n, w->k);
  if (w->scale_format > INT8W_FP8_SINGLE)
    return fail(INT8W_ERR_UNSUPPORTED, "unknown scale_format %u", w->scale_format);
  const uint64_t n = w->n, k = w->k;
  uint64_t scale_bytes = 0;
  switch (w->scale_format) {
    case INT8W_FP8_PER_ROW:
      if (!w->scale) return fail(INT8W_ERR_NULL, "per-row scale is NULL");
      if (!aligned(w->scale, 4)) return fail(INT8W_ERR_ALIGN, "per-row scale is not 4-byte aligned");
      scale_bytes = n * 4;
      break;
    case INT8W_FP8_BLOCK_BF16:
    case INT8W_FP8_BLOCK_F32: {
      const uint32_t bs = w->block_size;
      if (bs < 64 || bs > 1024 || (bs & (bs - 1)) != 0)
        return fail(INT8W_ERR_UNSUPPORTED, "block_size %u is not a power of two in 64..1024", bs);
      if (!w->scale) return fail(INT8W_ERR_NULL, "block scale is NULL");
      const uint64_t el = w->scale_format == INT8W_FP8_BLOCK_BF16 ? 2 : 4;
      if (!aligned(w->scale, el)) return fail(INT8W_ERR_ALIGN, "block scale is not %llu-byte aligned",
                                              (unsigned long long)el);
      scale_bytes = ((n + bs - 1) / bs) * ((k + bs - 1) / bs) * el;
      break;
    }
    default:
      if (w->scale) return fail(INT8W_ERR_SHAPE, "scale_format SINGLE takes no scale buffer (scale must be NULL)");
  }
  if (!x || !y) return fail(INT8W_ERR_NULL, "x or y is NULL");
  if (!aligned(w->weight, 16)) return fail(INT8W_ERR_ALIGN, "weight is not 16-byte aligned");
  if (!aligned(x, 16)) return fail(INT8W_ERR_ALIGN, "x is not 16-byte aligned");
  if (!aligned(y, 2)) return fail(INT8W_ERR_ALIGN, "y is not 2-byte aligned");
  Range ins[3] = {range("weight", w->weight, n * k), range("scale", w->scale, scale_bytes), range("x", x, k * 2)};
  int rc = check_alias(range("y", y, n * 2), ins, 3);
  if (rc) return rc;
  (void)hipGetLastError();
  return finish_launch(launch_fp8_gemv(w->weight, w->scale, (Fp8ScaleKind)w->scale_format, w->block_size,
                                       w->single_scale, w->n, w->k, x, y, as_stream(stream)),
                       as_stream(stream));
}

static int gemv_gated(const int8w_weight *w, const uint16_t *gate, const uint16_t *up, const uint16_t *x_resid,
                      uint16_t *y, uint64_t stream, bool with_resid) {
  int rc = validate(w);
  if (rc) return rc;
  if (!gate || !up || !y || (with_resid && !x_resid))
    return fail(INT8W_ERR_NULL, with_resid ? "gate, up, x_resid or y is NULL" : "gate, up or y is NULL");
  if (!aligned(gate, 16) || !aligned(up, 16)) return fail(INT8W_ERR_ALIGN, "gate/up are not 16-byte aligned");
  if (!aligned(y, 2) || (with_resid && !aligned(x_resid, 2)))
    return fail(INT8W_ERR_ALIGN, "y/x_resid are not 2-byte aligned");
  const uint64_t K = w->in_features, N = w->out_features;
  Range ins[6];
  weight_ranges(w, ins);
  ins[3] = range("gate", gate, K * 2);
  ins[4] = range("up", up, K * 2);
  int n_ins = 5;
  // y == x_resid exactly is the allowed in-place residual; any other overlap is not.
  if (with_resid && reinterpret_cast<const void *>(x_resid) != reinterpret_cast<const void *>(y))
    ins[n_ins++] = range("x_resid", x_resid, N * 2);
  rc = check_alias(range("y", y, N * 2), ins, n_ins);
  if (rc) return rc;
  (void)hipGetLastError();
  return finish_launch(launch_gemv(view(w), with_resid ? kEpiSiluGateResid : kEpiSiluGate, gate, up,
                                   with_resid ? x_resid : nullptr, y, as_stream(stream)),
                       as_stream(stream));
}

int int8_gemv_silu_gate(const int8w_weight *w, const uint16_t *gate, const uint16_t *up, uint16_t *y,
                        uint64_t stream) {
  return gemv_gated(w, gate, up, nullptr, y, stream, false);
}

int int8_gemv_silu_gate_resid(const int8w_weight *w, const uint16_t *gate, const uint16_t *up,
                              const uint16_t *x_resid, uint16_t *y, uint64_t stream) {
  return gemv_gated(w, gate, up, x_resid, y, stream, true);
}

}  // extern "C"

namespace int8w {

int report_error(int code, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
  va_end(ap);
  return code;
}

// gemm with an optional workspace (ws == nullptr: the tiled kernel never
// splits K).  ws_bytes is checked against what the chosen launch needs.
int gemm_common(const int8w_weight *w, const uint16_t *x, uint16_t *y, uint32_t m, void *ws, uint64_t ws_bytes,
                uint64_t stream) {
  int rc = validate(w);
  if (rc) return rc;
  if (m == 0) return ok();
  if (!x || !y) return fail(INT8W_ERR_NULL, "X or Y is NULL");
  if (!aligned(x, 16)) return fail(INT8W_ERR_ALIGN, "X is not 16-byte aligned");
  if (!aligned(y, 2)) return fail(INT8W_ERR_ALIGN, "Y is not 2-byte aligned");
  const uint64_t K = w->in_features, N = w->out_features;
  if ((uint64_t)m * K > 0xFFFFFFFFull || (uint64_t)m * N > 0xFFFFFFFFull)
    return fail(INT8W_ERR_SHAPE, "m=%u rows too many for this weight", m);
  // 16 < m <= 128 on a small grid: passes of the small-m kernel over slices of
  // 32 (or 16) rows
  const bool sm_ok = smallm_supported(w->in_features, w->group_size);
  // 2 or 3 rows (4 on weights of at most 8192 rows) on in_features 1024..4096:
  // the register-resident gemv form with several rows, measured faster there
  // than the small-m kernel (14336 x 4096, m = 2: 12.8 against 15.0 us)
  const bool rows = gemv_rows_supported(w->in_features, m) && (m <= 3u || N <= 8192u);
  // 2 rows on longer in_features at group size 32 or above 16384: the same
  // arithmetic with X's rows in LDS (4096 x 14336 gs32: 16.5 against 18.5 us)
  const bool lrows = !rows && gemv_rows_lds_supported(w->in_features, w->group_size, m);
  const uint32_t slice = m > 16u ? gemm_smallm_slice_rows(view(w), m, ws != nullptr) : 0u;
  const bool passes = slice != 0u;
  // the tiled kernel addresses a 256-row X tile with 32-bit byte offsets
  const bool tiled = !passes && !rows && !lrows && (m > 16u || (m > 1u && !sm_ok));
  if (tiled && K * 2u * 256u > 0xFFFFFFFFull)
    return fail(INT8W_ERR_SHAPE, "in_features=%u above 2^23 - 1 needs m = 1 or a small-m shape (m=%u)",
                w->in_features, m);
  const uint64_t need = tiled && ws ? gemm_prefill_workspace_bytes(view(w), m) : 0u;
  if (ws) {
    if (!aligned(ws, 256)) return fail(INT8W_ERR_ALIGN, "workspace is not 256-byte aligned");
    if (ws_bytes < need)
      return fail(INT8W_ERR_SHAPE, "workspace of %llu bytes, this call needs %llu", (unsigned long long)ws_bytes,
                  (unsigned long long)need);
  }
  Range ins[4];
  weight_ranges(w, ins);
  ins[3] = range("X", x, (uint64_t)m * K * 2);
  rc = check_alias(range("Y", y, (uint64_t)m * N * 2), ins, 4);
  if (rc) return rc;
  if (need) {
    const Range outs[2] = {range("Y", y, (uint64_t)m * N * 2), range("X", x, (uint64_t)m * K * 2)};
    rc = check_alias(range("workspace", ws, need), ins, 3);
    if (rc) return rc;
    rc = check_alias(range("workspace", ws, need), outs, 2);
    if (rc) return rc;
  }
  (void)hipGetLastError();
  hipStream_t s = as_stream(stream);
  hipError_t e;
  if (m == 1) {
    e = launch_gemv(view(w), kEpiNone, x, nullptr, nullptr, y, s);
  } else if (rows) {
    e = launch_gemv_rows(view(w), x, y, m, s);
  } else if (lrows) {
    e = launch_gemv_rows_lds(view(w), x, y, m, s);
  } else if (m <= 16 && sm_ok) {
    e = launch_gemm_smallm(view(w), x, y, m, s);
  } else if (passes) {
    // slices of `slice` rows; one of at most 16 rows takes the one-tile kernel
    e = hipSuccess;
    for (uint32_t r0 = 0; r0 < m && e == hipSuccess; r0 += slice) {
      const uint32_t mi = m - r0 < slice ? m - r0 : slice;
      e = mi > 16u ? launch_gemm_smallm32(view(w), x + (size_t)r0 * K, y + (size_t)r0 * N, mi, s)
                   : launch_gemm_smallm(view(w), x + (size_t)r0 * K, y + (size_t)r0 * N, mi, s);
    }
  } else {
    e = launch_gemm_prefill(view(w), x, y, m, need ? ws : nullptr, s);
  }
  return finish_launch(e, s);
}

}  // namespace int8w

extern "C" {

int int8_gemm(const int8w_weight *w, const uint16_t *x, uint16_t *y, uint32_t m, uint64_t stream) {
  return gemm_common(w, x, y, m, nullptr, 0, stream);
}

uint64_t int8_gemm_workspace_bytes(const int8w_weight *w, uint32_t m) {
  if (validate(w) != INT8W_OK || m <= 16u) return 0;
  const uint64_t K = w->in_features, N = w->out_features;
  if ((uint64_t)m * K > 0xFFFFFFFFull || (uint64_t)m * N > 0xFFFFFFFFull || K * 2u * 256u > 0xFFFFFFFFull) return 0;
  if (gemm_smallm_slice_rows(view(w), m, true) != 0u) return 0;
  return gemm_prefill_workspace_bytes(view(w), m);
}

int int8_gemm_ws(const int8w_weight *w, const uint16_t *x, uint16_t *y, uint32_t m, void *workspace,
                 uint64_t workspace_bytes, uint64_t stream) {
  if (!workspace) return fail(INT8W_ERR_NULL, "workspace is NULL (int8_gemm takes no workspace)");
  return gemm_common(w, x, y, m, workspace, workspace_bytes, stream);
}

const char *int8w_last_error(void) { return g_last_error; }

// ---- calibration kernels (int8w_measure.h)

static int check_stream_args(const void *src, uint64_t bytes) {
  if (!src) return fail(INT8W_ERR_NULL, "src is NULL");
  if (bytes == 0 || bytes % 1024u != 0 || bytes > (1ull << 40))
    return fail(INT8W_ERR_SHAPE, "bytes %llu is not a positive multiple of 1024 up to 2^40",
                (unsigned long long)bytes);
  if (!aligned(src, 16)) return fail(INT8W_ERR_ALIGN, "src is not 16-byte aligned");
  return INT8W_OK;
}

int int8w_stream_read(const void *src, uint64_t bytes, uint32_t *sink, uint64_t stream) {
  int rc = check_stream_args(src, bytes);
  if (rc) return rc;
  if (!sink) return fail(INT8W_ERR_NULL, "sink is NULL");
  if (!aligned(sink, 4)) return fail(INT8W_ERR_ALIGN, "sink is not 4-byte aligned");
  (void)hipGetLastError();
  hipStream_t s = as_stream(stream);
  return finish_launch(launch_stream_read(src, bytes, sink, s), s);
}

int int8w_stream_copy(const void *src, void *dst, uint64_t bytes, uint64_t stream) {
  int rc = check_stream_args(src, bytes);
  if (rc) return rc;
  if (!dst) return fail(INT8W_ERR_NULL, "dst is NULL");
  if (!aligned(dst, 16)) return fail(INT8W_ERR_ALIGN, "dst is not 16-byte aligned");
  if (overlaps(range("dst", dst, bytes), range("src", src, bytes)))
    return fail(INT8W_ERR_ALIAS, "dst overlaps src");
  (void)hipGetLastError();
  hipStream_t s = as_stream(stream);
  return finish_launch(launch_stream_copy(src, dst, bytes, s), s);
}

int int8w_stream_expand(const void *src, void *dst, uint64_t bytes, uint64_t stream) {
  int rc = check_stream_args(src, bytes);
  if (rc) return rc;
  if (!dst) return fail(INT8W_ERR_NULL, "dst is NULL");
  if (!aligned(dst, 16)) return fail(INT8W_ERR_ALIGN, "dst is not 16-byte aligned");
  if (overlaps(range("dst", dst, 2 * bytes), range("src", src, bytes)))
    return fail(INT8W_ERR_ALIAS, "dst overlaps src");
  (void)hipGetLastError();
  hipStream_t s = as_stream(stream);
  return finish_launch(launch_stream_expand(src, dst, bytes, s), s);
}

}  // extern "C"
