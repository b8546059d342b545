/*
 * int8w.h -- C-ABI of the MI355X (gfx950) library for 8-bit affine
 * group-quantized weight-only linear layers (libint8w.so).
 *
 * Source of the operations: the rustdoc page "MlxInt8Weight"
 * (metrale_gpu_runtime::mlx_int8): the struct description (one "8-bit affine"
 * linear weight resident on the GPU, no Drop), the field sections packed /
 * scales / biases, and the methods load (validation rules), dequantize_to,
 * gemv, gemv_silu_gate, gemv_silu_gate_resid, gemm and release (ownership).
 *
 * Weight encoding (the page's field sections; byte order, signedness and the
 * dequantization formula are this library's readings of them):
 *   packed  uint32 [out_features, in_features/4], row-major; code k of row n
 *           is byte (k % 4) of word packed[n*in_features/4 + k/4], least
 *           significant byte first; codes are unsigned, 0..255.
 *   scales  BF16 bit patterns [out_features, in_features/group_size], row-major.
 *   biases  BF16 bit patterns, same shape.
 *   w[n,k]  = q[n,k] * scales[n, k/group_size] + biases[n, k/group_size],
 *           an fp32 value (the product is exact, the sum rounds once).
 *
 * Conventions shared by every entry point:
 *   - Every pointer is a DEVICE pointer (HIP global memory); BF16 data are
 *     passed as uint16_t bit patterns.
 *   - The library never allocates, frees or retains caller memory.  All
 *     buffers are borrowed for the duration of the queued GPU work; the caller
 *     owns them and frees them once (the page's release method).
 *   - `stream` is a hipStream_t cast to uint64_t (0 = the null stream).  Calls
 *     validate on the host, enqueue the kernel(s) and return without waiting.
 *     Faults during execution surface at the caller's next synchronisation.
 *   - Return value: INT8W_OK, or a negative INT8W_ERR_* code; on any error
 *     nothing has been enqueued, and int8w_last_error() describes it.
 *   - Alignment: packed, x, gate, up, X and the dequantize_to output must be
 *     16-byte aligned; scales, biases, y, x_resid and Y 2-byte aligned.
 *   - Outputs must not overlap any input, except y == x_resid exactly
 *     (in-place residual: each output element reads only its own residual).
 *   - Results are deterministic: the same call on the same data gives the
 *     same bits (no atomics in any reduction).
 *   - The library is stateless and re-entrant apart from the thread-local
 *     last-error string.
 */
#ifndef INT8W_H
#define INT8W_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* A borrowed view of one quantized weight (the page's MlxInt8Weight struct). */
typedef struct int8w_weight {
  const uint32_t *packed; /* [out_features, in_features/4] code words (device) */
  const uint16_t *scales; /* [out_features, in_features/group_size] BF16 (device) */
  const uint16_t *biases; /* [out_features, in_features/group_size] BF16 (device) */
  uint32_t out_features;  /* N >= 1 */
  uint32_t in_features;   /* K >= group_size, K % group_size == 0, K <= 2^24 */
  uint32_t group_size;    /* 32, 64 or 128 */
} int8w_weight;

enum {
  INT8W_OK = 0,
  INT8W_ERR_NULL = -1,        /* a required pointer is NULL */
  INT8W_ERR_SHAPE = -2,       /* zero dimension, in_features % group_size != 0, N*K/16 >= 2^31, K > 2^24 */
  INT8W_ERR_UNSUPPORTED = -3, /* group_size not in {32, 64, 128} */
  INT8W_ERR_ALIGN = -4,       /* a pointer violates the alignment rule above */
  INT8W_ERR_ALIAS = -5,       /* an output overlaps an input */
  INT8W_ERR_HIP = -6          /* the HIP runtime reported an error at launch */
};

/* Source: "MlxInt8Weight", method load (its list of failure cases).
 * Check a weight view the way the page's load method checks its tensors: all
 * three buffers present, in_features divisible by group_size (hence by 4, the
 * codes per word), the per-group shape implied.  Also checks group_size is
 * supported and the pointers are aligned.  Touches no device memory. */
int int8w_validate(const int8w_weight *w);

/* Source: the DynQuantizedStorage trait page, method storage_size_in_bytes
 * (the analogue for this layout).
 * Bytes of the quantized storage: N*K codes + 2*2*N*(K/group_size) for the
 * BF16 scales and biases; 0 for an invalid shape. */
uint64_t int8w_storage_bytes(uint32_t out_features, uint32_t in_features, uint32_t group_size);

/* Source: "MlxInt8Weight", method dequantize_to (kernel mlx_int8_dequant; the
 * output holds at least out*in*2 bytes).
 * dequantize_to: write the full dequantised weight as BF16 to `out`, row-major
 * [out_features, in_features]; out[n*K + k] = RNE_bf16(w[n,k]) (round to
 * nearest, ties to even).  `out` must hold out_features*in_features*2 bytes;
 * exactly that many are written. */
int int8_dequantize_to(const int8w_weight *w, uint16_t *out, uint64_t stream);

/* Source: "MlxInt8Weight", method gemv (kernel mlx_int8_gemv: y = W x, x
 * BF16 [in], y BF16 with at least out elements).
 * gemv: y = W x.  x is BF16 [in_features]; y is BF16 with at least
 * out_features elements, of which exactly out_features are written:
 * y[n] = RNE_bf16(sum_k w[n,k] * x[k]), accumulated in fp32. */
int int8_gemv(const int8w_weight *w, const uint16_t *x, uint16_t *y, uint64_t stream);

/* quantize: the step before the weight exists -- a BF16 weight w [out_features,
 * in_features] (row-major, 16-byte aligned) is encoded into packed / scales /
 * biases with the layout of int8w_weight (rustdoc page of the DynQuantizedStorage
 * trait, method quantize; the pages give no formula, this is the plain affine
 * min/max reading).  Per group of group_size values v of a row, in fp32:
 *   lo = min v, hi = max v (a zero extreme, -0 or +0, taken as +0),
 *   scale = RNE_bf16((hi - lo) / 255), bias = lo,
 *   q = clamp(rint((v - bias) / scale), 0, 255), and q = 0 when scale == 0.
 * Then |q*scale + bias - v| <= scale/2 except at the top of a group whose
 * scale rounded down, where the clamp adds at most 255*((hi-lo)/255 - scale).
 * Inputs must be finite.  Outputs must not overlap w or each other; the shape
 * rules and error codes are those of int8w_validate applied to the outputs. */
int int8_quantize(const uint16_t *w, uint32_t out_features, uint32_t in_features, uint32_t group_size,
                  uint32_t *packed, uint16_t *scales, uint16_t *biases, uint64_t stream);

/* gemv_multi: y[i] = W[i] x for count weights (1 <= count <= INT8W_MAX_MULTI)
 * that share in_features and group_size, in one launch -- the projections of
 * one activation (q, k and v; gate and up) that the page's gemv method runs
 * one call at a time.  Each y[i] is computed with int8_gemv's arithmetic and
 * meets the same bound (the split of in_features into on-chip tiles, and so
 * the fp32 rounding, may differ).  `w` and `y` are HOST arrays of count
 * entries; y[i] is a device buffer of at least w[i].out_features BF16
 * elements.  Outputs must not overlap each other, x or any weight.
 * INT8W_ERR_SHAPE for count outside 1..INT8W_MAX_MULTI or mismatched
 * in_features / group_size. */
#define INT8W_MAX_MULTI 4
int int8_gemv_multi(const int8w_weight *w, uint32_t count, const uint16_t *x, uint16_t *const *y,
                    uint64_t stream);

/* moe_gemv: the expert-indexed product (rustdoc page of the DynQuantizedStorage
 * trait, provided method indexed_moe_forward, which gives the signature only:
 * the quantized tensor's shape, an input and the ids of the experts).  Read as:
 *   - `experts` holds num_experts experts of [N, in_features] stacked along
 *     rows: its out_features is num_experts * N, and expert e is rows
 *     e*N .. e*N + N - 1 (validated like any weight);
 *   - x is BF16 [tokens, x_rows, in_features], x_rows = 1 (every slot of a
 *     token reads the token's row) or x_rows = topk (each slot its own row);
 *   - ids is a DEVICE uint32 array [tokens, topk], 4-byte aligned, read by
 *     the kernel (never on the host);
 *   - y is BF16 [tokens, topk, N]: y[t, j, n] = sum_k w_e[n, k] x_(t,j)[k]
 *     with e = ids[t, j], with int8_gemv's arithmetic and bound.
 * A slot whose id is not below num_experts reads no weight and gets the BF16
 * quiet NaN 0x7FC0 in all N outputs.  One token: each slot streams its
 * expert's rows.  Several tokens with tokens * topk >= num_experts (at most
 * 256 slots, 512 experts, in_features 1024..4096 a multiple of 1024): each
 * named expert is streamed once for all the slots naming it; the results are
 * the same bits either way.  tokens = 0 or topk = 0 is a no-op.  Errors: INT8W_ERR_SHAPE for num_experts = 0 or not dividing
 * out_features, x_rows not 1 or topk, or more than INT8W_MAX_MOE_SLOTS slots;
 * INT8W_ERR_ALIGN for x not 16-byte or ids not 4-byte aligned; INT8W_ERR_ALIAS
 * for y overlapping the experts, x or ids. */
#define INT8W_MAX_MOE_SLOTS 65536
int int8_moe_gemv(const int8w_weight *experts, uint32_t num_experts, const uint16_t *x, uint32_t x_rows,
                  const uint32_t *ids, uint32_t tokens, uint32_t topk, uint16_t *y, uint64_t stream);

/* ---- FP8 E4M3 weights (rustdoc page "Fp8Weight": struct description and the
 * fields weight, row_scale, n, k, scale_format).  The weight is n x k E4M3
 * bytes, row-major (sign bit 7, exponent bits 6..3 with bias 7, mantissa bits
 * 2..0; exponent 0 is subnormal; 0x7F and 0xFF are NaN; no infinities), and
 * w[i,j] = E4M3(weight[i,j]) * scale with the scale laid out per the tag: */
enum {
  INT8W_FP8_PER_ROW = 0,    /* scale: device f32 [n], scale[i] */
  INT8W_FP8_BLOCK_BF16 = 1, /* scale: device BF16 [ceil(n/BS), ceil(k/BS)], scale[i/BS][j/BS] */
  INT8W_FP8_BLOCK_F32 = 2,  /* the same shape in f32 (the page gives block scales as BF16 in
                               its format list and as FP32 in its transpose method) */
  INT8W_FP8_SINGLE = 3      /* scale pointer NULL; single_scale is the one global value */
};

typedef struct {
  const uint8_t *weight; /* device, [n, k] E4M3 bytes, 16-byte aligned */
  const void *scale;     /* device, layout per scale_format (4-byte aligned f32, 2-byte BF16); NULL for SINGLE */
  uint32_t n;            /* output features (rows) */
  uint32_t k;            /* input features (columns), a multiple of 16 */
  uint32_t scale_format; /* INT8W_FP8_* */
  uint32_t block_size;   /* BS for the block formats: a power of two, 64..1024 (128 on the page) */
  float single_scale;    /* the global scale for INT8W_FP8_SINGLE */
} int8w_fp8_weight;

/* fp8_gemv: y = W x.  x is BF16 [k], 16-byte aligned; y is BF16 with at least
 * n elements, of which exactly n are written:
 *   y[i] = RNE_bf16(sum_j E4M3(weight[i,j]) * scale * x[j]), accumulated in fp32
 * (a block scale multiplies each 16-code run's partial sum, a row or global
 * scale the row's total); a NaN code gives a NaN output.  The bound is
 * int8_gemv's.  Errors: INT8W_ERR_NULL (weight, x, y, or the scale of a
 * non-SINGLE format is NULL), INT8W_ERR_SHAPE (n or k zero, k not a multiple of
 * 16, k > 2^24, n*k/16 >= 2^31, or a scale given with SINGLE),
 * INT8W_ERR_UNSUPPORTED (unknown format, block_size not a power of two in
 * 64..1024), INT8W_ERR_ALIGN, INT8W_ERR_ALIAS (y overlapping weight, scale or
 * x). */
int int8w_fp8_gemv(const int8w_fp8_weight *w, const uint16_t *x, uint16_t *y, uint64_t stream);

/* Source: "MlxInt8Weight", method gemv_silu_gate (kernel
 * mlx_int8_gemv_silu_gate: one launch, the gated product kept off memory).
 * gemv_silu_gate: y = W (silu(gate) * up) in one launch, silu(g) = g/(1+e^-g).
 * gate and up are BF16 [in_features]; the product silu(gate)*up is formed in
 * fp32 on chip and never written to memory.  y as for int8_gemv. */
int int8_gemv_silu_gate(const int8w_weight *w, const uint16_t *gate, const uint16_t *up, uint16_t *y,
                        uint64_t stream);

/* Source: "MlxInt8Weight", method gemv_silu_gate_resid (the residual form of
 * the fused gated product, one launch).
 * gemv_silu_gate_resid: the above plus a residual, in one launch:
 * y[n] = RNE_bf16(x_resid[n] + sum_k w[n,k] * silu(gate[k]) * up[k]), the
 * residual added in fp32 before the single rounding.  x_resid is BF16
 * [out_features]; y may be x_resid itself. */
int int8_gemv_silu_gate_resid(const int8w_weight *w, const uint16_t *gate, const uint16_t *up,
                              const uint16_t *x_resid, uint16_t *y, uint64_t stream);

/* Source: "MlxInt8Weight", method gemm (kernel mlx_int8_gemm: Y = X W^T for m
 * rows; its one-thread-per-output design is not followed here).
 * gemm: Y = X W^T.  X is BF16 [m, in_features] and Y BF16 [m, out_features],
 * both contiguous row-major.  Y[i,n] = RNE_bf16(sum_k w[n,k] * X[i,k]) with fp32
 * accumulation.  m = 1 runs the gemv; 2 <= m <= 16 the small-m kernel, which
 * multiplies the raw codes and applies each group's scale and bias to the
 * group's partial sums (except a few rows on some shapes: 2..4 rows on
 * in_features 1024..4096, and 2 rows on longer in_features at group size 32 or
 * above 16384, take the gemv's weight stream with each code converted once and
 * multiplied into every row); larger m the tiled kernel, where the weight enters the
 * matrix cores as RNE_bf16(w[n,k]) (the dequantize_to value).  For
 * 16 < m <= 128 on a weight that gives the tiled kernel few tiles per CU (so
 * that its time is set by walking all of in_features, whatever m), the rows
 * go through the small-m kernel in slices of 32 (16 where its two-tile form
 * does not fit the LDS) when that many passes over the weight are estimated
 * faster: one launch per slice, all on `stream`; each slice's rows are then
 * what gemm gives for that slice alone.  m == 0 enqueues nothing and
 * returns INT8W_OK.  INT8W_ERR_SHAPE also when m * in_features or
 * m * out_features exceeds 2^32 - 1, or when in_features >= 2^23 for an m
 * that takes the tiled kernel (m > 16 outside those slices, or an m >= 2
 * whose scale/bias rows do not fit the small-m kernel's LDS). */
int int8_gemm(const int8w_weight *w, const uint16_t *x, uint16_t *y, uint32_t m, uint64_t stream);

/* Source: "MlxInt8Weight", method gemm, as int8_gemm; this form takes a
 * workspace so that a grid with too few tiles to occupy the GPU (e.g. m = 512
 * on a 4096-row weight) can split in_features over several work items per
 * tile.  Each item stores its fp32 partial in the workspace and a second
 * launch on the same stream adds the parts in a fixed order, so results are
 * deterministic (they may differ from int8_gemm's in the last bits, within the
 * same bound).
 *   int8_gemm_workspace_bytes(w, m): the bytes int8_gemm_ws needs for m rows
 *     of this weight; 0 when it would not split (or for an invalid weight).
 *   int8_gemm_ws(w, x, y, m, workspace, workspace_bytes, stream): as
 *     int8_gemm.  workspace is a DEVICE buffer, 256-byte aligned, of at least
 *     int8_gemm_workspace_bytes(w, m) bytes; its contents are scratch (no
 *     initial value needed, none kept).  The library does not allocate it.
 *     Calls that share a workspace must not run concurrently.  INT8W_ERR_NULL
 *     for a NULL workspace, INT8W_ERR_ALIGN, INT8W_ERR_SHAPE if it is too
 *     small, INT8W_ERR_ALIAS if it overlaps X, Y or the weight; otherwise as
 *     int8_gemm. */
uint64_t int8_gemm_workspace_bytes(const int8w_weight *w, uint32_t m);
int int8_gemm_ws(const int8w_weight *w, const uint16_t *x, uint16_t *y, uint32_t m, void *workspace,
                 uint64_t workspace_bytes, uint64_t stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): int8_gemm_ws
 * with the workspace taken from a static device array that the library holds
 * on every GPU it runs on, INT8W_NOALLOC_SCRATCH_BYTES (64 MiB) each, until
 * the process ends.  Same arguments, kernels and result bits as int8_gemm_ws
 * with a workspace of at least int8_gemm_workspace_bytes(w, m); nothing is
 * allocated or freed (no hipMalloc / hipFree, no allocating library call).
 * The array needs no initial value and keeps the last call's partials.  All
 * calls on one GPU share it: calls that can overlap on that GPU (several
 * streams or host threads) race.  Errors: INT8W_ERR_SHAPE when
 * int8_gemm_workspace_bytes(w, m) exceeds INT8W_NOALLOC_SCRATCH_BYTES
 * (nothing is enqueued; int8_gemm_ws takes any size), INT8W_ERR_HIP when the
 * array's device address cannot be looked up; otherwise as int8_gemm. */
#define INT8W_NOALLOC_SCRATCH_BYTES (64u << 20)
int int8_gemm_noalloc(const int8w_weight *w, const uint16_t *x, uint16_t *y, uint32_t m, uint64_t stream);

/* Human-readable description of the calling thread's most recent error
 * ("" if none).  The pointer stays valid until the thread's next call. */
const char *int8w_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* INT8W_H */
