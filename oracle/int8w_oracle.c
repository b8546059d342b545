/*
 * int8w_oracle.c -- plain, slow CPU oracle for 8-bit affine group-quantized
 * weight-only linear layers.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the library under test links, loads or
 * calls this file; only the tests, the smoke check and the CPU-baseline leg of
 * the benchmark do.  It shares no code, header, table or helper with the HIP
 * path.
 *
 * Source: the rustdoc page "MlxInt8Weight" (metrale_gpu_runtime::mlx_int8),
 * struct description and the field/method sections cited at each function.
 *
 * Conventions (each one is a reading of the page; the page gives no formula):
 *   - packed is uint32 [N, K/4]; code k of row n is byte (k % 4) of word
 *     packed[n, k/4], little-endian (byte 0 = bits 0..7), unsigned 0..255.
 *   - scales, biases are BF16 bit patterns [N, K/gs].
 *   - The weight is affine: w = q * scale + bias, evaluated in fp32
 *     (one fp32 multiply, one fp32 add; the product is exact because both
 *     factors carry at most 8 significant bits).
 *   - dequantize_to rounds that fp32 value to BF16, round-to-nearest-even.
 *   - Dot products accumulate in fp64, ascending k, one output at a time.
 *   - silu(g) = g / (1 + exp(-g)), evaluated in fp64.
 *
 * Build: gcc -O2 -ffp-contract=off -fopenmp -fPIC -shared (no fast-math).
 * OpenMP splits only the independent output rows; every sum is sequential, so
 * results do not depend on the thread count.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ---- BF16 <-> fp32, written from the IEEE-754 binary32 / bfloat16 layouts ---- */

/* A BF16 value is the upper 16 bits of a binary32 value; widening is exact. */
float orc_bf16_to_f32(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return f;
}

/* Round a binary32 value to BF16, nearest, ties to even.  The 16 dropped bits
 * are compared with one half unit in the last kept place (0x8000); above half
 * rounds up, below rounds down, exactly half rounds to the even neighbour.  A
 * carry out of the mantissa moves into the exponent, which is the correct
 * next representable value (and gives infinity past the largest finite BF16).
 * NaN stays NaN (quiet bit set, sign kept); infinities pass through. */
uint16_t orc_f32_to_bf16_rne(float f) {
  uint32_t u;
  memcpy(&u, &f, sizeof u);
  uint32_t exp_bits = (u >> 23) & 0xFFu;
  uint32_t man_bits = u & 0x7FFFFFu;
  if (exp_bits == 0xFFu && man_bits != 0) return (uint16_t)((u >> 16) | 0x0040u);
  uint32_t upper = u >> 16;
  uint32_t dropped = u & 0xFFFFu;
  if (dropped > 0x8000u || (dropped == 0x8000u && (upper & 1u))) upper += 1u;
  return (uint16_t)upper;
}

void orc_f32_to_bf16_rne_array(const uint32_t *in_bits, uint16_t *out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) {
    float f;
    memcpy(&f, &in_bits[i], sizeof f);
    out[i] = orc_f32_to_bf16_rne(f);
  }
}

/* ---- weight encoding: page "MlxInt8Weight", field sections packed/scales/biases ---- */

/* Code k of one packed row: byte k%4 of word k/4, least significant byte first. */
static uint32_t code_at(const uint32_t *row_words, int64_t k) {
  return (row_words[k >> 2] >> (8 * (k & 3))) & 0xFFu;
}

void orc_unpack(const uint32_t *packed, int64_t n_words, uint8_t *codes) {
  for (int64_t i = 0; i < n_words; ++i)
    for (int64_t j = 0; j < 4; ++j) codes[4 * i + j] = (uint8_t)code_at(packed + i, j);
}

/* fp32 affine value of one weight: q * scale + bias, one fp32 multiply and one
 * fp32 add (the struct description calls the weight "8-bit affine"; the scales
 * and biases sections give one BF16 pair per group of group_size codes). */
static float affine_f32(uint32_t q, uint16_t s_bits, uint16_t b_bits) {
  float s = orc_bf16_to_f32(s_bits);
  float b = orc_bf16_to_f32(b_bits);
  float prod = (float)q * s;
  float w = prod + b;
  return w;
}

/* One full fp32 row of the weight. */
static void weight_row_f32(const uint32_t *packed, const uint16_t *scales, const uint16_t *biases,
                           int64_t K, int64_t gs, int64_t n, float *w_row) {
  const int64_t G = K / gs;
  const uint32_t *words = packed + n * (K / 4);
  for (int64_t k = 0; k < K; ++k) {
    int64_t g = k / gs;
    w_row[k] = affine_f32(code_at(words, k), scales[n * G + g], biases[n * G + g]);
  }
}

/* All fp32 affine weights [N, K]. */
void orc_weight_f32(const uint32_t *packed, const uint16_t *scales, const uint16_t *biases,
                    int64_t N, int64_t K, int64_t gs, float *w32) {
#pragma omp parallel for schedule(static)
  for (int64_t n = 0; n < N; ++n) weight_row_f32(packed, scales, biases, K, gs, n, w32 + n * K);
}

/* dequantize_to: the full weight as BF16, row-major [N, K]
 * (page "MlxInt8Weight", method dequantize_to). */
void orc_dequantize_to(const uint32_t *packed, const uint16_t *scales, const uint16_t *biases,
                       int64_t N, int64_t K, int64_t gs, uint16_t *out) {
#pragma omp parallel
  {
    float *w_row = (float *)malloc((size_t)K * sizeof(float));
#pragma omp for schedule(static)
    for (int64_t n = 0; n < N; ++n) {
      weight_row_f32(packed, scales, biases, K, gs, n, w_row);
      for (int64_t k = 0; k < K; ++k) out[n * K + k] = orc_f32_to_bf16_rne(w_row[k]);
    }
    free(w_row);
  }
}

/* ---- products: page "MlxInt8Weight", methods gemv, gemv_silu_gate(_resid), gemm ---- */

/* Y[i, n] = sum_k w[n, k] * a[i, k] for fp64 activations a [m, K]; also
 * Aabs[i, n] = sum_k |w[n, k] * a[i, k]|.  Sums run in ascending k in fp64. */
void orc_matmul_act_f64(const uint32_t *packed, const uint16_t *scales, const uint16_t *biases,
                        int64_t N, int64_t K, int64_t gs, const double *a, int64_t m, double *Y,
                        double *Aabs) {
#pragma omp parallel
  {
    float *w_row = (float *)malloc((size_t)K * sizeof(float));
#pragma omp for schedule(static)
    for (int64_t n = 0; n < N; ++n) {
      weight_row_f32(packed, scales, biases, K, gs, n, w_row);
      for (int64_t i = 0; i < m; ++i) {
        const double *ai = a + i * K;
        double sum = 0.0, sum_abs = 0.0;
        for (int64_t k = 0; k < K; ++k) {
          double t = (double)w_row[k] * ai[k];
          sum += t;
          sum_abs += fabs(t);
        }
        Y[i * N + n] = sum;
        if (Aabs) Aabs[i * N + n] = sum_abs;
      }
    }
    free(w_row);
  }
}

/* gemm: Y = X W^T with X BF16 [m, K] (method gemm). */
void orc_gemm(const uint32_t *packed, const uint16_t *scales, const uint16_t *biases, int64_t N,
              int64_t K, int64_t gs, const uint16_t *X, int64_t m, double *Y, double *Aabs) {
  double *a = (double *)malloc((size_t)(m * K > 0 ? m * K : 1) * sizeof(double));
  for (int64_t j = 0; j < m * K; ++j) a[j] = (double)orc_bf16_to_f32(X[j]);
  orc_matmul_act_f64(packed, scales, biases, N, K, gs, a, m, Y, Aabs);
  free(a);
}

/* gemv: y = W x with x BF16 [K] (method gemv). */
void orc_gemv(const uint32_t *packed, const uint16_t *scales, const uint16_t *biases, int64_t N,
              int64_t K, int64_t gs, const uint16_t *x, double *y, double *Aabs) {
  orc_gemm(packed, scales, biases, N, K, gs, x, 1, y, Aabs);
}

/* silu(g) = g * sigmoid(g) = g / (1 + exp(-g)), fp64.  For g -> -inf the
 * quotient tends to -0, which is the limit of silu there. */
static double silu_f64(double g) { return g / (1.0 + exp(-g)); }

/* The gated activation silu(gate[k]) * up[k], fp64, never rounded to BF16
 * (method gemv_silu_gate: the product is not written out). */
void orc_silu_gate_act(const uint16_t *gate, const uint16_t *up, int64_t K, double *a) {
  for (int64_t k = 0; k < K; ++k)
    a[k] = silu_f64((double)orc_bf16_to_f32(gate[k])) * (double)orc_bf16_to_f32(up[k]);
}

/* gemv_silu_gate: y = W (silu(gate) * up). */
void orc_gemv_silu_gate(const uint32_t *packed, const uint16_t *scales, const uint16_t *biases,
                        int64_t N, int64_t K, int64_t gs, const uint16_t *gate, const uint16_t *up,
                        double *y, double *Aabs) {
  double *a = (double *)malloc((size_t)(K > 0 ? K : 1) * sizeof(double));
  orc_silu_gate_act(gate, up, K, a);
  orc_matmul_act_f64(packed, scales, biases, N, K, gs, a, 1, y, Aabs);
  free(a);
}

/* gemv_silu_gate_resid: y[n] = x_resid[n] + sum_k W[n,k] (silu(gate[k]) up[k]).
 * Aabs excludes the residual term. */
void orc_gemv_silu_gate_resid(const uint32_t *packed, const uint16_t *scales,
                              const uint16_t *biases, int64_t N, int64_t K, int64_t gs,
                              const uint16_t *gate, const uint16_t *up, const uint16_t *x_resid,
                              double *y, double *Aabs) {
  orc_gemv_silu_gate(packed, scales, biases, N, K, gs, gate, up, y, Aabs);
  for (int64_t n = 0; n < N; ++n) y[n] = (double)orc_bf16_to_f32(x_resid[n]) + y[n];
}

/* ---- quantizer: BF16 weight -> codes, scales, biases.
 *
 * Source: the rustdoc page of the DynQuantizedStorage trait (fuel_quantized),
 * required method quantize, and the MlxInt8Weight page's field sections for
 * the target layout.  The pages give no formula; this is the plain affine
 * min/max reading, evaluated in fp32 one operation at a time:
 *   per group of gs consecutive values v of a row (BF16, widened exactly):
 *     lo = min v, hi = max v               a zero extreme (-0 or +0) is taken as +0,
 *                                          so neither depends on the order of -0/+0
 *     s  = RNE_bf16((hi - lo) / 255)       fp32 subtraction, fp32 division
 *     b  = lo                              already a BF16 value
 *     q  = clamp(rint((v - b) / s), 0, 255)  fp32 subtraction and division,
 *                                           round half to even
 *   and q = 0 for every value of a group whose s is zero.
 * Inputs must be finite. */
static uint32_t quantize_code(float v, float b, float s) {
  if (s == 0.0f) return 0u;
  float d = v - b;
  float t = d / s;
  float r = rintf(t); /* current rounding mode: nearest, ties to even */
  if (r < 0.0f) r = 0.0f;
  if (r > 255.0f) r = 255.0f;
  return (uint32_t)r;
}

void orc_quantize(const uint16_t *w, int64_t N, int64_t K, int64_t gs, uint32_t *packed,
                  uint16_t *scales, uint16_t *biases) {
  const int64_t G = K / gs;
#pragma omp parallel for schedule(static)
  for (int64_t n = 0; n < N; ++n) {
    const uint16_t *row = w + n * K;
    uint32_t *out = packed + n * (K / 4);
    for (int64_t k = 0; k < K / 4; ++k) out[k] = 0u;
    for (int64_t g = 0; g < G; ++g) {
      float lo = orc_bf16_to_f32(row[g * gs]);
      float hi = lo;
      for (int64_t i = 1; i < gs; ++i) {
        float v = orc_bf16_to_f32(row[g * gs + i]);
        if (v < lo) lo = v;
        if (v > hi) hi = v;
      }
      if (lo == 0.0f) lo = 0.0f; /* a zero extreme is +0: an all-zero group has scale +0 and */
      if (hi == 0.0f) hi = 0.0f; /* bias +0 whichever signed zero comes first               */
      float span = hi - lo;
      float sf = span / 255.0f;
      uint16_t s_bits = orc_f32_to_bf16_rne(sf);
      uint16_t b_bits = orc_f32_to_bf16_rne(lo); /* exact: lo is a BF16 value */
      scales[n * G + g] = s_bits;
      biases[n * G + g] = b_bits;
      float s = orc_bf16_to_f32(s_bits), b = orc_bf16_to_f32(b_bits);
      for (int64_t i = 0; i < gs; ++i) {
        int64_t k = g * gs + i;
        uint32_t q = quantize_code(orc_bf16_to_f32(row[k]), b, s);
        out[k / 4] |= q << (8 * (k % 4));
      }
    }
  }
}

/* ---- expert-indexed product: the DynQuantizedStorage trait page, provided
 * method indexed_moe_forward.  The page gives only the signature (the
 * quantized tensor's shape, an input, and ids selecting experts); the reading
 * taken here:
 *   - the quantized tensor holds E experts of [N, K], stacked along rows, so
 *     expert e is rows e*N .. e*N + N - 1 of one packed/scales/biases set;
 *   - the input is BF16 [T, S, K] with S = 1 (every slot of a token reads the
 *     token's row) or S = topk (slot j of token t reads its own row);
 *   - ids are uint32 [T, topk]; slot (t, j) uses expert ids[t, j];
 *   - the output is [T, topk, N]: y[t, j, :] = W_e x_(t, j) with e = ids[t, j].
 * A slot whose id is not below E has no expert: its outputs are NaN.  Each
 * slot's product is the gemm above on that expert's rows, so the arithmetic
 * (fp32 weight, fp64 sums) is the same. */
void orc_moe_gemv(const uint32_t *packed, const uint16_t *scales, const uint16_t *biases, int64_t E,
                  int64_t N, int64_t K, int64_t gs, const uint16_t *x, int64_t S, const uint32_t *ids,
                  int64_t T, int64_t topk, double *y, double *Aabs) {
  const int64_t G = K / gs;
  for (int64_t t = 0; t < T; ++t) {
    for (int64_t j = 0; j < topk; ++j) {
      const int64_t slot = t * topk + j;
      const uint32_t e = ids[slot];
      double *ys = y + slot * N;
      double *as = Aabs + slot * N;
      if ((int64_t)e >= E) {
        for (int64_t n = 0; n < N; ++n) {
          ys[n] = NAN;
          as[n] = 0.0;
        }
        continue;
      }
      const uint16_t *xs = x + (t * S + (S == 1 ? 0 : j)) * K;
      orc_gemm(packed + (int64_t)e * N * (K / 4), scales + (int64_t)e * N * G, biases + (int64_t)e * N * G, N, K,
               gs, xs, 1, ys, as);
    }
  }
}

/* ---- FP8 E4M3 weight: the rustdoc page "Fp8Weight" (spark_model::weight_map),
 * struct description and fields weight, row_scale, n, k, scale_format.
 *
 * The page names the format (E4M3) and the three scale layouts but gives no
 * formulas.  Readings taken here:
 *   - E4M3 is the 8-bit floating-point format with sign bit 7, exponent bits
 *     6..3 (bias 7) and mantissa bits 2..0: exponent 0 gives the subnormals
 *     (m/8) * 2^-6, exponents 1..15 give (1 + m/8) * 2^(e-7), and the two codes
 *     with all of exponent and mantissa set (0x7F, 0xFF) are NaN; there are no
 *     infinities (largest finite value 448).
 *   - The weight is w[n, k] = E4M3(q[n, k]) * scale, the scale taken from:
 *       format 0, per-row:   f32 [N], scale[n];
 *       format 1, per-block: BF16 [ceil(N/BS), ceil(K/BS)], scale[n/BS][k/BS];
 *       format 2, per-block: the same shape in f32 (the page gives the block
 *                            scales as BF16 in its format list and as FP32 in
 *                            its transpose method; both are accepted);
 *       format 3, single:    one global f32 value (the page bakes it into the
 *                            kernel; here it is an argument).
 *   - y[n] = sum_k w[n, k] x[k] for BF16 x, evaluated in fp64 ascending k; the
 *     decoded value (4 significant bits) times an f32 or BF16 scale, and that
 *     times a BF16 x, are exact in fp64, so only the sum rounds. */
double orc_e4m3_to_f64(uint8_t c) {
  const int sign = (c >> 7) & 1, e = (c >> 3) & 0xF, m = c & 7;
  double v;
  if (e == 0xF && m == 7) return NAN;
  if (e == 0)
    v = ldexp((double)m / 8.0, -6);
  else
    v = ldexp(1.0 + (double)m / 8.0, e - 7);
  return sign ? -v : v;
}

static double fp8_scale(const void *scale, int fmt, int64_t bs, double single, int64_t n, int64_t k, int64_t K) {
  switch (fmt) {
    case 0: return (double)((const float *)scale)[n];
    case 1: {
      const int64_t kb = (K + bs - 1) / bs;
      return (double)orc_bf16_to_f32(((const uint16_t *)scale)[(n / bs) * kb + k / bs]);
    }
    case 2: {
      const int64_t kb = (K + bs - 1) / bs;
      return (double)((const float *)scale)[(n / bs) * kb + k / bs];
    }
    default: return single;
  }
}

void orc_fp8_gemv(const uint8_t *w, const void *scale, int64_t N, int64_t K, int fmt, int64_t bs, double single,
                  const uint16_t *x, double *y, double *Aabs) {
#pragma omp parallel for schedule(static)
  for (int64_t n = 0; n < N; ++n) {
    double sum = 0.0, sum_abs = 0.0;
    for (int64_t k = 0; k < K; ++k) {
      const double wv = orc_e4m3_to_f64(w[n * K + k]) * fp8_scale(scale, fmt, bs, single, n, k, K);
      const double t = wv * (double)orc_bf16_to_f32(x[k]);
      sum += t;
      sum_abs += fabs(t);
    }
    y[n] = sum;
    Aabs[n] = sum_abs;
  }
}

int orc_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* Threads for the row loops from now on (timing the oracle at 1 thread and at
 * all cores); results do not depend on it. */
void orc_set_threads(int n) {
#ifdef _OPENMP
  if (n > 0) omp_set_num_threads(n);
#else
  (void)n;
#endif
}
