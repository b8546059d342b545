// gemm_smallm.hip -- Y = X W^T for 2 <= m <= 16 rows on gfx950 matrix cores
// (rustdoc page "MlxInt8Weight", method gemm: X BF16 [m, in_features],
// Y BF16 [m, out_features]).
//
// Still HBM-bound (each code byte is read once and used m times), but m fp32
// FMAs per code would swamp the vector ALUs, so the products go to
// v_mfma_f32_16x16x32_bf16:
//  * The raw codes 0..255 are exact in BF16 (8 significant bits), so they
//    enter the MFMA unscaled; the affine terms are applied per window of 32 or
//    64 codes that lies inside one group:
//        sum_{k in win} (q s + b) x = s * sum q x + b * sum x
//    The first sum is the MFMA on raw codes; the second comes from a second
//    MFMA against a constant all-ones operand, which leaves sum_k X[i,k] in
//    exactly the accumulator lanes that need it.  Products q*x are exact.
//  * MFMA D[i][j] = sum_k A[i][k] B[k][j] with A = X (i: input row, padded to
//    16 with zeros), B = codes (j: weight row).  For this shape lane l holds
//    A[l%16][8*(l/16) .. +7], B[8*(l/16) .. +7][l%16] and D[4*(l/16)+r][l%16].
//    Any lane->k assignment works as long as A and B use the same one.
//  * gs >= 64: a lane loads 16 consecutive codes (16 B) of its weight row per
//    64-code step; the two MFMAs of the step take codes 0..7 and 8..15 of each
//    lane, so a step is one window inside one group.
//    gs == 32: a lane loads 8 codes from each 32-code half of the step, so
//    each MFMA sees exactly one group.
//  * A workgroup of 4 waves owns RT tiles of 16 weight rows; its waves split K
//    into interleaved 64-code steps and meet in LDS at the end (fixed order,
//    no atomics: deterministic).
#include "common.h"
#include "launch.h"

namespace int8w {

namespace {

constexpr int kSmallmThreads = 256;  // 4 waves, K split 4 ways

__device__ __forceinline__ uint32_t codes_to_bf16x2(uint32_t word, int half) {
  // bytes (2*half, 2*half+1) of word -> packed BF16 pair (exact for 0..255)
  return half == 0 ? pack_bf16x2(code_f32(word, 0), code_f32(word, 1))
                   : pack_bf16x2(code_f32(word, 2), code_f32(word, 3));
}

__device__ __forceinline__ bf16x8 codes8_to_bf16x8(uint32_t w0, uint32_t w1) {
  uint4 v = make_uint4(codes_to_bf16x2(w0, 0), codes_to_bf16x2(w0, 1), codes_to_bf16x2(w1, 0),
                       codes_to_bf16x2(w1, 1));
  return __builtin_bit_cast(bf16x8, v);
}

template <int RT, bool G32>
__global__ __launch_bounds__(kSmallmThreads) void k_gemm_smallm(
    const uint8_t *__restrict__ codes, const uint16_t *__restrict__ scales,
    const uint16_t *__restrict__ biases, const uint16_t *__restrict__ X, uint16_t *__restrict__ Y,
    uint32_t N, uint32_t K, uint32_t m, uint32_t gs_log2) {
  __shared__ f32x4 red[4][RT][64];

  const uint32_t lane = threadIdx.x & 63u;
  const uint32_t wave = threadIdx.x >> 6;
  const uint32_t lr = lane & 15u;   // row of A (input row) / column of B (weight row)
  const uint32_t lg = lane >> 4;    // 8-wide k block of this lane
  const uint32_t n0 = blockIdx.x * (16u * RT);
  const uint32_t G = K >> gs_log2;
  const uint32_t steps = (K + 63u) >> 6;

  const bool xrow_ok = lr < m;
  const uint16_t *xrow = X + (size_t)(xrow_ok ? lr : 0) * K;

  const uint8_t *wrow[RT];
  uint32_t nrow[RT];
  bool wrow_ok[RT];
#pragma unroll
  for (int t = 0; t < RT; ++t) {
    nrow[t] = n0 + 16u * t + lr;
    wrow_ok[t] = nrow[t] < N;
    wrow[t] = codes + (size_t)(wrow_ok[t] ? nrow[t] : 0) * K;
  }

  const bf16x8 ones = __builtin_bit_cast(bf16x8, make_uint4(0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u));
  f32x4 acc[RT];
#pragma unroll
  for (int t = 0; t < RT; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (uint32_t st = wave; st < steps; st += 4) {
    const uint32_t k0 = st << 6;
    // ---- loads: X fragments (2 x 8 bf16) and RT weight fragments (16 codes)
    uint4 xa = make_uint4(0, 0, 0, 0), xb = make_uint4(0, 0, 0, 0);
    uint32_t kA, kB;  // first k of the two 8-code pieces of this lane
    if constexpr (G32) {
      kA = k0 + 8u * lg;
      kB = k0 + 32u + 8u * lg;
    } else {
      kA = k0 + 16u * lg;
      kB = kA + 8u;
    }
    const bool okA = kA < K, okB = kB < K;
    if (xrow_ok) {
      if (okA) xa = *reinterpret_cast<const uint4 *>(xrow + kA);
      if (okB) xb = *reinterpret_cast<const uint4 *>(xrow + kB);
    }
    uint32_t wq[RT][4];
    float sA[RT], bA[RT], sB[RT], bB[RT];
#pragma unroll
    for (int t = 0; t < RT; ++t) {
      if constexpr (G32) {
        uint2 pa = make_uint2(0, 0), pb = make_uint2(0, 0);
        if (wrow_ok[t] && okA) pa = load_nt(reinterpret_cast<const uint2 *>(wrow[t] + kA));
        if (wrow_ok[t] && okB) pb = load_nt(reinterpret_cast<const uint2 *>(wrow[t] + kB));
        wq[t][0] = pa.x; wq[t][1] = pa.y; wq[t][2] = pb.x; wq[t][3] = pb.y;
      } else {
        uint4 p = make_uint4(0, 0, 0, 0);
        if (wrow_ok[t] && okA) p = load_nt(reinterpret_cast<const uint4 *>(wrow[t] + kA));
        wq[t][0] = p.x; wq[t][1] = p.y; wq[t][2] = p.z; wq[t][3] = p.w;
      }
      const size_t grow = (size_t)(wrow_ok[t] ? nrow[t] : 0) * G;
      const uint32_t gA = okA ? (kA >> gs_log2) : 0;
      sA[t] = bf16_bits_to_f32(scales[grow + gA]);
      bA[t] = bf16_bits_to_f32(biases[grow + gA]);
      if constexpr (G32) {
        const uint32_t gB = okB ? (kB >> gs_log2) : 0;
        sB[t] = bf16_bits_to_f32(scales[grow + gB]);
        bB[t] = bf16_bits_to_f32(biases[grow + gB]);
      }
    }
    // ---- input sums of the window(s): MFMA against ones
    const bf16x8 xa8 = __builtin_bit_cast(bf16x8, xa), xb8 = __builtin_bit_cast(bf16x8, xb);
    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
    f32x4 SA = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa8, ones, zero, 0, 0, 0);
    f32x4 SB = zero;
    if constexpr (G32) {
      SB = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xb8, ones, zero, 0, 0, 0);
    } else {
      SA = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xb8, ones, SA, 0, 0, 0);
    }
    // ---- raw-code products and per-window affine rescale
#pragma unroll
    for (int t = 0; t < RT; ++t) {
      const bf16x8 qa = codes8_to_bf16x8(wq[t][0], wq[t][1]);
      const bf16x8 qb = codes8_to_bf16x8(wq[t][2], wq[t][3]);
      if constexpr (G32) {
        f32x4 PA = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa8, qa, zero, 0, 0, 0);
        f32x4 PB = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xb8, qb, zero, 0, 0, 0);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float v = __builtin_fmaf(sA[t], PA[r], __builtin_fmaf(bA[t], SA[r], acc[t][r]));
          acc[t][r] = __builtin_fmaf(sB[t], PB[r], __builtin_fmaf(bB[t], SB[r], v));
        }
      } else {
        f32x4 P = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa8, qa, zero, 0, 0, 0);
        P = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xb8, qb, P, 0, 0, 0);
#pragma unroll
        for (int r = 0; r < 4; ++r)
          acc[t][r] = __builtin_fmaf(sA[t], P[r], __builtin_fmaf(bA[t], SA[r], acc[t][r]));
      }
    }
  }

  // ---- combine the 4 K-slices in a fixed order and store
#pragma unroll
  for (int t = 0; t < RT; ++t) red[wave][t][lane] = acc[t];
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int t = 0; t < RT; ++t) {
    f32x4 v = red[0][t][lane];
#pragma unroll
    for (int w = 1; w < 4; ++w) {
      const f32x4 o = red[w][t][lane];
      v[0] += o[0]; v[1] += o[1]; v[2] += o[2]; v[3] += o[3];
    }
    const uint32_t n = n0 + 16u * t + lr;
    if (n < N) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const uint32_t i = 4u * lg + r;
        if (i < m) Y[(size_t)i * N + n] = to_bf16_bits(v[r]);
      }
    }
  }
}

template <int RT>
hipError_t launch_rt(const WeightView &w, const uint16_t *X, uint16_t *Y, uint32_t m, hipStream_t stream) {
  const uint32_t blocks = (w.N + 16u * RT - 1u) / (16u * RT);
  const uint32_t gs_log2 = (uint32_t)__builtin_ctz(w.gs);
  const uint8_t *codes = reinterpret_cast<const uint8_t *>(w.packed);
  if (w.gs == 32)
    hipLaunchKernelGGL((k_gemm_smallm<RT, true>), dim3(blocks), dim3(kSmallmThreads), 0, stream, codes,
                       w.scales, w.biases, X, Y, w.N, w.K, m, gs_log2);
  else
    hipLaunchKernelGGL((k_gemm_smallm<RT, false>), dim3(blocks), dim3(kSmallmThreads), 0, stream, codes,
                       w.scales, w.biases, X, Y, w.N, w.K, m, gs_log2);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_smallm(const WeightView &w, const uint16_t *X, uint16_t *Y, uint32_t m,
                              hipStream_t stream) {
  const uint32_t cus = (uint32_t)device_cu_count();
  // Enough 16-row tiles per workgroup to keep the tile count near 2 per CU.
  const uint32_t tiles = (w.N + 15u) / 16u;
  if (tiles >= 4u * cus) return launch_rt<2>(w, X, Y, m, stream);
  return launch_rt<1>(w, X, Y, m, stream);
}

}  // namespace int8w
