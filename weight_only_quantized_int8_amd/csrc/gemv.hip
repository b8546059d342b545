// gemv.hip -- m = 1 products for gfx950 (rustdoc page "MlxInt8Weight",
// methods gemv, gemv_silu_gate and gemv_silu_gate_resid):
//   gemv                  y[n] = sum_k w[n,k] x[k]
//   gemv_silu_gate        y[n] = sum_k w[n,k] silu(gate[k]) up[k]
//   gemv_silu_gate_resid  y[n] = x_resid[n] + sum_k w[n,k] silu(gate[k]) up[k]
// with w[n,k] = q[n,k] * s[n, k/gs] + b[n, k/gs].
//
// Design (HBM-bound: the codes are ~94% of the bytes at gs = 64):
//  * The activation a[k] (x, or silu(gate)*up in fp32) is formed once per
//    workgroup and K-tile into LDS, together with the sum of each run of 16
//    activations.  The gated product therefore never leaves the chip and its
//    exp/divide cost is shared by every row of the workgroup.
//  * Each lane owns runs of 16 consecutive codes (one 16-byte load), so one
//    wave-wide load streams 1 KiB of a row, fully coalesced, non-temporal.
//  * A run never straddles a group (gs is a multiple of 16), so the affine
//    terms factor out of the run:  sum_k (q_k s + b) a_k = s*sum_k q_k a_k +
//    b*sum_k a_k.  Per code: one byte convert and one fp32 FMA; the bias costs
//    nothing per code.
//  * Each wave carries R rows at once (the LDS activation reads are shared by
//    the R rows) and keeps U*R code loads in flight.  Waves of a workgroup
//    may also split K (WK-way) for short, wide matrices; partial sums meet in
//    LDS.  The lane partials are summed with cross-lane shuffles; there are no
//    atomics, so results are deterministic.
//  * fp32 accumulation throughout; the residual is added in fp32 before the
//    one rounding to BF16.
#include "common.h"
#include "launch.h"

namespace int8w {

namespace {

constexpr int kGemvThreads = 512;      // 8 waves
constexpr uint32_t kTileChunksMax = 1024;  // 16384 activations per LDS tile (68 KiB)

template <int EPI, int R, int U>
__global__ __launch_bounds__(kGemvThreads) void k_gemv(
    const uint4 *__restrict__ packed, const uint16_t *__restrict__ scales,
    const uint16_t *__restrict__ biases, const uint16_t *__restrict__ xg,
    const uint16_t *__restrict__ up, const uint16_t *resid, uint16_t *y, uint32_t N, uint32_t K, uint32_t gs_log2, uint32_t wk_split, uint32_t tile_chunks) {
  extern __shared__ float4 lds4[];
  const uint32_t CT = tile_chunks;
  float4 *a4 = lds4;                                  // [4][CT] float4: activation, run-interleaved
  float *csum = reinterpret_cast<float *>(lds4 + 4 * CT);  // [CT] run sums

  const uint32_t lane = threadIdx.x & 63u;
  const uint32_t wave = threadIdx.x >> 6;
  const uint32_t WK = wk_split;
  const uint32_t WR = (blockDim.x >> 6) / WK;
  const uint32_t wr = wave / WK, wk = wave % WK;
  const uint32_t row0 = (blockIdx.x * WR + wr) * R;
  const uint32_t cpr = K >> 4;        // 16-code runs per row
  const uint32_t G = K >> gs_log2;    // groups per row

  float acc[R];
#pragma unroll
  for (int i = 0; i < R; ++i) acc[i] = 0.f;

  for (uint32_t t0 = 0; t0 < cpr; t0 += CT) {
    const uint32_t ct = (cpr - t0) < CT ? (cpr - t0) : CT;
    if (t0) __syncthreads();
    // ---- stage the activation tile into LDS
    for (uint32_t e = threadIdx.x; e < ct; e += blockDim.x) {
      const uint32_t c = t0 + e;
      const uint4 *src = reinterpret_cast<const uint4 *>(xg) + 2 * c;
      uint4 v0 = src[0], v1 = src[1];
      const uint32_t wv[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
      float a[16];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        a[2 * i] = bf16_lo(wv[i]);
        a[2 * i + 1] = bf16_hi(wv[i]);
      }
      if constexpr (EPI != kEpiNone) {
        const uint4 *usrc = reinterpret_cast<const uint4 *>(up) + 2 * c;
        uint4 u0 = usrc[0], u1 = usrc[1];
        const uint32_t uw[8] = {u0.x, u0.y, u0.z, u0.w, u1.x, u1.y, u1.z, u1.w};
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          a[2 * i] = silu_mul(a[2 * i], bf16_lo(uw[i]));
          a[2 * i + 1] = silu_mul(a[2 * i + 1], bf16_hi(uw[i]));
        }
      }
      float s = 0.f;
#pragma unroll
      for (int i = 0; i < 16; ++i) s += a[i];
#pragma unroll
      for (int f = 0; f < 4; ++f)
        a4[f * CT + e] = make_float4(a[4 * f], a[4 * f + 1], a[4 * f + 2], a[4 * f + 3]);
      csum[e] = s;
    }
    __syncthreads();

    // ---- stream the code rows of this tile
    for (uint32_t jb = wk * 64u; jb < ct; jb += WK * 64u * U) {
      uint4 q[U][R];
      float sc[U][R], bi[U][R];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const uint32_t e = jb + u * WK * 64u + lane;
        const uint32_t c = t0 + e;
        const bool valid = e < ct;
        const uint32_t g = (c << 4) >> gs_log2;
#pragma unroll
        for (int i = 0; i < R; ++i) {
          const uint32_t row = row0 + i;
          if (valid && row < N) {
            q[u][i] = load_nt(packed + (size_t)row * cpr + c);
            sc[u][i] = bf16_bits_to_f32(scales[(size_t)row * G + g]);
            bi[u][i] = bf16_bits_to_f32(biases[(size_t)row * G + g]);
          } else {
            q[u][i] = make_uint4(0, 0, 0, 0);
            sc[u][i] = 0.f;
            bi[u][i] = 0.f;
          }
        }
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const uint32_t e = jb + u * WK * 64u + lane;
        if (e < ct) {
          const float4 a0 = a4[e], a1 = a4[CT + e], a2 = a4[2 * CT + e], a3 = a4[3 * CT + e];
          const float S = csum[e];
#pragma unroll
          for (int i = 0; i < R; ++i) {
            const uint4 w = q[u][i];
            float p = code_f32(w.x, 0) * a0.x;
            p = __builtin_fmaf(code_f32(w.x, 1), a0.y, p);
            p = __builtin_fmaf(code_f32(w.x, 2), a0.z, p);
            p = __builtin_fmaf(code_f32(w.x, 3), a0.w, p);
            p = __builtin_fmaf(code_f32(w.y, 0), a1.x, p);
            p = __builtin_fmaf(code_f32(w.y, 1), a1.y, p);
            p = __builtin_fmaf(code_f32(w.y, 2), a1.z, p);
            p = __builtin_fmaf(code_f32(w.y, 3), a1.w, p);
            p = __builtin_fmaf(code_f32(w.z, 0), a2.x, p);
            p = __builtin_fmaf(code_f32(w.z, 1), a2.y, p);
            p = __builtin_fmaf(code_f32(w.z, 2), a2.z, p);
            p = __builtin_fmaf(code_f32(w.z, 3), a2.w, p);
            p = __builtin_fmaf(code_f32(w.w, 0), a3.x, p);
            p = __builtin_fmaf(code_f32(w.w, 1), a3.y, p);
            p = __builtin_fmaf(code_f32(w.w, 2), a3.z, p);
            p = __builtin_fmaf(code_f32(w.w, 3), a3.w, p);
            acc[i] = __builtin_fmaf(sc[u][i], p, __builtin_fmaf(bi[u][i], S, acc[i]));
          }
        }
      }
    }
  }

  // ---- reduce the lane partials, then the K-split partials, then store
#pragma unroll
  for (int i = 0; i < R; ++i) acc[i] = wave_sum(acc[i]);

  float mine = 0.f;  // lane i < R keeps row i's total
#pragma unroll
  for (int i = 0; i < R; ++i)
    if (lane == (uint32_t)i) mine = acc[i];

  if (WK > 1) {
    __syncthreads();
    float *red = reinterpret_cast<float *>(lds4);
    if (lane < (uint32_t)R) red[(wr * WK + wk) * R + lane] = mine;
    __syncthreads();
    if (wk != 0) return;
    if (lane < (uint32_t)R) {
      float t = 0.f;
      for (uint32_t j = 0; j < WK; ++j) t += red[(wr * WK + j) * R + lane];
      mine = t;
    }
  }
  if (lane < (uint32_t)R) {
    const uint32_t row = row0 + lane;
    if (row < N) {
      float v = mine;
      if constexpr (EPI == kEpiSiluGateResid) v += bf16_bits_to_f32(resid[row]);
      y[row] = to_bf16_bits(v);
    }
  }
}

template <int EPI, int R>
hipError_t launch_r(dim3 grid, size_t lds, hipStream_t stream, const WeightView &w,
                    const uint16_t *xg, const uint16_t *up, const uint16_t *resid, uint16_t *y,
                    uint32_t wk, uint32_t ct) {
  constexpr int U = 2;
  auto kern = k_gemv<EPI, R, U>;
  static bool configured = false;  // raise the dynamic-LDS cap once per instantiation
  if (!configured) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
    if (e != hipSuccess) return e;
    configured = true;
  }
  hipLaunchKernelGGL(kern, grid, dim3(kGemvThreads), lds, stream,
                     reinterpret_cast<const uint4 *>(w.packed), w.scales, w.biases, xg, up, resid,
                     y, w.N, w.K, (uint32_t)__builtin_ctz(w.gs), wk, ct);
  return hipGetLastError();
}

template <int EPI>
hipError_t launch_epi(int R, dim3 grid, size_t lds, hipStream_t stream, const WeightView &w,
                      const uint16_t *xg, const uint16_t *up, const uint16_t *resid, uint16_t *y,
                      uint32_t wk, uint32_t ct) {
  switch (R) {
    case 1: return launch_r<EPI, 1>(grid, lds, stream, w, xg, up, resid, y, wk, ct);
    case 2: return launch_r<EPI, 2>(grid, lds, stream, w, xg, up, resid, y, wk, ct);
    case 3: return launch_r<EPI, 3>(grid, lds, stream, w, xg, up, resid, y, wk, ct);
    case 4: return launch_r<EPI, 4>(grid, lds, stream, w, xg, up, resid, y, wk, ct);
    case 5: return launch_r<EPI, 5>(grid, lds, stream, w, xg, up, resid, y, wk, ct);
    case 6: return launch_r<EPI, 6>(grid, lds, stream, w, xg, up, resid, y, wk, ct);
    case 7: return launch_r<EPI, 7>(grid, lds, stream, w, xg, up, resid, y, wk, ct);
    default: return launch_r<EPI, 8>(grid, lds, stream, w, xg, up, resid, y, wk, ct);
  }
}

}  // namespace

hipError_t launch_gemv(const WeightView &w, GemvEpilogue epi, const uint16_t *x_or_gate,
                       const uint16_t *up, const uint16_t *x_resid, uint16_t *y,
                       hipStream_t stream) {
  const uint32_t waves = kGemvThreads / 64;
  const uint32_t cus = (uint32_t)device_cu_count();
  // Rows are spread so that one workgroup of 8 waves per CU covers N: each
  // wave carries R rows, or, for short matrices, waves split K instead.
  uint32_t R = 1, wk = 1;
  if (w.N >= cus * waves) {
    R = (w.N + cus * waves - 1) / (cus * waves);
    if (R > 8) R = 8;
  } else {
    uint32_t rows_per_wg = (w.N + cus - 1) / cus;  // 1 .. waves-1
    uint32_t wr = 1;
    while (wr < rows_per_wg && wr < waves) wr <<= 1;
    wk = waves / wr;
  }
  const uint32_t rows_per_block = (waves / wk) * R;
  const uint32_t blocks = (w.N + rows_per_block - 1) / rows_per_block;
  const uint32_t cpr = w.K / 16u;
  uint32_t ntiles = (cpr + kTileChunksMax - 1) / kTileChunksMax;
  uint32_t ct = (cpr + ntiles - 1) / ntiles;
  size_t lds = (size_t)ct * 68u;
  size_t red = (size_t)waves * R * sizeof(float);
  if (lds < red) lds = red;
  switch (epi) {
    case kEpiNone:
      return launch_epi<kEpiNone>(R, dim3(blocks), lds, stream, w, x_or_gate, nullptr, nullptr, y, wk, ct);
    case kEpiSiluGate:
      return launch_epi<kEpiSiluGate>(R, dim3(blocks), lds, stream, w, x_or_gate, up, nullptr, y, wk, ct);
    default:
      return launch_epi<kEpiSiluGateResid>(R, dim3(blocks), lds, stream, w, x_or_gate, up, x_resid, y, wk, ct);
  }
}

}  // namespace int8w
