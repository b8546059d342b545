// gemm_prefill.hip -- Y = X W^T for many rows (prefill) on gfx950 matrix
// cores (rustdoc page "MlxInt8Weight", method gemm: X BF16 [m, in_features],
// Y BF16 [m, out_features]).
//
// A dense contraction, bound by v_mfma_f32_16x16x32_bf16 throughput:
//  * Block tile BM x BN = 128 x 128 outputs, K step 64, 4 waves (2 x 2), each
//    wave 64 x 64 outputs = 4 x 4 MFMA tiles of 16 x 16, fp32 accumulators.
//  * Per K step the block stages a 128 x 64 BF16 tile of X and a 128 x 64
//    tile of the weight into LDS.  The weight arrives as codes (16 per lane,
//    one 16-byte load) and is dequantized on the way in: w = q*s + b in fp32
//    (one FMA), rounded to BF16 nearest-even -- the same values
//    dequantize_to writes.  Each code is thus dequantized once per block and
//    reused by all 128 rows of X in the block.
//  * LDS is double-buffered: the next step's global loads are in flight while
//    the MFMAs consume the current buffer; one barrier per step.
//  * LDS rows are 128 B (64 BF16); 16-byte chunk c of row r is stored at
//    chunk c ^ (r & 7), so the 16 lanes reading 16 consecutive rows of one
//    chunk hit distinct banks.
//  * Work order: the M tiles of one N tile are consecutive, and consecutive
//    work items are kept on one XCD (workgroups are dealt round-robin over
//    the 8 XCDs), so the blocks sharing a weight tile share an L2.
#include "common.h"
#include "launch.h"

namespace int8w {

namespace {

constexpr int kPfThreads = 256;
constexpr int BM = 128, BN = 128, BK = 64;
constexpr int kXcds = 8;

__device__ __forceinline__ uint32_t swz(uint32_t row, uint32_t chunk) {
  return row * (BK * 2) + ((chunk ^ (row & 7u)) << 4);
}

__global__ __launch_bounds__(kPfThreads) void k_gemm_prefill(
    const uint8_t *__restrict__ codes, const uint16_t *__restrict__ scales,
    const uint16_t *__restrict__ biases, const uint16_t *__restrict__ X, uint16_t *__restrict__ Y,
    uint32_t N, uint32_t K, uint32_t m, uint32_t gs_log2, uint32_t mtiles, uint32_t nwork) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[2][(BM + BN) * BK * 2];

  // ---- work item: XCD-grouped, M-fastest
  uint32_t bid = blockIdx.x;
  if (nwork % kXcds == 0) bid = (bid % kXcds) * (nwork / kXcds) + bid / kXcds;
  const uint32_t mt = bid % mtiles, nt = bid / mtiles;
  const uint32_t m0 = mt * BM, n0 = nt * BN;

  const uint32_t tid = threadIdx.x;
  const uint32_t lane = tid & 63u, wave = tid >> 6;
  const uint32_t wm = wave >> 1, wn = wave & 1u;
  const uint32_t G = K >> gs_log2;
  const uint32_t ksteps = (K + BK - 1) / BK;

  // global->LDS assignment
  // X: 4 passes of 32 rows, 8 threads per row, 8 BF16 (16 B) each
  const uint32_t xr = tid >> 3, xc = tid & 7u;
  // W: 2 passes of 64 rows, 4 threads per row, 16 codes each
  const uint32_t wr = tid >> 2, wp = tid & 3u;

  uint4 xreg[4];
  uint4 wreg[2];
  float wsc[2], wbi[2];

  auto load_tile = [&](uint32_t k0) {
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const uint32_t row = m0 + p * 32u + xr;
      const uint32_t k = k0 + xc * 8u;
      xreg[p] = (row < m && k < K) ? *reinterpret_cast<const uint4 *>(X + (size_t)row * K + k)
                                   : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const uint32_t row = n0 + p * 64u + wr;
      const uint32_t k = k0 + wp * 16u;
      if (row < N && k < K) {
        wreg[p] = load_nt(reinterpret_cast<const uint4 *>(codes + (size_t)row * K + k));
        const size_t gi = (size_t)row * G + (k >> gs_log2);
        wsc[p] = bf16_bits_to_f32(scales[gi]);
        wbi[p] = bf16_bits_to_f32(biases[gi]);
      } else {
        wreg[p] = make_uint4(0, 0, 0, 0);
        wsc[p] = 0.f;  // q*0 + 0 = 0: padding contributes nothing
        wbi[p] = 0.f;
      }
    }
  };

  auto store_tile = [&](uint8_t *buf, uint32_t k0) {
    uint8_t *xs = buf;
    uint8_t *ws = buf + BM * BK * 2;
#pragma unroll
    for (int p = 0; p < 4; ++p)
      *reinterpret_cast<uint4 *>(xs + swz(p * 32u + xr, xc)) = xreg[p];
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const uint32_t word[4] = {wreg[p].x, wreg[p].y, wreg[p].z, wreg[p].w};
      uint32_t o[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        o[2 * i] = pack_bf16x2(__builtin_fmaf(code_f32(word[i], 0), wsc[p], wbi[p]),
                               __builtin_fmaf(code_f32(word[i], 1), wsc[p], wbi[p]));
        o[2 * i + 1] = pack_bf16x2(__builtin_fmaf(code_f32(word[i], 2), wsc[p], wbi[p]),
                                   __builtin_fmaf(code_f32(word[i], 3), wsc[p], wbi[p]));
      }
      const uint32_t row = p * 64u + wr;
      *reinterpret_cast<uint4 *>(ws + swz(row, 2u * wp)) = make_uint4(o[0], o[1], o[2], o[3]);
      *reinterpret_cast<uint4 *>(ws + swz(row, 2u * wp + 1u)) = make_uint4(o[4], o[5], o[6], o[7]);
    }
    (void)k0;
  };

  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  load_tile(0);
  store_tile(lds[0], 0);
  __syncthreads();

  const uint32_t lr = lane & 15u, lg = lane >> 4;
  for (uint32_t ks = 0; ks < ksteps; ++ks) {
    const bool more = ks + 1 < ksteps;
    if (more) load_tile((ks + 1) * BK);
    const uint8_t *xs = lds[ks & 1];
    const uint8_t *ws = xs + BM * BK * 2;
#pragma unroll
    for (int kh = 0; kh < 2; ++kh) {
      const uint32_t chunk = 4u * kh + lg;
      bf16x8 a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        a[i] = *reinterpret_cast<const bf16x8 *>(xs + swz(wm * 64u + 16u * i + lr, chunk));
#pragma unroll
      for (int j = 0; j < 4; ++j)
        b[j] = *reinterpret_cast<const bf16x8 *>(ws + swz(wn * 64u + 16u * j + lr, chunk));
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
    }
    if (more) store_tile(lds[(ks + 1) & 1], (ks + 1) * BK);
    __syncthreads();
  }

  // ---- epilogue: lane holds D[4*lg + r][lr] of each 16 x 16 tile
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t n = n0 + wn * 64u + 16u * j + lr;
      if (n >= N) continue;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const uint32_t row = m0 + wm * 64u + 16u * i + 4u * lg + r;
        if (row < m) Y[(size_t)row * N + n] = to_bf16_bits(acc[i][j][r]);
      }
    }
  }
}

}  // namespace

hipError_t launch_gemm_prefill(const WeightView &w, const uint16_t *X, uint16_t *Y, uint32_t m,
                               hipStream_t stream) {
  const uint32_t mtiles = (m + BM - 1) / BM;
  const uint32_t ntiles = (w.N + BN - 1) / BN;
  const uint32_t nwork = mtiles * ntiles;
  hipLaunchKernelGGL(k_gemm_prefill, dim3(nwork), dim3(kPfThreads), 0, stream,
                     reinterpret_cast<const uint8_t *>(w.packed), w.scales, w.biases, X, Y, w.N, w.K, m,
                     (uint32_t)__builtin_ctz(w.gs), mtiles, nwork);
  return hipGetLastError();
}

}  // namespace int8w
