// gemm_prefill.hip -- Y = X W^T for many rows (prefill) on gfx950 matrix
// cores (rustdoc page "MlxInt8Weight", method gemm: X BF16 [m, in_features],
// Y BF16 [m, out_features]).
//
// A dense contraction, bound by v_mfma_f32_16x16x32_bf16 throughput:
//  * Block tile BM x BN = 256 x 128 outputs over 8 waves (4 x 2, each wave
//    64 x 64), or 128 x 128 / 128 x 64 over 4 waves when there are too few
//    large tiles to occupy the CUs; K step 64; MFMA tiles of 16 x 16 with
//    fp32 accumulators.
//  * Per K step the block stages a 128 x 64 BF16 tile of X and a 128 x 64
//    tile of the weight into LDS.  The weight arrives as codes (16 per lane,
//    one 16-byte load) and is dequantized on the way in: w = q*s + b in fp32
//    (one FMA), rounded to BF16 nearest-even -- the same values
//    dequantize_to writes.  Each code is thus dequantized once per block and
//    reused by all 128 rows of X in the block.
//  * Pipeline: the global loads of the next two K steps are in flight in two
//    register sets while the MFMAs consume the LDS copy of the current one;
//    LDS is double-buffered, one barrier per step.  Every global load goes
//    through a bounded buffer resource (past the matrix edges it reads
//    zeros: a zero code with zero scale and bias is a zero weight), so the
//    loop has no branches but its exits.
//  * LDS rows are 128 B (64 BF16); 16-byte chunk c of row r is stored at
//    chunk c ^ (r & 7), so the 16 lanes reading 16 consecutive rows of one
//    chunk hit distinct banks.
//  * Work order: the M tiles of one N tile are consecutive, and consecutive
//    work items are kept on one XCD (workgroups are dealt round-robin over
//    the 8 XCDs), so the blocks sharing a weight tile share an L2.
//  * The large shape (256 x 128) specialises waves: 8 MFMA waves consume step
//    k while producer waves load, dequantize and store a later step, with one
//    barrier per step.  With one workgroup per CU the waves of the
//    single-role design moved in lockstep between an MFMA phase and a
//    dequantize-and-store phase; here the two phases overlap (measured +10 %
//    at m = 2048, MFMA busy 30 % before).  k_gemm_prefill_dma (the usual
//    case, K % (8 gs) == 0) stages X and the scales/biases by DMA over three
//    LDS stages; k_gemm_prefill_ws (any K) loads through registers.
#include <type_traits>

#include "common.h"
#include "launch.h"

namespace int8w {

namespace {

constexpr int BK = 64;
constexpr int kXcds = 8;

__device__ __forceinline__ uint32_t swz(uint32_t row, uint32_t chunk) {
  return row * (BK * 2) + ((chunk ^ (row & 7u)) << 4);
}

__device__ __forceinline__ uint32_t uniform_pf(uint32_t v) { return __builtin_amdgcn_readfirstlane(v); }

// Global loads of one K step held in registers.
template <int XP, int WP>
struct PfRegs {
  u32x4 x[XP];
  u32x4 w[WP];
  uint16_t s[WP], b[WP];
};

// WGM x WGN waves; wave (wm, wn) owns rows wm*BM/WGM.. and columns wn*BN/WGN.. of the tile.
template <int BM, int BN, int WGM, int WGN>
__global__ __launch_bounds__(64 * WGM * WGN) void k_gemm_prefill(
    const uint8_t *__restrict__ codes, const uint16_t *__restrict__ scales,
    const uint16_t *__restrict__ biases, const uint16_t *__restrict__ X, uint16_t *__restrict__ Y,
    uint32_t N, uint32_t K, uint32_t m, uint32_t gs_log2, uint32_t mtiles, uint32_t nwork) {
  constexpr int kThreads = 64 * WGM * WGN;
  constexpr int XR = kThreads / 8;  // X rows per load pass (8 chunks of 16 B per row)
  constexpr int WR = kThreads / 4;  // weight rows per load pass (4 chunks of 16 codes per row)
  constexpr int XP = BM / XR;       // X loads per thread per step
  constexpr int WP = BN / WR;       // weight loads per thread per step
  constexpr int WTM = BM / WGM, WTN = BN / WGN;  // wave tile
  constexpr int TI = WTM / 16;      // 16-row MFMA tiles per wave
  constexpr int TJ = WTN / 16;      // 16-column MFMA tiles per wave
  static_assert(XP >= 1 && WP >= 1 && BM % XR == 0 && BN % WR == 0, "whole load passes");
  constexpr uint32_t kStage = (BM + BN) * BK * 2;
  extern __shared__ __attribute__((aligned(16))) uint8_t lds_pf[];
  uint8_t *lds[2] = {lds_pf, lds_pf + kStage};

  // ---- work item: XCD-grouped, M-fastest
  uint32_t bid = blockIdx.x;
  if (nwork % kXcds == 0) bid = (bid % kXcds) * (nwork / kXcds) + bid / kXcds;
  const uint32_t mt = bid % mtiles, nt = bid / mtiles;
  const uint32_t m0 = mt * BM, n0 = nt * BN;

  const uint32_t tid = threadIdx.x;
  const uint32_t lane = tid & 63u, wave = tid >> 6;
  const uint32_t wm = wave / WGN, wn = wave % WGN;
  const uint32_t G = K >> gs_log2;
  const uint32_t ksteps = (K + BK - 1) / BK;
  const uint32_t mrows = m - m0 < (uint32_t)BM ? m - m0 : (uint32_t)BM;
  const uint32_t nrows = N - n0 < (uint32_t)BN ? N - n0 : (uint32_t)BN;

  // bounded views of this tile's rows; the step's k is the uniform soffset
  const auto rx = make_rsrc(X + (size_t)m0 * K, mrows * K * 2u);
  const auto rw = make_rsrc(codes + (size_t)n0 * K, nrows * K);
  const auto rs = make_rsrc(scales + (size_t)n0 * G, nrows * G * 2u);
  const auto rb = make_rsrc(biases + (size_t)n0 * G, nrows * G * 2u);

  // global->LDS assignment
  // X: XP passes of XR rows, 8 threads per row, 8 BF16 (16 B) each
  const uint32_t xr = tid >> 3, xc = tid & 7u;
  // W: WP passes of WR rows, 4 threads per row, 16 codes each (one group)
  const uint32_t wr = tid >> 2, wp = tid & 3u;
  uint32_t vx[XP], vw[WP], vsb[WP];
#pragma unroll
  for (int p = 0; p < XP; ++p) {
    const uint32_t row = p * XR + xr;
    vx[p] = row < mrows ? row * K * 2u + xc * 16u : kOutOfRange;
  }
#pragma unroll
  for (int p = 0; p < WP; ++p) {
    const uint32_t row = p * WR + wr;
    vw[p] = row < nrows ? row * K + wp * 16u : kOutOfRange;
    vsb[p] = row < nrows ? row * G * 2u : kOutOfRange;
  }

  using Regs = PfRegs<XP, WP>;
  auto issue = [&](Regs &r, uint32_t ks) {
    const bool live = ks < ksteps;
    const uint32_t k0 = live ? ks * BK : 0u;
    const bool xin = live && k0 + xc * 8u < K;
    const bool win = live && k0 + wp * 16u < K;
#pragma unroll
    for (int p = 0; p < XP; ++p)
      r.x[p] = __builtin_amdgcn_raw_buffer_load_b128(rx, (int)(xin ? vx[p] : kOutOfRange), (int)uniform_pf(2u * k0), 0);
#pragma unroll
    for (int p = 0; p < WP; ++p) {
      r.w[p] = __builtin_amdgcn_raw_buffer_load_b128(rw, (int)(win ? vw[p] : kOutOfRange), (int)uniform_pf(k0),
                                                     kAuxNontemporal);
      // the lane's 16 codes lie in one group (gs >= 32)
      const uint32_t go = win ? vsb[p] + 2u * ((k0 + wp * 16u) >> gs_log2) : kOutOfRange;
      r.s[p] = __builtin_amdgcn_raw_buffer_load_b16(rs, (int)go, 0, 0);
      r.b[p] = __builtin_amdgcn_raw_buffer_load_b16(rb, (int)go, 0, 0);
    }
  };

  auto store = [&](const Regs &r, uint8_t *buf) {
    uint8_t *xs = buf;
    uint8_t *ws = buf + BM * BK * 2;
#pragma unroll
    for (int p = 0; p < XP; ++p) *reinterpret_cast<u32x4 *>(xs + swz(p * XR + xr, xc)) = r.x[p];
#pragma unroll
    for (int p = 0; p < WP; ++p) {
      const float sc = bf16_bits_to_f32(r.s[p]), bi = bf16_bits_to_f32(r.b[p]);
      const uint32_t word[4] = {r.w[p].x, r.w[p].y, r.w[p].z, r.w[p].w};
      uint32_t o[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        o[2 * i] = pack_bf16x2(__builtin_fmaf(code_f32(word[i], 0), sc, bi), __builtin_fmaf(code_f32(word[i], 1), sc, bi));
        o[2 * i + 1] =
            pack_bf16x2(__builtin_fmaf(code_f32(word[i], 2), sc, bi), __builtin_fmaf(code_f32(word[i], 3), sc, bi));
      }
      const uint32_t row = p * WR + wr;
      *reinterpret_cast<u32x4 *>(ws + swz(row, 2u * wp)) = u32x4{o[0], o[1], o[2], o[3]};
      *reinterpret_cast<u32x4 *>(ws + swz(row, 2u * wp + 1u)) = u32x4{o[4], o[5], o[6], o[7]};
    }
  };

  f32x4 acc[TI][TJ];
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int j = 0; j < TJ; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const uint32_t lr = lane & 15u, lg = lane >> 4;
  auto compute = [&](const uint8_t *buf) {
    const uint8_t *xs = buf;
    const uint8_t *ws = buf + BM * BK * 2;
#pragma unroll
    for (int kh = 0; kh < 2; ++kh) {
      const uint32_t chunk = 4u * kh + lg;
      bf16x8 a[TI], b[TJ];
#pragma unroll
      for (int i = 0; i < TI; ++i)
        a[i] = *reinterpret_cast<const bf16x8 *>(xs + swz(wm * WTM + 16u * i + lr, chunk));
#pragma unroll
      for (int j = 0; j < TJ; ++j)
        b[j] = *reinterpret_cast<const bf16x8 *>(ws + swz(wn * WTN + 16u * j + lr, chunk));
#pragma unroll
      for (int i = 0; i < TI; ++i)
#pragma unroll
        for (int j = 0; j < TJ; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
    }
  };

  // ---- pipeline: R0/R1 hold steps ks+1 and ks+2 in flight while step ks is
  // consumed from LDS; the only branches are the loop exits
  Regs R0, R1;
  issue(R0, 0);
  issue(R1, 1);
  store(R0, lds[0]);
  __syncthreads();
  issue(R0, 2);
  for (uint32_t ks = 0;;) {
    compute(lds[ks & 1u]);
    if (ks + 1u >= ksteps) break;
    store(R1, lds[(ks + 1u) & 1u]);
    __syncthreads();
    issue(R1, ks + 3u);
    ++ks;
    compute(lds[ks & 1u]);
    if (ks + 1u >= ksteps) break;
    store(R0, lds[(ks + 1u) & 1u]);
    __syncthreads();
    issue(R0, ks + 3u);
    ++ks;
  }

  // ---- epilogue: lane holds D[4*lg + r][lr] of each 16 x 16 tile
#pragma unroll
  for (int i = 0; i < TI; ++i) {
#pragma unroll
    for (int j = 0; j < TJ; ++j) {
      const uint32_t n = n0 + wn * WTN + 16u * j + lr;
      if (n >= N) continue;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const uint32_t row = m0 + wm * WTM + 16u * i + 4u * lg + r;
        if (row < m) Y[(size_t)row * N + n] = to_bf16_bits(acc[i][j][r]);
      }
    }
  }
}

// Wave-specialised variant: WGM x WGN MFMA waves and NP producer waves.  The
// producers load, dequantize and store step k+1 into one LDS buffer while
// the MFMA waves consume step k from the other; one workgroup barrier per
// step.  Each role runs its own loop with the same number of barriers.
template <int BM, int BN, int WGM, int WGN, int NP>
__global__ __launch_bounds__(64 * (WGM * WGN + NP)) void k_gemm_prefill_ws(
    const uint8_t *__restrict__ codes, const uint16_t *__restrict__ scales,
    const uint16_t *__restrict__ biases, const uint16_t *__restrict__ X, uint16_t *__restrict__ Y,
    uint32_t N, uint32_t K, uint32_t m, uint32_t gs_log2, uint32_t mtiles, uint32_t nwork) {
  constexpr int kMma = WGM * WGN;          // MFMA waves
  constexpr int kPT = 64 * NP;             // producer threads
  constexpr int XR = kPT / 8;              // X rows per producer pass
  constexpr int WR = kPT / 4;              // weight rows per producer pass
  constexpr int XP = BM / XR;
  constexpr int WP = BN / WR;
  constexpr int WTM = BM / WGM, WTN = BN / WGN;
  constexpr int TI = WTM / 16, TJ = WTN / 16;
  static_assert(XP >= 1 && WP >= 1 && BM % XR == 0 && BN % WR == 0, "whole load passes");
  constexpr uint32_t kStage = (BM + BN) * BK * 2;
  extern __shared__ __attribute__((aligned(16))) uint8_t lds_pf[];
  auto lds = [&](uint32_t i) { return lds_pf + (i ? kStage : 0u); };

  uint32_t bid = blockIdx.x;
  if (nwork % kXcds == 0) bid = (bid % kXcds) * (nwork / kXcds) + bid / kXcds;
  const uint32_t mt = bid % mtiles, nt = bid / mtiles;
  const uint32_t m0 = mt * BM, n0 = nt * BN;
  const uint32_t tid = threadIdx.x;
  const uint32_t lane = tid & 63u, wave = uniform_pf(tid >> 6);
  const uint32_t ksteps = (K + BK - 1) / BK;

  if (wave >= (uint32_t)kMma) {
    // ---------------- producer waves
    const uint32_t ptid = tid - 64u * kMma;
    const uint32_t G = K >> gs_log2;
    const uint32_t mrows = m - m0 < (uint32_t)BM ? m - m0 : (uint32_t)BM;
    const uint32_t nrows = N - n0 < (uint32_t)BN ? N - n0 : (uint32_t)BN;
    const auto rx = make_rsrc(X + (size_t)m0 * K, mrows * K * 2u);
    const auto rw = make_rsrc(codes + (size_t)n0 * K, nrows * K);
    const auto rs = make_rsrc(scales + (size_t)n0 * G, nrows * G * 2u);
    const auto rb = make_rsrc(biases + (size_t)n0 * G, nrows * G * 2u);
    const uint32_t xr = ptid >> 3, xc = ptid & 7u;
    const uint32_t wr = ptid >> 2, wp = ptid & 3u;
    uint32_t vx[XP], vw[WP], vsb[WP];
#pragma unroll
    for (int p = 0; p < XP; ++p) {
      const uint32_t row = p * XR + xr;
      vx[p] = row < mrows ? row * K * 2u + xc * 16u : kOutOfRange;
    }
#pragma unroll
    for (int p = 0; p < WP; ++p) {
      const uint32_t row = p * WR + wr;
      vw[p] = row < nrows ? row * K + wp * 16u : kOutOfRange;
      vsb[p] = row < nrows ? row * G * 2u : kOutOfRange;
    }
    using Regs = PfRegs<XP, WP>;
    auto issue = [&](Regs &r, uint32_t ks) {
      const bool live = ks < ksteps;
      const uint32_t k0 = live ? ks * BK : 0u;
      const bool xin = live && k0 + xc * 8u < K;
      const bool win = live && k0 + wp * 16u < K;
#pragma unroll
      for (int p = 0; p < XP; ++p)
        r.x[p] = __builtin_amdgcn_raw_buffer_load_b128(rx, (int)(xin ? vx[p] : kOutOfRange), (int)uniform_pf(2u * k0), 0);
#pragma unroll
      for (int p = 0; p < WP; ++p) {
        r.w[p] = __builtin_amdgcn_raw_buffer_load_b128(rw, (int)(win ? vw[p] : kOutOfRange), (int)uniform_pf(k0),
                                                       kAuxNontemporal);
        const uint32_t go = win ? vsb[p] + 2u * ((k0 + wp * 16u) >> gs_log2) : kOutOfRange;
        r.s[p] = __builtin_amdgcn_raw_buffer_load_b16(rs, (int)go, 0, 0);
        r.b[p] = __builtin_amdgcn_raw_buffer_load_b16(rb, (int)go, 0, 0);
      }
    };
    auto store = [&](const Regs &r, uint8_t *buf) {
      uint8_t *xs = buf;
      uint8_t *ws = buf + BM * BK * 2;
#pragma unroll
      for (int p = 0; p < XP; ++p) *reinterpret_cast<u32x4 *>(xs + swz(p * XR + xr, xc)) = r.x[p];
#pragma unroll
      for (int p = 0; p < WP; ++p) {
        const float sc = bf16_bits_to_f32(r.s[p]), bi = bf16_bits_to_f32(r.b[p]);
        const uint32_t word[4] = {r.w[p].x, r.w[p].y, r.w[p].z, r.w[p].w};
        uint32_t o[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          o[2 * i] = pack_bf16x2(__builtin_fmaf(code_f32(word[i], 0), sc, bi), __builtin_fmaf(code_f32(word[i], 1), sc, bi));
          o[2 * i + 1] =
              pack_bf16x2(__builtin_fmaf(code_f32(word[i], 2), sc, bi), __builtin_fmaf(code_f32(word[i], 3), sc, bi));
        }
        const uint32_t row = p * WR + wr;
        *reinterpret_cast<u32x4 *>(ws + swz(row, 2u * wp)) = u32x4{o[0], o[1], o[2], o[3]};
        *reinterpret_cast<u32x4 *>(ws + swz(row, 2u * wp + 1u)) = u32x4{o[4], o[5], o[6], o[7]};
      }
    };
    Regs R0, R1;
    issue(R0, 0);
    issue(R1, 1);
    store(R0, lds(0u));
    __syncthreads();  // step 0 is in LDS
    issue(R0, 2);
    // while the MFMA waves consume step k, store step k + 1 and request k + 3
    for (uint32_t k = 0;;) {
      if (k + 1u >= ksteps) break;
      store(R1, lds((k + 1u) & 1u));
      issue(R1, k + 3u);
      __syncthreads();
      ++k;
      if (k + 1u >= ksteps) break;
      store(R0, lds((k + 1u) & 1u));
      issue(R0, k + 3u);
      __syncthreads();
      ++k;
    }
    return;
  }

  // ---------------- MFMA waves
  const uint32_t wm = wave / WGN, wn = wave % WGN;
  f32x4 acc[TI][TJ];
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int j = 0; j < TJ; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  const uint32_t lr = lane & 15u, lg = lane >> 4;
  auto compute = [&](const uint8_t *buf) {
    const uint8_t *xs = buf;
    const uint8_t *ws = buf + BM * BK * 2;
#pragma unroll
    for (int kh = 0; kh < 2; ++kh) {
      const uint32_t chunk = 4u * kh + lg;
      bf16x8 a[TI], b[TJ];
#pragma unroll
      for (int i = 0; i < TI; ++i)
        a[i] = *reinterpret_cast<const bf16x8 *>(xs + swz(wm * WTM + 16u * i + lr, chunk));
#pragma unroll
      for (int j = 0; j < TJ; ++j)
        b[j] = *reinterpret_cast<const bf16x8 *>(ws + swz(wn * WTN + 16u * j + lr, chunk));
#pragma unroll
      for (int i = 0; i < TI; ++i)
#pragma unroll
        for (int j = 0; j < TJ; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
    }
  };
  __syncthreads();  // step 0 is in LDS
  for (uint32_t k = 0;;) {
    compute(lds(k & 1u));
    if (k + 1u >= ksteps) break;
    __syncthreads();  // step k + 1 is in LDS, and everyone is done with step k's buffer
    ++k;
  }
#pragma unroll
  for (int i = 0; i < TI; ++i) {
#pragma unroll
    for (int j = 0; j < TJ; ++j) {
      const uint32_t n = n0 + wn * WTN + 16u * j + lr;
      if (n >= N) continue;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const uint32_t row = m0 + wm * WTM + 16u * i + 4u * lg + r;
        if (row < m) Y[(size_t)row * N + n] = to_bf16_bits(acc[i][j][r]);
      }
    }
  }
}

// The main prefill kernel: wave-specialised like k_gemm_prefill_ws, with the
// operands staged by DMA (buffer_load_dwordx4 ... lds: memory straight into
// LDS, no registers, no LDS stores).
//  * LDS holds three K steps.  Between barriers k - 1 and k the producers
//    request step k + 2's X tile into stage (k + 2) % 3 (it held step k - 1,
//    whose readers passed barrier k - 1), dequantize step k + 1's weight tile
//    into stage (k + 1) % 3 from codes loaded three steps ahead into
//    registers, and wait for step k + 1's X DMA, issued one iteration
//    earlier; barrier k then publishes step k + 1 while the MFMA waves
//    consume step k.
//  * Scales and biases arrive by DMA in blocks of 8 groups per row (16
//    bytes; gs / 8 steps), double-buffered in LDS: per step a producer reads
//    one scale and one bias per row it dequantizes from LDS instead of
//    issuing two 2-byte global loads.  Needs K % (8 gs) == 0.
//  * Measured on MI355X (m = 2048, 14336 x 4096): per-instruction costs of
//    the producers' global loads set the pace, not the MFMAs; staging X and
//    the scales/biases by DMA took 292 us to about 268 us.
template <int BM, int BN, int WGM, int WGN, int NP>
__global__ __launch_bounds__(64 * (WGM * WGN + NP)) void k_gemm_prefill_dma(
    const uint8_t *__restrict__ codes, const uint16_t *__restrict__ scales,
    const uint16_t *__restrict__ biases, const uint16_t *__restrict__ X, uint16_t *__restrict__ Y,
    uint32_t N, uint32_t K, uint32_t m, uint32_t gs_log2, uint32_t mtiles, uint32_t nbig, uint32_t mt_half,
    uint32_t nt_big, uint32_t nwork) {
  constexpr int kMma = WGM * WGN;          // MFMA waves
  constexpr int kPT = 64 * NP;             // producer threads
  constexpr int XR = kPT / 8;              // X rows per producer pass
  constexpr int WR = kPT / 4;              // weight rows per producer pass
  constexpr int XP = BM / XR;
  constexpr int WP = BN / WR;
  constexpr int WTM = BM / WGM, WTN = BN / WGN;
  constexpr int TI = WTM / 16, TJ = WTN / 16;
  static_assert(XP >= 1 && WP >= 1 && BM % XR == 0 && BN % WR == 0, "whole load passes");
  constexpr uint32_t kSbW = BN / 64;  // waves per array in the scale/bias DMA (64 rows each)
  static_assert(BN % 64 == 0 && 2 * (BN / 64) <= NP, "scale/bias staging: 64 rows of scales or biases per wave");
  constexpr uint32_t kStage = (BM + BN) * BK * 2;
  constexpr uint32_t kSbBytes = BN * 16u * 2u;  // one block: 8 groups of scales and of biases per row
  extern __shared__ __attribute__((aligned(16))) uint8_t lds_pf[];
  auto stage = [&](uint32_t i) { return lds_pf + i * kStage; };
  auto next3 = [](uint32_t i) { return i == 2u ? 0u : i + 1u; };

  // Work items: nbig tiles of BM x BN (N tiles 0 .. nt_big - 1), then tiles of
  // BM/2 x BN for the remaining N tiles.  The half tiles are dispatched last,
  // so that a grid of 3.5 rounds of full tiles ends in one round of half tiles
  // instead of half a round of full ones.  Within each kind, consecutive
  // items (the M tiles of one N tile) stay on one XCD.
  uint32_t bid = blockIdx.x;
  bool half;
  uint32_t m0, n0;
  if (bid < nbig) {
    if (nbig % kXcds == 0) bid = (bid % kXcds) * (nbig / kXcds) + bid / kXcds;
    half = false;
    m0 = (bid % mtiles) * BM;
    n0 = (bid / mtiles) * BN;
  } else {
    uint32_t h = bid - nbig;
    const uint32_t nh = nwork - nbig;
    if (nh % kXcds == 0) h = (h % kXcds) * (nh / kXcds) + h / kXcds;
    half = true;
    m0 = (h % mt_half) * (BM / 2);
    n0 = (nt_big + h / mt_half) * BN;
  }
  const uint32_t tile_rows = half ? (uint32_t)BM / 2u : (uint32_t)BM;
  const uint32_t tid = threadIdx.x;
  const uint32_t lane = tid & 63u, wave = uniform_pf(tid >> 6);
  const uint32_t ksteps = (K + BK - 1) / BK;

  if (wave >= (uint32_t)kMma) {
    // ---------------- producer waves
    const uint32_t ptid = tid - 64u * kMma;
    const uint32_t G = K >> gs_log2;
    const uint32_t mrows = m - m0 < tile_rows ? m - m0 : tile_rows;
    const uint32_t nrows = N - n0 < (uint32_t)BN ? N - n0 : (uint32_t)BN;
    const auto rx = make_rsrc(X + (size_t)m0 * K, mrows * K * 2u);
    const auto rw = make_rsrc(codes + (size_t)n0 * K, nrows * K);
    const auto rs = make_rsrc(scales + (size_t)n0 * G, nrows * G * 2u);
    const auto rb = make_rsrc(biases + (size_t)n0 * G, nrows * G * 2u);
    const uint32_t wr = ptid >> 2, wp = ptid & 3u;
    // The producer schedule, for XJN X loads per wave and step (the wait
    // counts below are compile-time immediates, hence a template).
    auto run = [&](auto xjn) {
      constexpr int XJN = decltype(xjn)::value;
      // X by DMA: one instruction fills 8 LDS rows (1 KiB, lane i -> byte 16 i);
      // lane i carries row r0 + i / 8 and, through the swizzle, logical chunk
      // (i % 8) ^ (i / 8).  Producer wave pw fills rows 8 (j NP + pw) .. + 7.
      constexpr int XJ = XJN;  // X loads per wave and step (half for a half tile)
      const uint32_t pw = wave - (uint32_t)kMma, plane = lane;
      const uint32_t xchunk = (plane & 7u) ^ (plane >> 3);
      uint32_t vxd[XJ];
#pragma unroll
      for (int j = 0; j < XJ; ++j) {
        const uint32_t row = (j * NP + pw) * 8u + (plane >> 3);
        vxd[j] = row < mrows ? row * K * 2u + xchunk * 16u : kOutOfRange;
      }
      auto xdma = [&](uint32_t ks, uint32_t st) {
        const bool live = ks < ksteps;
        const uint32_t k0 = live ? ks * BK : 0u;
        const bool xin = live && k0 + xchunk * 8u < K;
#pragma unroll
        for (int j = 0; j < XJ; ++j)
          __builtin_amdgcn_raw_ptr_buffer_load_lds(
              rx, (__attribute__((address_space(3))) void *)(stage(st) + (j * NP + pw) * 8u * (BK * 2)), 16,
              (int)(xin ? vxd[j] : kOutOfRange), (int)uniform_pf(2u * k0), 0, 0);
      };
      // Scales and biases by DMA, a block of 8 groups (8 gs codes, gs / 8
      // steps) at a time, double-buffered: wave pw copies 16 bytes per row for
      // rows 64 (pw % kSbW) .. + 63 of the scales (pw < kSbW) or biases.
      // Needs K % (8 gs) == 0, so that every row's block is 16 whole bytes.
      const uint32_t sbs_log2 = gs_log2 - 3u;  // steps per block, log2
      const uint32_t nblk = K >> (gs_log2 + 3u);
      auto sbuf = [&](uint32_t i) { return lds_pf + 3u * kStage + i * kSbBytes; };
      const uint32_t sbrow = (pw % kSbW) * 64u + plane;
      const uint32_t vsbd = sbrow < nrows ? sbrow * G * 2u : kOutOfRange;
      auto sbdma = [&](uint32_t blk) {
        if (pw < 2u * kSbW)
          __builtin_amdgcn_raw_ptr_buffer_load_lds(
              pw >= kSbW ? rb : rs,
              (__attribute__((address_space(3))) void *)(sbuf(blk & 1u) + (pw / kSbW) * (BN * 16u) +
                                                         (pw % kSbW) * 1024u),
              16, (int)vsbd, (int)uniform_pf(blk * 16u), 0, 0);
      };
      uint32_t vw[WP];
#pragma unroll
      for (int p = 0; p < WP; ++p) {
        const uint32_t row = p * WR + wr;
        vw[p] = row < nrows ? row * K + wp * 16u : kOutOfRange;
      }
      struct Regs {
        u32x4 w[WP];
      };
      auto issue = [&](Regs &r, uint32_t ks) {
        const bool live = ks < ksteps;
        const uint32_t k0 = live ? ks * BK : 0u;
        const bool win = live && k0 + wp * 16u < K;
#pragma unroll
        for (int p = 0; p < WP; ++p)
          r.w[p] = __builtin_amdgcn_raw_buffer_load_b128(rw, (int)(win ? vw[p] : kOutOfRange), (int)uniform_pf(k0),
                                                         kAuxNontemporal);
      };
      // Every pass's scale and bias of step ks, read from LDS in one round
      // trip before the step's DMA and stores are issued (the compiler keeps
      // LDS reads behind LDS writes that might alias them).
      struct SbVals {
        float sc[WP], bi[WP];
      };
      auto read_sb = [&](uint32_t ks) {
        SbVals v;
        const uint8_t *sb = sbuf((ks >> sbs_log2) & 1u);
        const uint32_t g = ((ks * BK + wp * 16u) >> gs_log2) & 7u;
#pragma unroll
        for (int p = 0; p < WP; ++p) {
          const uint32_t srow = p * WR + wr;
          v.sc[p] = bf16_bits_to_f32(*reinterpret_cast<const uint16_t *>(sb + srow * 16u + 2u * g));
          v.bi[p] = bf16_bits_to_f32(*reinterpret_cast<const uint16_t *>(sb + BN * 16u + srow * 16u + 2u * g));
        }
        return v;
      };
      auto store = [&](const Regs &r, uint8_t *buf, const SbVals &v) {
        uint8_t *ws = buf + BM * BK * 2;
#pragma unroll
        for (int p = 0; p < WP; ++p) {
          const float sc = v.sc[p], bi = v.bi[p];
          const uint32_t word[4] = {r.w[p].x, r.w[p].y, r.w[p].z, r.w[p].w};
          uint32_t o[8];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            o[2 * i] = pack_bf16x2(__builtin_fmaf(code_f32(word[i], 0), sc, bi), __builtin_fmaf(code_f32(word[i], 1), sc, bi));
            o[2 * i + 1] =
                pack_bf16x2(__builtin_fmaf(code_f32(word[i], 2), sc, bi), __builtin_fmaf(code_f32(word[i], 3), sc, bi));
          }
          const uint32_t row = p * WR + wr;
          *reinterpret_cast<u32x4 *>(ws + swz(row, 2u * wp)) = u32x4{o[0], o[1], o[2], o[3]};
          *reinterpret_cast<u32x4 *>(ws + swz(row, 2u * wp + 1u)) = u32x4{o[4], o[5], o[6], o[7]};
        }
      };
      // vmcnt(n) with expcnt and lgkmcnt left open
#define INT8W_VMCNT(n) __builtin_amdgcn_s_waitcnt((((n) >> 4) << 14) | 0x0F70 | ((n) & 15))
      // vmcnt(n) and lgkmcnt(0)
#define INT8W_VMCNT_LGKM0(n) __builtin_amdgcn_s_waitcnt((((n) >> 4) << 14) | 0x0070 | ((n) & 15))
      Regs R0, R1, R2;
      // Iteration k (between barriers k - 1 and k): the X DMA of step k + 2
      // goes to stage (k + 2) % 3 (it held step k - 1, read before barrier
      // k - 1); step k + 1's weights are dequantized into stage (k + 1) % 3;
      // step k + 4's codes are requested; and the X DMA of step k + 1, issued
      // one iteration earlier, is awaited.  Barrier k thus publishes step k + 1
      // and every X DMA has two iterations to land.
      sbdma(0u);
      if (1u < nblk) sbdma(1u);
      issue(R0, 0);
      issue(R1, 1);
      issue(R2, 2);
      xdma(0u, 0u);
      xdma(1u, 1u);
      INT8W_VMCNT(3 * WP + 2 * XJ);  // scale/bias blocks 0 and 1 have landed
      __syncthreads();  // ... for every producer wave
      store(R0, stage(0u), read_sb(0u));
      issue(R0, 3);
      INT8W_VMCNT(XJ + WP);  // the X DMA of step 0 has landed
      __syncthreads();  // step 0 is in LDS
      auto step = [&](Regs &r, uint32_t k, uint32_t sx, uint32_t sw) {
        const uint32_t s = k + 1u;
        const SbVals v = read_sb(s);
        xdma(k + 2u, sx);
        store(r, stage(sw), v);
        issue(r, k + 4u);
        // at the first step of scale/bias block b, block b + 1 goes into the
        // buffer that held block b - 1
        if (s != 0u && (s & ((1u << sbs_log2) - 1u)) == 0u && (s >> sbs_log2) + 1u < nblk) sbdma((s >> sbs_log2) + 1u);
        // The X DMA of step k + 1 has landed and this wave's LDS stores are
        // done; then a bare barrier.  A fenced barrier would also wait for
        // every load still in flight -- step k + 2's X and the codes of step
        // k + 4 -- and so expose their latency on every step.  (A scale/bias
        // block requested here is older than step k + 3's X, so the wait two
        // iterations on covers it, before its first reader, gs / 8 >= 4
        // steps on.)
        INT8W_VMCNT_LGKM0(XJ + 2 * WP);
        asm volatile("s_barrier" ::: "memory");
      };
#undef INT8W_VMCNT
#undef INT8W_VMCNT_LGKM0
      // Steps 0 .. ksteps - 2, three to an iteration and the rest after the
      // loop.  The loop has a single exit: with an exit after every step the
      // compiler's wait counts at the loop head also cover the paths that
      // leave, and it waited for every load in flight once per iteration.
      const uint32_t nst = ksteps - 1u;
      uint32_t k = 0;
      for (; k + 3u <= nst; k += 3u) {
        step(R1, k, 2u, 1u);
        step(R2, k + 1u, 0u, 2u);
        step(R0, k + 2u, 1u, 0u);
      }
      if (k < nst) {
        step(R1, k, 2u, 1u);
        if (k + 1u < nst) step(R2, k + 1u, 0u, 2u);
      }

    };
    if (half)
      run(std::integral_constant<int, BM / (16 * NP)>{});
    else
      run(std::integral_constant<int, BM / (8 * NP)>{});
    return;
  }

  // ---------------- MFMA waves
  const uint32_t wm = wave / WGN, wn = wave % WGN;
  f32x4 acc[TI][TJ];
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int j = 0; j < TJ; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  const uint32_t lr = lane & 15u, lg = lane >> 4;
  // operand fragments of one half step (32 of the 64 K positions)
  auto load_frags = [&](bf16x8 *a, bf16x8 *b, const uint8_t *buf, uint32_t kh) {
    const uint8_t *xs = buf;
    const uint8_t *ws = buf + BM * BK * 2;
    const uint32_t chunk = 4u * kh + lg;
#pragma unroll
    for (int i = 0; i < TI; ++i) a[i] = *reinterpret_cast<const bf16x8 *>(xs + swz(wm * WTM + 16u * i + lr, chunk));
#pragma unroll
    for (int j = 0; j < TJ; ++j) b[j] = *reinterpret_cast<const bf16x8 *>(ws + swz(wn * WTN + 16u * j + lr, chunk));
  };
  auto mma = [&](const bf16x8 *a, const bf16x8 *b) {
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
      for (int j = 0; j < TJ; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
  };
  // one half step's operands at a time: the other MFMA wave on the SIMD
  // covers the LDS latency (measured equal to or faster than reading both
  // halves ahead, with fewer registers)
  bf16x8 a[TI], b[TJ];
  __syncthreads();  // the producers' scale/bias staging
  __syncthreads();  // step 0 is in LDS
  // on a half tile the waves of the lower rows have nothing to multiply (but
  // keep the barrier count)
  if (wm * (uint32_t)WTM >= tile_rows) {
    for (uint32_t k = 1; k < ksteps; ++k) __syncthreads();
    return;
  }
  uint32_t s = 0;
  for (uint32_t k = 0;;) {
    load_frags(a, b, stage(s), 0u);
    mma(a, b);
    load_frags(a, b, stage(s), 1u);
    mma(a, b);
    if (k + 1u >= ksteps) break;
    __syncthreads();  // step k + 1 is in LDS; everyone is done with step k
    s = next3(s);
    ++k;
  }
#pragma unroll
  for (int i = 0; i < TI; ++i) {
#pragma unroll
    for (int j = 0; j < TJ; ++j) {
      const uint32_t n = n0 + wn * WTN + 16u * j + lr;
      if (n >= N) continue;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const uint32_t row = m0 + wm * WTM + 16u * i + 4u * lg + r;
        if (row < m) Y[(size_t)row * N + n] = to_bf16_bits(acc[i][j][r]);
      }
    }
  }
}

template <int BM, int BN, int WGM, int WGN, int NP>
hipError_t launch_tile_dma(const WeightView &w, const uint16_t *X, uint16_t *Y, uint32_t m, hipStream_t stream) {
  auto kern = k_gemm_prefill_dma<BM, BN, WGM, WGN, NP>;
  static bool configured = false;
  if (!configured) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
    if (e != hipSuccess) return e;
    configured = true;
  }
  const uint32_t mtiles = (m + BM - 1) / BM;
  const uint32_t ntiles = (w.N + BN - 1) / BN;
  // When the full tiles leave a last round at most half full, the N tiles of
  // that round are done as half-height tiles (twice as many, about half the
  // time each) in one last round.
  const uint32_t cus = (uint32_t)device_cu_count();
  const uint32_t full = mtiles * ntiles, rem = full % cus;
  uint32_t nt_half = 0;
  if (full > cus && rem != 0 && 2u * rem <= cus) {
    nt_half = (rem + mtiles - 1) / mtiles;
    if (nt_half >= ntiles) nt_half = 0;
  }
  const uint32_t nt_big = ntiles - nt_half;
  const uint32_t mt_half = (m + BM / 2 - 1) / (BM / 2);
  const uint32_t nbig = mtiles * nt_big;
  const uint32_t nwork = nbig + mt_half * nt_half;
  const size_t lds = 3u * (BM + BN) * BK * 2u + BN * 16u * 2u * 2u;
  hipLaunchKernelGGL(kern, dim3(nwork), dim3(64 * (WGM * WGN + NP)), lds, stream,
                     reinterpret_cast<const uint8_t *>(w.packed), w.scales, w.biases, X, Y, w.N, w.K, m,
                     (uint32_t)__builtin_ctz(w.gs), mtiles, nbig, mt_half, nt_big, nwork);
  return hipGetLastError();
}

template <int BM, int BN, int WGM, int WGN, int NP>
hipError_t launch_tile_ws(const WeightView &w, const uint16_t *X, uint16_t *Y, uint32_t m, hipStream_t stream) {
  auto kern = k_gemm_prefill_ws<BM, BN, WGM, WGN, NP>;
  static bool configured = false;
  if (!configured) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
    if (e != hipSuccess) return e;
    configured = true;
  }
  const uint32_t mtiles = (m + BM - 1) / BM;
  const uint32_t ntiles = (w.N + BN - 1) / BN;
  const uint32_t nwork = mtiles * ntiles;
  const size_t lds = 2u * (BM + BN) * BK * 2u;
  hipLaunchKernelGGL(kern, dim3(nwork), dim3(64 * (WGM * WGN + NP)), lds, stream,
                     reinterpret_cast<const uint8_t *>(w.packed), w.scales, w.biases, X, Y, w.N, w.K, m,
                     (uint32_t)__builtin_ctz(w.gs), mtiles, nwork);
  return hipGetLastError();
}

template <int BM, int BN, int WGM, int WGN>
hipError_t launch_tile(const WeightView &w, const uint16_t *X, uint16_t *Y, uint32_t m, hipStream_t stream) {
  auto kern = k_gemm_prefill<BM, BN, WGM, WGN>;
  static bool configured = false;
  if (!configured) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
    if (e != hipSuccess) return e;
    configured = true;
  }
  const uint32_t mtiles = (m + BM - 1) / BM;
  const uint32_t ntiles = (w.N + BN - 1) / BN;
  const uint32_t nwork = mtiles * ntiles;
  const size_t lds = 2u * (BM + BN) * BK * 2u;
  hipLaunchKernelGGL(kern, dim3(nwork), dim3(64 * WGM * WGN), lds, stream, reinterpret_cast<const uint8_t *>(w.packed),
                     w.scales, w.biases, X, Y, w.N, w.K, m, (uint32_t)__builtin_ctz(w.gs), mtiles, nwork);
  return hipGetLastError();
}

}  // namespace

// Tile shapes (BM x BN, waves): 0 = 128 x 128 (2 x 2), 1 = 128 x 64 (2 x 2),
// 2 = 256 x 128 (4 x 2 MFMA waves + 8 producer waves), 3 = 256 x 128 staged
// by DMA (4 x 2 MFMA waves + 4 producer waves; K % (8 gs) == 0), 4 = 128 x 64
// staged by DMA (2 x 2 MFMA waves + 4 producer waves; K % (8 gs) == 0).
hipError_t launch_gemm_prefill_tile(int t, const WeightView &w, const uint16_t *X, uint16_t *Y, uint32_t m,
                                    hipStream_t stream) {
  switch (t) {
    case 1: return launch_tile<128, 64, 2, 2>(w, X, Y, m, stream);
    case 2: return launch_tile_ws<256, 128, 4, 2, 8>(w, X, Y, m, stream);
    case 3:
      if (w.K % (8u * w.gs) != 0u) return hipErrorInvalidValue;
      return launch_tile_dma<256, 128, 4, 2, 4>(w, X, Y, m, stream);
    case 4:
      if (w.K % (8u * w.gs) != 0u) return hipErrorInvalidValue;
      return launch_tile_dma<128, 64, 2, 2, 4>(w, X, Y, m, stream);
    default: return launch_tile<128, 128, 2, 2>(w, X, Y, m, stream);
  }
}

namespace {

// Where K allows the DMA-staged kernel (K % (8 gs) == 0) it runs 256 x 128 or
// 128 x 64 tiles, whichever an estimate puts first: a 64-deep K step takes
// about 0.85 us per round of 256 x 128 tiles over the CUs (half a round for a
// last round at most half full, done as half-height tiles) and 0.45 us per
// round of 128 x 64 ones (whole rounds: their half-height tiles are slow).
// Measured (graph-timed) against the 128 x 128 single-role kernel the rule
// used before: 4096 x 14336, m = 768 / 1024: 178 / 179 us against 229 / 234;
// 4096 x 4096, m = 768 / 1024: 57 / 57 against 64 / 66; 14336 x 4096,
// m = 256: 59 against 70.  Other K: 256 x 128 tiles when they give at least
// ~3/4 of a tile per CU, else 128 x 128, else 128 x 64.
int prefill_shape(const WeightView &w, uint32_t m, uint32_t cus) {
  const uint32_t t256 = ((m + 255u) / 256u) * ((w.N + 127u) / 128u);
  if (w.K % (8u * w.gs) == 0u) {
    const uint32_t t12864 = ((m + 127u) / 128u) * ((w.N + 63u) / 64u);
    const uint32_t rem = t256 % cus;
    const double r256 = t256 <= cus ? 1.0 : (double)(t256 / cus) + (rem == 0u ? 0.0 : 2u * rem <= cus ? 0.5 : 1.0);
    const double r12864 = (double)((t12864 + cus - 1u) / cus);
    return r256 * 0.85 <= r12864 * 0.45 ? 3 : 4;
  }
  const uint32_t t128 = ((m + 127u) / 128u) * ((w.N + 127u) / 128u);
  return 4u * t256 >= 3u * cus ? 2 : 4u * t128 >= 3u * cus ? 0 : 1;
}

}  // namespace

hipError_t launch_gemm_prefill(const WeightView &w, const uint16_t *X, uint16_t *Y, uint32_t m,
                               hipStream_t stream) {
  return launch_gemm_prefill_tile(prefill_shape(w, m, (uint32_t)device_cu_count()), w, X, Y, m, stream);
}

// On the 128 x 64 grids (fewer than ~3/4 of a 128 x 128 tile per CU) the
// tiled kernel's time hardly depends on m: one workgroup per CU walks all of
// K, about 0.42 us per 64-deep step for each round of tiles over the CUs.  A
// small-m pass streams the weight once: about 3 TB/s plus ~3 us with two X
// tiles (32 rows), 4 TB/s plus ~3 us with one.  The passes are taken when
// they are estimated at least 10 % faster.  Measured (graph-timed), 32-row
// passes against the tiled kernel: 4096 x 14336 gs64, m = 32 / 64 / 96 / 128:
// 24 / 46 / 72 / 96 against 90 / 91 / 91 / 92 us; 4096 x 4096, m = 32 / 64:
// 10 / 19 against 28 / 29 us; 8192 x 28672 gs128, m = 64: 136 against 175
// us; 14336 x 4096 (224 such tiles), m = 32 / 48: 25 / 48 against 30 / 30 us.
uint32_t gemm_smallm_slice_rows(const WeightView &w, uint32_t m) {
  if (m <= 16u || m > 128u) return 0;
  const uint32_t cus = (uint32_t)device_cu_count();
  const int shape = prefill_shape(w, m, cus);
  if (shape != 4 && shape != 1) return 0;
  const double tiles = (double)((m + 127u) / 128u) * (double)((w.N + 63u) / 64u);
  const double rounds = (double)(uint32_t)((tiles + cus - 1.0) / cus);
  const double t_tiled = rounds * (double)((w.K + 63u) / 64u) * 0.42;
  const double bytes = (double)w.N * w.K + 4.0 * w.N * (w.K / w.gs);
  uint32_t rows;
  double t_pass;
  if (smallm32_supported(w.N, w.K, w.gs)) {
    rows = 32u;
    t_pass = bytes / 3.0e6 + 3.0;  // us at 3 TB/s
  } else if (smallm_supported(w.K, w.gs)) {
    rows = 16u;
    t_pass = bytes / 4.0e6 + 3.0;
  } else {
    return 0;
  }
  return (double)((m + rows - 1u) / rows) * t_pass < 0.9 * t_tiled ? rows : 0u;
}

}  // namespace int8w
