// gemm_smallm.hip -- Y = X W^T for 2 <= m <= 16 rows (one 16-row X tile), or
// up to 32 (two tiles, MT = 2), on gfx950 matrix cores (rustdoc page
// "MlxInt8Weight", method gemm: X BF16 [m, in_features], Y BF16
// [m, out_features]).
//
// Still HBM-bound (each code byte is read once and used m times), but m fp32
// FMAs per code would swamp the vector ALUs, so the products go to
// v_mfma_f32_16x16x32_bf16:
//  * The raw codes 0..255 are exact in BF16 (8 significant bits), so they
//    enter the MFMA unscaled; the affine terms are applied per window of 32
//    or 64 codes that lies inside one group:
//        sum_{k in win} (q s + b) x = s * sum q x + b * sum x
//    The first sum is the MFMA on raw codes; the second comes from an MFMA
//    against a constant all-ones operand, which leaves sum_k X[i,k] in exactly
//    the accumulator lanes that need it.  Products q*x are exact.
//  * MFMA D[i][j] = sum_k A[i][k] B[k][j] with A = X (i: input row, rows past
//    m are zero), B = codes (j: weight row).  Lane l holds
//    A[l%16][8*(l/16) .. +7], B[8*(l/16) .. +7][l%16] and D[4*(l/16)+r][l%16];
//    the k positions behind a lane's 8 values are the same for A and B.
//    gs >= 64: a 64-code step is two MFMAs over codes 16*(l/16) + 0..7 and
//    + 8..15 of each lane (one group); gs == 32: the two MFMAs take 8 codes of
//    each 32-code half, one group each.
//  * A workgroup of KS waves owns RT tiles of 16 weight rows and walks K in
//    blocks of KB = 64*KS*SPW codes.  Each block (the tiles' codes and the
//    16 MT X rows, rows past m zero) is copied by DMA (buffer_load_dwordx4 ... lds)
//    with every load reading whole 16-byte chunks of one row in contiguous
//    runs (the weight stream stays sequential in HBM) and landing in LDS with
//    the 16-byte chunks of row r XOR-swizzled by r mod 16 (so the 16 rows an
//    MFMA operand read touches sit in distinct banks), then read back in MFMA
//    operand layout.  Wave w takes the SPW steps [w*SPW, (w+1)*SPW) of every
//    block for all RT tiles; with MT = 2 each code fragment, converted once,
//    feeds the MFMAs of both X tiles.
//  * Pipeline: NS LDS block buffers; the DMA of NS - 1 blocks is in flight
//    while one is consumed; one workgroup barrier per block.  Every global
//    load goes through a bounded buffer resource: past the end it reads (or
//    writes to LDS) zeros.
//  * Scales and biases of the workgroup's rows are staged in LDS once, packed
//    as BF16 pairs.  The KS partial sums meet in LDS in wave order (no
//    atomics: deterministic).
#include "common.h"
#include "launch.h"

namespace int8w {

namespace {

__device__ __forceinline__ uint32_t uniform_sm(uint32_t v) { return __builtin_amdgcn_readfirstlane(v); }

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

template <int KS, int RT, int SPW, bool G32, int MT = 1, int XR = 16>
struct SmShape {
  static constexpr int kThreads = 64 * KS;
  static constexpr uint32_t KB = 64u * KS * SPW;         // codes per block
  static constexpr uint32_t CPR = KB / 16u;               // 16-byte code chunks per row per block
  static constexpr uint32_t XCPR = 2u * CPR;              // 16-byte X chunks per row per block
  static constexpr uint32_t CODE_BYTES = 16u * RT * KB;   // one block of codes in LDS
  static constexpr uint32_t X_BYTES = XR * MT * 2u * KB;  // XR MT X rows (rows past m are zero)
  static constexpr uint32_t BUF_BYTES = CODE_BYTES + X_BYTES;
  static constexpr int NC = (int)(CODE_BYTES / 1024u / KS);  // code loads per wave per block
  static constexpr int NX = (int)(X_BYTES / 1024u / KS);     // X loads per wave per block
  static_assert(CODE_BYTES % (1024u * KS) == 0 && X_BYTES % (1024u * KS) == 0, "whole loads per wave");
  static_assert(CPR >= 16, "swizzle needs 16 chunks per row");
};

// LDS (dynamic): NS block buffers [codes | X], then sb [16*RT][G+1] packed
// (scale | bias << 16).  The partial-sum exchange reuses the block buffers.
template <int KS, int RT, int SPW, int NS, bool G32, int MT, int XR>
__global__ __launch_bounds__(64 * KS) void k_gemm_smallm(
    const uint8_t *__restrict__ codes, const uint16_t *__restrict__ scales,
    const uint16_t *__restrict__ biases, const uint16_t *__restrict__ X, uint16_t *__restrict__ Y,
    uint32_t N, uint32_t K, uint32_t m, uint32_t gs_log2) {
  using S = SmShape<KS, RT, SPW, G32, MT, XR>;
  static_assert(XR == 16 || MT == 1, "fewer staged X rows only with one X tile");
  extern __shared__ __attribute__((aligned(16))) uint8_t lds_sm[];
  const uint32_t G = K >> gs_log2;
  const uint32_t SBP = G + 1u;  // odd pitch: the 16 rows of a read hit distinct banks
  uint32_t *sb = reinterpret_cast<uint32_t *>(lds_sm + NS * S::BUF_BYTES);

  const uint32_t tid = threadIdx.x;
  const uint32_t lane = tid & 63u;
  const uint32_t wave = uniform_sm(tid >> 6);
  const uint32_t lr = lane & 15u;  // X row of A / weight row of B within a tile
  const uint32_t lg = lane >> 4;   // 8-wide k block of this lane
  const uint32_t n0 = blockIdx.x * (16u * RT);
  const uint32_t rows = N - n0 < 16u * RT ? N - n0 : 16u * RT;  // rows of the workgroup
  const uint32_t nb = (K + S::KB - 1u) / S::KB;                   // blocks

  const auto rw = make_rsrc(codes + (size_t)n0 * K, rows * K);
  const auto rx = make_rsrc(X, m * K * 2u);

  // ---- per-lane global offsets of this wave's loads (the block's k is added
  // per block).  Load j of the wave fills LDS bytes [q*1024, (q+1)*1024) of
  // the block's code (or X) region, q = wave*NC + j; lane i writes the 16
  // bytes at q*1024 + 16*i, i.e. (row, physical chunk p) with the logical
  // chunk c = p ^ (row & 15) read from global memory.
  uint32_t vc[S::NC], vx[S::NX];
  uint32_t cchunk[S::NC], xchunk[S::NX];  // logical chunk (for the k bound)
#pragma unroll
  for (int j = 0; j < S::NC; ++j) {
    const uint32_t slot = (wave * S::NC + j) * 64u + lane;
    const uint32_t row = slot / S::CPR, p = slot % S::CPR;
    const uint32_t c = p ^ (row & 15u);
    cchunk[j] = c;
    vc[j] = row < rows ? row * K + 16u * c : kOutOfRange;
  }
#pragma unroll
  for (int j = 0; j < S::NX; ++j) {
    const uint32_t slot = (wave * S::NX + j) * 64u + lane;
    const uint32_t row = slot / S::XCPR, p = slot % S::XCPR;
    const uint32_t c = p ^ (row & 15u);
    xchunk[j] = c;
    vx[j] = row < m ? row * K * 2u + 16u * c : kOutOfRange;
  }

  // With 8 or more waves, X loads that start on a row past m are skipped
  // (those LDS rows are zeroed once; measured 5-8 % faster on the
  // 4096 x 14336 shape at m <= 9, and 2 % slower with 4 waves); xlive is the
  // same for all lanes of the wave.
  constexpr bool kSkipX = KS >= 8;
  bool xlive[S::NX];
  uint32_t nlive = 0;
#pragma unroll
  for (int j = 0; j < S::NX; ++j) {
    xlive[j] = !kSkipX || (wave * S::NX + j) * 64u / S::XCPR < m;
    nlive += xlive[j] ? 1u : 0u;
  }

  // Block blk goes straight from memory into LDS buffer `buf` by DMA
  // (buffer_load_dwordx4 ... lds: lane i of a wave's load j writes the 16
  // bytes at (wave NC + j) 1024 + 16 i, the layout above); past the end of a
  // row or of X a lane writes zeros.
  auto dma = [&](uint32_t blk, uint32_t buf) {
    const bool live = blk < nb;
    const uint32_t kb = live ? blk * S::KB : 0u;
    uint8_t *base = lds_sm + buf * S::BUF_BYTES;
#pragma unroll
    for (int j = 0; j < S::NC; ++j) {
      const bool in = live && kb + 16u * cchunk[j] < K;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rw, (__attribute__((address_space(3))) void *)(base + (wave * S::NC + j) * 1024u), 16,
          (int)(in ? vc[j] : kOutOfRange), (int)uniform_sm(kb), 0, kAuxNontemporal);
    }
#pragma unroll
    for (int j = 0; j < S::NX; ++j) {
      if (!xlive[j]) continue;  // rows past m: zeroed once below
      const bool in = live && 2u * kb + 16u * xchunk[j] < 2u * K;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rx, (__attribute__((address_space(3))) void *)(base + S::CODE_BYTES + (wave * S::NX + j) * 1024u), 16,
          (int)(in ? vx[j] : kOutOfRange), (int)uniform_sm(2u * kb), 0, 0);
    }
  };

  // ---- scales and biases of the workgroup's rows, all groups, packed as
  // (scale | bias << 16); the first NS - 1 blocks are requested first so that
  // they stream in meanwhile.
  const auto rs = make_rsrc(scales + (size_t)n0 * G, rows * G * 2u);
  const auto rb = make_rsrc(biases + (size_t)n0 * G, rows * G * 2u);
  const uint32_t total = 16u * RT * G;
  const uint32_t spare = 16u * RT * SBP;  // slot for entries past the end (branch-free writes)
#pragma unroll
  for (int d = 0; d < NS - 1; ++d) dma((uint32_t)d, (uint32_t)d);
  for (uint32_t e0 = 0; e0 < total; e0 += 4u * S::kThreads) {
    uint16_t sv[4], bv[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t e = e0 + tid + (uint32_t)j * S::kThreads;
      const uint32_t off = e < total ? e * 2u : kOutOfRange;
      sv[j] = buf_load_b16(rs, off);
      bv[j] = buf_load_b16(rb, off);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t e = e0 + tid + (uint32_t)j * S::kThreads;
      const uint32_t r = e / G, g = e - r * G;
      sb[e < total ? r * SBP + g : spare] = (uint32_t)sv[j] | ((uint32_t)bv[j] << 16);
    }
  }

  const bf16x8 ones = __builtin_bit_cast(bf16x8, make_uint4(0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u));
  const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
  f32x4 acc[MT][RT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int t = 0; t < RT; ++t) acc[mt][t] = zero;

  auto compute = [&](uint32_t blk, uint32_t buf) {
    const uint8_t *cb = lds_sm + buf * S::BUF_BYTES;
    const uint8_t *xbp = cb + S::CODE_BYTES;
#pragma unroll
    for (int st = 0; st < SPW; ++st) {
      const uint32_t kl = 64u * (wave * SPW + st);  // step's first code within the block
      const uint32_t kg = blk * S::KB + kl;          // ... within the row
      uint32_t g = kg >> gs_log2;
      if (g >= G) g = G - 1u;  // a step past K holds zeros: any finite pair
      // X fragments of the step's two MFMAs (row 16 mt + lr of each X tile;
      // its chunks are swizzled by lr like every other row's)
      bf16x8 xa8[MT], xb8[MT];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const uint8_t *xr = xbp + (XR * mt + lr) * (2u * S::KB);
        u32x4 xa = {0u, 0u, 0u, 0u}, xb = {0u, 0u, 0u, 0u};
        if (XR < 16 && lr >= XR) {
          // rows XR .. 15 of the A operand are zero and not staged
        } else if constexpr (G32) {
          const uint32_t ca = (kl + 8u * lg) >> 3, cbx = (kl + 32u + 8u * lg) >> 3;  // 16-byte X chunks
          xa = *reinterpret_cast<const u32x4 *>(xr + 16u * (ca ^ lr));
          xb = *reinterpret_cast<const u32x4 *>(xr + 16u * (cbx ^ lr));
        } else {
          const uint32_t ca = (kl + 16u * lg) >> 3;
          xa = *reinterpret_cast<const u32x4 *>(xr + 16u * (ca ^ lr));
          xb = *reinterpret_cast<const u32x4 *>(xr + 16u * ((ca + 1u) ^ lr));
        }
        xa8[mt] = __builtin_bit_cast(bf16x8, xa);
        xb8[mt] = __builtin_bit_cast(bf16x8, xb);
      }
      if constexpr (G32) {
        f32x4 SA[MT], SB[MT];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          SA[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa8[mt], ones, zero, 0, 0, 0);
          SB[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xb8[mt], ones, zero, 0, 0, 0);
        }
        const uint32_t gb = g + 1u < G ? g + 1u : g;
#pragma unroll
        for (int t = 0; t < RT; ++t) {
          const uint32_t row = 16u * t + lr;
          const uint8_t *rp = cb + row * S::KB;
          const uint32_t c0 = (kl + 8u * lg) >> 4, c1 = (kl + 32u + 8u * lg) >> 4, h = 8u * (lg & 1u);
          const u32x2 qa = *reinterpret_cast<const u32x2 *>(rp + 16u * (c0 ^ lr) + h);
          const u32x2 qb = *reinterpret_cast<const u32x2 *>(rp + 16u * (c1 ^ lr) + h);
          const uint32_t pa = sb[row * SBP + g], pb = sb[row * SBP + gb];
          const float sa = __uint_as_float(pa << 16), ba = __uint_as_float(pa & 0xFFFF0000u);
          const float sbv = __uint_as_float(pb << 16), bbv = __uint_as_float(pb & 0xFFFF0000u);
          const bf16x8 qa8 = codes8_to_bf16x8(qa.x, qa.y), qb8 = codes8_to_bf16x8(qb.x, qb.y);
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) {
            const f32x4 PA = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa8[mt], qa8, zero, 0, 0, 0);
            const f32x4 PB = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xb8[mt], qb8, zero, 0, 0, 0);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const float v = __builtin_fmaf(sa, PA[r], __builtin_fmaf(ba, SA[mt][r], acc[mt][t][r]));
              acc[mt][t][r] = __builtin_fmaf(sbv, PB[r], __builtin_fmaf(bbv, SB[mt][r], v));
            }
          }
        }
      } else {
        f32x4 Sx[MT];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          Sx[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa8[mt], ones, zero, 0, 0, 0);
          Sx[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xb8[mt], ones, Sx[mt], 0, 0, 0);
        }
#pragma unroll
        for (int t = 0; t < RT; ++t) {
          const uint32_t row = 16u * t + lr;
          const uint32_t c = (kl >> 4) + lg;
          const u32x4 q = *reinterpret_cast<const u32x4 *>(cb + row * S::KB + 16u * (c ^ lr));
          const uint32_t p = sb[row * SBP + g];
          const float s = __uint_as_float(p << 16), b = __uint_as_float(p & 0xFFFF0000u);
          const bf16x8 qa8 = codes8_to_bf16x8(q.x, q.y), qb8 = codes8_to_bf16x8(q.z, q.w);
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) {
            f32x4 P = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa8[mt], qa8, zero, 0, 0, 0);
            P = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xb8[mt], qb8, P, 0, 0, 0);
#pragma unroll
            for (int r = 0; r < 4; ++r)
              acc[mt][t][r] = __builtin_fmaf(s, P[r], __builtin_fmaf(b, Sx[mt][r], acc[mt][t][r]));
          }
        }
      }
    }
  };

  // ---- pipeline: NS LDS buffers.  At the top of step b, block b's DMA (the
  // oldest in flight) is awaited and a barrier makes every wave's part of it
  // visible -- and frees buffer (b - 1) % NS, which the DMA of block
  // b + NS - 1 then refills while block b is consumed.  The explicit wait
  // counts only this wave's DMA: the loop issues no other memory loads.
#define INT8W_VMCNT(n) __builtin_amdgcn_s_waitcnt((((n) >> 4) << 14) | 0x0F70 | ((n) & 15))
  static_assert((NS - 2) * (S::NC + S::NX) < 64, "vmcnt range");
  static_assert(S::NX <= 8, "wait table");
  // X rows m .. 15 of every buffer: zeros (the MFMA A operand's unused rows)
  for (uint32_t o = (kSkipX ? m : XR * MT) * 2u * S::KB + 16u * tid; o < S::X_BYTES; o += 16u * S::kThreads) {
#pragma unroll
    for (int u = 0; u < NS; ++u)
      *reinterpret_cast<u32x4 *>(lds_sm + u * S::BUF_BYTES + S::CODE_BYTES + o) = u32x4{0u, 0u, 0u, 0u};
  }
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): the scale/bias and zero stores are done before the first barrier
  // this wave's block b has landed: NS - 2 younger blocks of NC + nlive loads may still fly
  auto wait_block = [&]() {
    switch (nlive) {
      case 0: INT8W_VMCNT((NS - 2) * (S::NC + 0)); break;
      case 1: INT8W_VMCNT((NS - 2) * (S::NC + 1)); break;
      case 2: INT8W_VMCNT((NS - 2) * (S::NC + 2)); break;
      case 3: INT8W_VMCNT((NS - 2) * (S::NC + 3)); break;
      case 4: INT8W_VMCNT((NS - 2) * (S::NC + 4)); break;
      case 5: INT8W_VMCNT((NS - 2) * (S::NC + 5)); break;
      case 6: INT8W_VMCNT((NS - 2) * (S::NC + 6)); break;
      case 7: INT8W_VMCNT((NS - 2) * (S::NC + 7)); break;
      default: INT8W_VMCNT((NS - 2) * (S::NC + 8)); break;
    }
  };
  // Unrolled NS times so that every buffer index is a constant: the
  // compiler can then tell the DMA's LDS writes from this step's LDS reads
  // and does not wait for the DMA before reading.
  for (uint32_t b = 0;;) {
#pragma unroll
    for (int u = 0; u < NS; ++u) {
      // A bare barrier: a fenced one would also wait for the DMA still in
      // flight into the other buffers.  What it must order is explicit: this
      // wave's part of block b has landed, and its reads of block b - 1 have
      // returned (the compiler may place their last uses after this point).
      wait_block();
      __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
      asm volatile("s_barrier" ::: "memory");
      dma(b + NS - 1u, (uint32_t)((u + NS - 1) % NS));
      compute(b, (uint32_t)u);
      if (++b >= nb) goto pipeline_done;
    }
  }
pipeline_done:
#undef INT8W_VMCNT

  // ---- combine the KS partial sums in wave order and store
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the look-ahead DMA (zeros past the end) has landed
  __syncthreads();  // every wave is done with the block buffers
  f32x4 *red = reinterpret_cast<f32x4 *>(lds_sm);
  constexpr int kTiles = MT * RT;  // accumulator tiles per wave
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int t = 0; t < RT; ++t) red[(wave * kTiles + mt * RT + t) * 64u + lane] = acc[mt][t];
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
    for (int t = 0; t < RT; ++t) {
      f32x4 v = red[(mt * RT + t) * 64u + lane];
#pragma unroll
      for (int w = 1; w < KS; ++w) {
        const f32x4 o = red[(w * kTiles + mt * RT + t) * 64u + lane];
        v[0] += o[0]; v[1] += o[1]; v[2] += o[2]; v[3] += o[3];
      }
      const uint32_t n = n0 + 16u * t + lr;
      if (n < N) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const uint32_t i = 16u * mt + 4u * lg + r;
          if (i < m) Y[(size_t)i * N + n] = to_bf16_bits(v[r]);
        }
      }
    }
  }
}

template <int KS, int RT, int SPW, int NS, int MT = 1, int XR = 16>
size_t smallm_lds_bytes(uint32_t K, uint32_t gs) {
  using S = SmShape<KS, RT, SPW, false, MT, XR>;
  const size_t G = K / gs;
  size_t bytes = NS * S::BUF_BYTES + (16u * RT * (G + 1u) + 1u) * 4u;  // + the spare slot
  const size_t red = (size_t)KS * RT * MT * 64u * 16u;
  return bytes > red ? bytes : red;
}

template <int KS, int RT, int SPW, int NS, bool G32, int MT = 1, int XR = 16>
hipError_t launch_sm(const WeightView &w, const uint16_t *X, uint16_t *Y, uint32_t m, hipStream_t stream) {
  auto kern = k_gemm_smallm<KS, RT, SPW, NS, G32, MT, XR>;
  static bool configured = false;
  if (!configured) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
    if (e != hipSuccess) return e;
    configured = true;
  }
  const uint32_t blocks = (w.N + 16u * RT - 1u) / (16u * RT);
  const size_t lds = smallm_lds_bytes<KS, RT, SPW, NS, MT, XR>(w.K, w.gs);
  hipLaunchKernelGGL(kern, dim3(blocks), dim3(64 * KS), lds, stream,
                     reinterpret_cast<const uint8_t *>(w.packed), w.scales, w.biases, X, Y, w.N, w.K, m,
                     (uint32_t)__builtin_ctz(w.gs));
  return hipGetLastError();
}

}  // namespace

// Launch shapes (ks waves per workgroup, rt tiles of 16 rows, spw steps of 64
// codes per wave per block, ns LDS block buffers).  Shape 0: 4/2/1/3 (many
// rows: two tiles share each X block); shape 1: 16/1/1/3 (few rows, long K:
// more waves per tile); shape 2: 8/1/1/3; shape 3: 4/1/2/3.
constexpr int kSmShapes = 4;
#define INT8W_SM_SHAPE0 4, 2, 1, 3
#define INT8W_SM_SHAPE1 16, 1, 1, 3
#define INT8W_SM_SHAPE2 8, 1, 1, 3
#define INT8W_SM_SHAPE3 4, 1, 2, 3

size_t smallm_shape_lds(int shape, uint32_t K, uint32_t gs) {
  switch (shape) {
    case 0: return smallm_lds_bytes<INT8W_SM_SHAPE0>(K, gs);
    case 1: return smallm_lds_bytes<INT8W_SM_SHAPE1>(K, gs);
    case 2: return smallm_lds_bytes<INT8W_SM_SHAPE2>(K, gs);
    default: return smallm_lds_bytes<INT8W_SM_SHAPE3>(K, gs);
  }
}

int smallm_choose(uint32_t N, uint32_t K, uint32_t gs) {
  const uint32_t cus = (uint32_t)device_cu_count();
  const uint32_t tiles = (N + 15u) / 16u;
  int shape;
  if (tiles >= 2u * cus) shape = 0;       // >= 2 tile pairs per CU
  else if (tiles >= cus / 2u) shape = 1;  // a 16-wave workgroup per tile
  else shape = 1;
  // fall back to smaller LDS footprints when the staged scale/bias rows are long
  if (smallm_shape_lds(shape, K, gs) > 160u * 1024u) shape = 2;
  if (smallm_shape_lds(shape, K, gs) > 160u * 1024u) shape = 3;
  return shape;
}

bool smallm_supported(uint32_t K, uint32_t gs) {
  for (int s = 0; s < kSmShapes; ++s)
    if (smallm_shape_lds(s, K, gs) <= 160u * 1024u) return true;
  return false;
}

hipError_t launch_gemm_smallm_shape(int shape, const WeightView &w, const uint16_t *X, uint16_t *Y, uint32_t m,
                                    hipStream_t stream) {
  const bool g32 = w.gs == 32;
  switch (shape) {
    case 0: return g32 ? launch_sm<INT8W_SM_SHAPE0, true>(w, X, Y, m, stream) : launch_sm<INT8W_SM_SHAPE0, false>(w, X, Y, m, stream);
    case 1: return g32 ? launch_sm<INT8W_SM_SHAPE1, true>(w, X, Y, m, stream) : launch_sm<INT8W_SM_SHAPE1, false>(w, X, Y, m, stream);
    case 2: return g32 ? launch_sm<INT8W_SM_SHAPE2, true>(w, X, Y, m, stream) : launch_sm<INT8W_SM_SHAPE2, false>(w, X, Y, m, stream);
    default: return g32 ? launch_sm<INT8W_SM_SHAPE3, true>(w, X, Y, m, stream) : launch_sm<INT8W_SM_SHAPE3, false>(w, X, Y, m, stream);
  }
}

hipError_t launch_gemm_smallm(const WeightView &w, const uint16_t *X, uint16_t *Y, uint32_t m,
                              hipStream_t stream) {
  const int shape = smallm_choose(w.N, w.K, w.gs);
  // Few rows (m <= 8) on a weight that wants the 16-wave shape but whose
  // scale/bias rows do not leave it room for three blocks of 16 X rows (e.g.
  // 4096 x 14336 at gs 32): stage only 8 X rows (the A operand's rows 8..15
  // are zeros from registers) and keep the 16-wave shape instead of falling
  // back to 8 waves.  Measured (graph-timed, interleaved): 4096 x 14336 gs32
  // m = 3..8 18.1-19.6 -> 16.6-17.5 us, 1024 x 20480 gs32 21.8 -> 17.6 us.
  // Same results: the zeros are the same, the sums meet in the same order.
  if (m <= 8u && shape >= 2 && (w.N + 15u) / 16u < 2u * (uint32_t)device_cu_count() &&
      smallm_lds_bytes<INT8W_SM_SHAPE1, 1, 8>(w.K, w.gs) <= 160u * 1024u)
    return w.gs == 32 ? launch_sm<INT8W_SM_SHAPE1, true, 1, 8>(w, X, Y, m, stream)
                      : launch_sm<INT8W_SM_SHAPE1, false, 1, 8>(w, X, Y, m, stream);
  return launch_gemm_smallm_shape(shape, w, X, Y, m, stream);
}

// Two X tiles (up to 32 rows) per pass: each code fragment converted once
// feeds both tiles' MFMAs.  Shapes: 4/2/1/3 with many rows, 8/1/1/3 with few.
#define INT8W_SM32_SHAPE0 4, 2, 1, 3
#define INT8W_SM32_SHAPE1 8, 1, 1, 3
int smallm32_choose(uint32_t N, uint32_t K, uint32_t gs) {
  const uint32_t cus = (uint32_t)device_cu_count();
  const int shape = (N + 15u) / 16u >= 2u * cus ? 0 : 1;
  const size_t lds = shape == 0 ? smallm_lds_bytes<INT8W_SM32_SHAPE0, 2>(K, gs)
                                : smallm_lds_bytes<INT8W_SM32_SHAPE1, 2>(K, gs);
  if (lds <= 160u * 1024u) return shape;
  return smallm_lds_bytes<INT8W_SM32_SHAPE1, 2>(K, gs) <= 160u * 1024u ? 1 : -1;
}

bool smallm32_supported(uint32_t N, uint32_t K, uint32_t gs) { return smallm32_choose(N, K, gs) >= 0; }

hipError_t launch_gemm_smallm32(const WeightView &w, const uint16_t *X, uint16_t *Y, uint32_t m,
                                hipStream_t stream) {
  const int shape = smallm32_choose(w.N, w.K, w.gs);
  if (shape < 0 || m > 32u) return hipErrorInvalidValue;
  const bool g32 = w.gs == 32;
  if (shape == 0)
    return g32 ? launch_sm<INT8W_SM32_SHAPE0, true, 2>(w, X, Y, m, stream)
               : launch_sm<INT8W_SM32_SHAPE0, false, 2>(w, X, Y, m, stream);
  return g32 ? launch_sm<INT8W_SM32_SHAPE1, true, 2>(w, X, Y, m, stream)
             : launch_sm<INT8W_SM32_SHAPE1, false, 2>(w, X, Y, m, stream);
}

}  // namespace int8w
