// fp8_gemv.hip -- y = W x for an FP8 E4M3 weight on gfx950 (rustdoc page
// "Fp8Weight": struct description, fields weight, row_scale, n, k and
// scale_format):
//   w[n,k] = E4M3(q[n,k]) * scale, the scale per row (f32 [N]), per block of
//   BS x BS (BF16 or f32 [ceil(N/BS), ceil(K/BS)]) or one global value.
//
// HBM-bound: one byte per weight, the scales are a few KB.  The design is
// the int8 gemv's:
//  * Activation.  x is widened to fp32 once per workgroup and K-tile into LDS.
//  * Codes.  A lane owns runs of 16 consecutive codes (one 16-byte load); a
//    wave-wide load streams 1 KiB of a row.  Each wave streams a balanced,
//    contiguous range of rows (RP side by side), through bounded buffer
//    resources, two blocks of loads in flight; past its last row a wave
//    re-reads its last item.  The first block goes out after the activation
//    and scale loads (vmcnt counts in order: waiting for those never waits
//    for it).
//  * Arithmetic.  The hardware converts two E4M3 codes to two fp32 values
//    per instruction (v_cvt_pk_f32_fp8, OCP E4M3 on gfx950: exact), then one
//    FMA per code.  A run never straddles a scale block (BS >= 64), so the
//    scale factors out of the run: a block scale multiplies each run's
//    partial; a row or global scale multiplies the row's total once.
//  * Reduction.  Fixed DPP order, K-tiles meet in LDS in tile order; no
//    atomics.
//  * Short rows (k = 1024..4096, a multiple of 1024): a lane's activations
//    (16 per 1 KiB segment) stay in its registers and a block scale is loaded
//    with the codes, so a wave needs no LDS, no barrier and no staging before
//    its first block (one block = one row, two rows in flight).
#include <type_traits>

#include "common.h"
#include "launch.h"

namespace int8w {

namespace {

constexpr uint32_t kFp8TileRunsMax = 1024;  // 16384 activations per LDS tile
constexpr int kFp8LoadsPerBlock = 4;        // 1 KiB wave loads per pipeline block
constexpr uint32_t kFp8MaxRowsPerWave = 16;
constexpr size_t kFp8LdsPerCu = 156 * 1024;

enum Fp8Scale { kSfRow = 0, kSfBlockBf16 = 1, kSfBlockF32 = 2 };

typedef float f32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t uni(uint32_t v) { return __builtin_amdgcn_readfirstlane(v); }

// sum_i E4M3(q_i) a_i over one lane's 16 codes
__device__ __forceinline__ float fp8_run_dot(const u32x4 &w, const float4 &a0, const float4 &a1, const float4 &a2,
                                             const float4 &a3) {
  const uint32_t words[4] = {w.x, w.y, w.z, w.w};
  const float av[16] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w,
                        a2.x, a2.y, a2.z, a2.w, a3.x, a3.y, a3.z, a3.w};
  float p = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)words[i], false);  // bytes 0, 1
    const f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)words[i], true);   // bytes 2, 3
    p = __builtin_fmaf(lo.x, av[4 * i + 0], p);
    p = __builtin_fmaf(lo.y, av[4 * i + 1], p);
    p = __builtin_fmaf(hi.x, av[4 * i + 2], p);
    p = __builtin_fmaf(hi.y, av[4 * i + 3], p);
  }
  return p;
}

// Sum over the 64 lanes in a fixed order; the total lands in lane 63.
__device__ __forceinline__ float sum_lane63(float v) {
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x111, 0xf, 0xf, true));
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x112, 0xf, 0xf, true));
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x114, 0xf, 0xf, true));
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x118, 0xf, 0xf, true));
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x142, 0xa, 0xf, false));
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x143, 0xc, 0xf, false));
  return v;
}

template <int U, int RP, int SF = 0>
struct Fp8Block {
  u32x4 q[U][RP];
  // block scales: the entry of each item's lane (its row block, its run's k-block)
  std::conditional_t<SF == 1, uint16_t, uint32_t> s[SF != 0 ? U : 1][SF != 0 ? RP : 1];
};

struct Fp8Cfg {
  int waves;          // per workgroup (8 or 16)
  int rp;             // rows side by side (1 or 2)
  uint32_t blocks;
  uint32_t ct;        // 16-code runs per LDS tile (multiple of 64)
  uint32_t max_rows;  // most rows any wave owns
  bool tail;          // k not a multiple of 1024
};

// The LDS bytes of one workgroup:
//   act  [NSEG][4][64] float4   activations of lane l's 16 codes in segment s
//   part [W][max_rows] float    row partials across K-tiles
// (block scales are loaded with the codes: each item's lane needs one entry)
size_t fp8_lds_bytes(const Fp8Cfg &c) { return (size_t)c.ct * 64u + (size_t)c.waves * c.max_rows * 4u; }

template <int SF, int W, int RP, int U, bool TAIL>
__global__ __launch_bounds__(64 * W) void k_fp8_gemv(const uint8_t *__restrict__ codes, const void *__restrict__ scale,
                                                     float single, const uint16_t *__restrict__ xg, uint16_t *y,
                                                     uint32_t N, uint32_t K, uint32_t bs_log2, uint32_t tile_runs,
                                                     uint32_t max_rows) {
  constexpr int kThreads = 64 * W;
  constexpr int kStage = (int)(kFp8TileRunsMax + kThreads - 1) / kThreads;
  constexpr bool kBlock = SF != kSfRow;
  extern __shared__ float4 lds4[];
  const uint32_t CT = tile_runs;
  const uint32_t NSEG = CT >> 6;
  float4 *act = lds4;
  float *part_all = reinterpret_cast<float *>(lds4 + NSEG * 256);

  const uint32_t tid = threadIdx.x;
  const uint32_t lane = tid & 63u;
  const uint32_t wave = uni(tid >> 6);
  const uint32_t lw = blockIdx.x * W + wave;
  const uint32_t TW = gridDim.x * W;
  const uint32_t rq = N / TW, rr = N % TW;
  const uint32_t rbeg = lw * rq + (lw < rr ? lw : rr);
  const uint32_t nr = rq + (lw < rr ? 1u : 0u);
  const uint32_t ngrp = (nr + RP - 1) / RP;
  const uint32_t cpr = K >> 4;
  const uint32_t KB = (K + (1u << bs_log2) - 1u) >> bs_log2;  // scale blocks along k
  const uint32_t NB = (N + (1u << bs_log2) - 1u) >> bs_log2;  // and along n
  constexpr uint32_t kEl = SF == kSfBlockBf16 ? 2u : 4u;  // block scale entry bytes

  const auto rw = make_rsrc(codes + (size_t)rbeg * K, nr * K);
  const auto rx = make_rsrc(xg, K * 2u);
  const auto rsc = make_rsrc(scale, kBlock ? NB * KB * kEl : 0u);
  float *part = part_all + wave * max_rows;

  const uint32_t vo_w = lane << 4;
  const uint32_t v_act = lane << 4;
  const uint32_t v_kb = kBlock ? (((lane << 4) >> bs_log2) * kEl) : 0u;  // this lane's k-block in a segment, bytes

  float acc[RP];
#pragma unroll
  for (int r = 0; r < RP; ++r) acc[r] = 0.f;
  Fp8Block<U, RP, SF> A, B;

  for (uint32_t t0 = 0; t0 < cpr; t0 += CT) {
    const uint32_t ct = (cpr - t0) < CT ? (cpr - t0) : CT;
    const bool last_tile = t0 + ct == cpr;
    const uint32_t nseg = (ct + 63u) >> 6;
    const uint32_t nitems = ngrp * nseg;
    const uint32_t nblk = (nitems + U - 1) / U;
    const uint32_t last_lanes = ct - ((nseg - 1u) << 6);
    const uint32_t vo_w_last = TAIL && lane >= last_lanes ? kOutOfRange : vo_w;
    // lanes past the end of the last segment load no scale (their codes are zero)
    const uint32_t v_kb_last = TAIL && lane >= last_lanes ? kOutOfRange : v_kb;
    const uint32_t grp_skip = RP * K - (nseg << 10);
    const uint32_t last_off = (nr ? nr - 1u : 0u) * K + (t0 << 4) + ((nseg - 1u) << 10);
    const uint32_t kb0 = (t0 << 4) >> bs_log2;
    const uint32_t seg_kb = kBlock ? (1024u >> bs_log2) : 0u;  // k-blocks per segment

    uint32_t i_off = t0 << 4, i_seg = 0, i_grp = 0;
    auto issue = [&](Fp8Block<U, RP, SF> &blk) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        uint32_t vw = vo_w, vk = v_kb;
        if constexpr (TAIL) {
          vw = (i_seg == nseg - 1u) ? vo_w_last : vo_w;
          vk = (i_seg == nseg - 1u) ? v_kb_last : v_kb;
        }
#pragma unroll
        for (int r = 0; r < RP; ++r) {
          const bool live = i_grp < ngrp && i_grp * RP + r < nr;
          const uint32_t sw = uni(live ? i_off + r * K : last_off);
          const uint32_t vwr = live ? vw : vo_w_last;
          blk.q[u][r] = __builtin_amdgcn_raw_buffer_load_b128(rw, (int)vwr, (int)sw, kAuxNontemporal);
          if constexpr (kBlock) {
            // the entry of (row block, k-block of the lane's run); past the
            // wave's rows, the last row's (any finite value: not used)
            const uint32_t row = rbeg + (live ? i_grp * RP + r : (nr ? nr - 1u : 0u));
            const uint32_t ss = uni(((row >> bs_log2) * KB + kb0 + i_seg * seg_kb) * kEl);
            if constexpr (SF == kSfBlockBf16)
              blk.s[u][r] = __builtin_amdgcn_raw_buffer_load_b16(rsc, (int)vk, (int)ss, 0);
            else
              blk.s[u][r] = __builtin_amdgcn_raw_buffer_load_b32(rsc, (int)vk, (int)ss, 0);
          }
        }
        i_off += 1024u;
        if (++i_seg == nseg) { i_seg = 0; ++i_grp; i_off += grp_skip; }
      }
    };
    uint32_t c_grp = 0, c_seg = 0;
    auto consume = [&](const Fp8Block<U, RP, SF> &blk) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (c_grp < ngrp) {
          const float4 *ap = reinterpret_cast<const float4 *>(reinterpret_cast<const char *>(act) +
                                                              uni(c_seg << 12) + v_act);
          const float4 a0 = ap[0], a1 = ap[64], a2 = ap[128], a3 = ap[192];
#pragma unroll
          for (int r = 0; r < RP; ++r) {
            const float p = fp8_run_dot(blk.q[u][r], a0, a1, a2, a3);
            if constexpr (kBlock) {
              const float s = SF == kSfBlockBf16 ? bf16_bits_to_f32((uint16_t)blk.s[u][r])
                                                 : __uint_as_float((uint32_t)blk.s[u][r]);
              acc[r] = __builtin_fmaf(s, p, acc[r]);
            } else {
              acc[r] += p;
            }
          }
          if (c_seg == nseg - 1u) {
#pragma unroll
            for (int r = 0; r < RP; ++r) {
              const uint32_t row = c_grp * RP + r;
              if (row < nr) {
                const float tot = sum_lane63(acc[r]);
                if (lane == 63u) {
                  float v = t0 ? part[row] + tot : tot;
                  if (last_tile) {
                    if constexpr (!kBlock) v *= scale ? reinterpret_cast<const float *>(scale)[rbeg + row] : single;
                    y[rbeg + row] = to_bf16_bits(v);
                  } else {
                    part[row] = v;
                  }
                }
              }
              acc[r] = 0.f;
            }
          }
        }
        if (++c_seg == nseg) { c_seg = 0; ++c_grp; }
      }
    };

    // 1. activation loads, then the first weight block
    u32x4 xv[kStage][2];
#pragma unroll
    for (int s = 0; s < kStage; ++s) {
      const uint32_t e = tid + s * kThreads;
      const uint32_t off = e < ct ? (t0 + e) * 32u : kOutOfRange;
      xv[s][0] = buf_load_b128(rx, off);
      xv[s][1] = buf_load_b128(rx, off + 16u);
    }
    // the first weight block goes out after the small loads and
    // unconditionally, so that waiting for them never waits for it
    issue(A);
    if (t0) __syncthreads();  // everyone is done with the previous tile
    // 2. the activation tile; runs past the end are zeros
#pragma unroll
    for (int s = 0; s < kStage; ++s) {
      const uint32_t e = tid + s * kThreads;
      if (e < (nseg << 6)) {
        const uint32_t wv[8] = {xv[s][0].x, xv[s][0].y, xv[s][0].z, xv[s][0].w,
                                xv[s][1].x, xv[s][1].y, xv[s][1].z, xv[s][1].w};
        float4 *dst = act + (e >> 6) * 256u + (e & 63u);
#pragma unroll
        for (int f = 0; f < 4; ++f)
          dst[f * 64] = make_float4(bf16_lo(wv[2 * f]), bf16_hi(wv[2 * f]), bf16_lo(wv[2 * f + 1]),
                                    bf16_hi(wv[2 * f + 1]));
      }
    }
    __syncthreads();
    // 3. two-stage pipeline in a loop with a single exit, two blocks per
    //    iteration and the rest after it (an exit after every block made the
    //    compiler wait at the loop head for the block just issued); after
    //    each consume only the other block's U RP loads may be in flight,
    //    said explicitly because a consume past the wave's rows waits for
    //    nothing
    constexpr int kBlk = (kBlock ? 2 : 1) * U * RP;  // codes (and block scales) of U RP items
    uint32_t b = 0;
    for (; b + 2u < nblk; b += 2u) {
      issue(B);
      consume(A);
      __builtin_amdgcn_s_waitcnt(((kBlk >> 4) << 14) | 0x0F70 | (kBlk & 15));
      issue(A);
      consume(B);
      __builtin_amdgcn_s_waitcnt(((kBlk >> 4) << 14) | 0x0F70 | (kBlk & 15));
    }
    if (b + 1u < nblk) {
      issue(B);
      consume(A);
      consume(B);
    } else if (b < nblk) {
      consume(A);
    }
  }
}

// The register-resident form for k = NS * 1024.  Same row partition,
// decode, scale placement and reduction as k_fp8_gemv.
template <int SF, int NS>
__global__ __launch_bounds__(512) void k_fp8_gemv_rx(const uint8_t *__restrict__ codes,
                                                     const void *__restrict__ scale, float single,
                                                     const uint16_t *__restrict__ xg, uint16_t *y, uint32_t N,
                                                     uint32_t bs_log2) {
  constexpr uint32_t K = NS * 1024u;
  constexpr bool kBlock = SF != kSfRow;
  constexpr uint32_t kEl = SF == kSfBlockBf16 ? 2u : 4u;  // block scale entry bytes
  const uint32_t lane = threadIdx.x & 63u;
  const uint32_t lw = blockIdx.x * 8u + uni(threadIdx.x >> 6);
  const uint32_t TW = gridDim.x * 8u;
  const uint32_t rq = N / TW, rr = N % TW;
  const uint32_t rbeg = lw * rq + (lw < rr ? lw : rr);
  const uint32_t nr = rq + (lw < rr ? 1u : 0u);
  const uint32_t KB = (K + (1u << bs_log2) - 1u) >> bs_log2;
  const uint32_t NB = (N + (1u << bs_log2) - 1u) >> bs_log2;
  const auto rw = make_rsrc(codes + (size_t)rbeg * K, nr * K);
  const auto rx = make_rsrc(xg, K * 2u);
  const auto rs = make_rsrc(scale, kBlock ? NB * KB * kEl : 0u);
  const uint32_t vo_w = lane << 4;
  const uint32_t v_kb = kBlock ? ((lane << 4) >> bs_log2) * kEl : 0u;  // the lane's k-block in a segment, bytes

  struct RowBlock {
    u32x4 q[NS];
    // block scale bits of each segment's run; BF16 ones stay 16-bit values
    // until they are used (no arithmetic on a block just requested)
    std::conditional_t<SF == kSfBlockBf16, uint16_t, uint32_t> s[kBlock ? NS : 1];
  };
  u32x4 xw[NS][2];
#pragma unroll
  for (int u = 0; u < NS; ++u) {
    xw[u][0] = buf_load_b128(rx, (u << 11) + (lane << 5));
    xw[u][1] = buf_load_b128(rx, (u << 11) + (lane << 5) + 16u);
  }
  uint32_t i_row = 0;
  auto issue = [&](RowBlock &blk) {
    // past the wave's rows a block re-reads its last row
    const uint32_t row = i_row < nr ? i_row : (nr ? nr - 1u : 0u);
#pragma unroll
    for (int u = 0; u < NS; ++u) {
      blk.q[u] = __builtin_amdgcn_raw_buffer_load_b128(rw, (int)vo_w, (int)uni(row * K + (u << 10)), kAuxNontemporal);
      if constexpr (kBlock) {
        const uint32_t so = uni((((rbeg + row) >> bs_log2) * KB + (((uint32_t)u << 10) >> bs_log2)) * kEl);
        if constexpr (SF == kSfBlockBf16)
          blk.s[u] = __builtin_amdgcn_raw_buffer_load_b16(rs, (int)v_kb, (int)so, 0);
        else
          blk.s[u] = __builtin_amdgcn_raw_buffer_load_b32(rs, (int)v_kb, (int)so, 0);
      }
    }
    ++i_row;
  };
  RowBlock A, B;
  issue(A);
  float a[NS][16];
#pragma unroll
  for (int u = 0; u < NS; ++u) {
    const uint32_t wv[8] = {xw[u][0].x, xw[u][0].y, xw[u][0].z, xw[u][0].w,
                            xw[u][1].x, xw[u][1].y, xw[u][1].z, xw[u][1].w};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      a[u][2 * i] = bf16_lo(wv[i]);
      a[u][2 * i + 1] = bf16_hi(wv[i]);
    }
  }
  uint32_t c_row = 0;
  auto consume = [&](const RowBlock &blk) {
    float acc = 0.f;
#pragma unroll
    for (int u = 0; u < NS; ++u) {
      const float p = fp8_run_dot(blk.q[u], make_float4(a[u][0], a[u][1], a[u][2], a[u][3]),
                                  make_float4(a[u][4], a[u][5], a[u][6], a[u][7]),
                                  make_float4(a[u][8], a[u][9], a[u][10], a[u][11]),
                                  make_float4(a[u][12], a[u][13], a[u][14], a[u][15]));
      if constexpr (kBlock) {
        float sc;
        if constexpr (SF == kSfBlockBf16)
          sc = bf16_bits_to_f32(blk.s[u]);
        else
          sc = __uint_as_float(blk.s[u]);
        acc = __builtin_fmaf(sc, p, acc);
      } else {
        acc += p;
      }
    }
    const float tot = sum_lane63(acc);
    if (lane == 63u) {
      float v = tot;
      if constexpr (!kBlock) v *= scale ? reinterpret_cast<const float *>(scale)[rbeg + c_row] : single;
      y[rbeg + c_row] = to_bf16_bits(v);
    }
    ++c_row;
  };
  // two-stage pipeline in a loop with a single exit (as in k_fp8_gemv)
  uint32_t b = 0;
  for (; b + 2u < nr; b += 2u) {
    issue(B);
    consume(A);
    issue(A);
    consume(B);
  }
  if (b + 1u < nr) {
    issue(B);
    consume(A);
    consume(B);
  } else if (b < nr) {
    consume(A);
  }
}

template <int SF>
hipError_t launch_fp8_rx(const Fp8Cfg &c, const uint8_t *codes, const void *scale, float single, uint32_t bs_log2,
                         const uint16_t *x, uint16_t *y, uint32_t N, uint32_t K, hipStream_t stream) {
  switch (K / 1024u) {
    case 1:
      hipLaunchKernelGGL((k_fp8_gemv_rx<SF, 1>), dim3(c.blocks), dim3(512), 0, stream, codes, scale, single, x, y, N,
                         bs_log2);
      break;
    case 2:
      hipLaunchKernelGGL((k_fp8_gemv_rx<SF, 2>), dim3(c.blocks), dim3(512), 0, stream, codes, scale, single, x, y, N,
                         bs_log2);
      break;
    case 3:
      hipLaunchKernelGGL((k_fp8_gemv_rx<SF, 3>), dim3(c.blocks), dim3(512), 0, stream, codes, scale, single, x, y, N,
                         bs_log2);
      break;
    default:
      hipLaunchKernelGGL((k_fp8_gemv_rx<SF, 4>), dim3(c.blocks), dim3(512), 0, stream, codes, scale, single, x, y, N,
                         bs_log2);
  }
  return hipGetLastError();
}

template <typename Kern>
hipError_t lds_cap(Kern kern, bool &configured) {
  if (configured) return hipSuccess;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
  if (e == hipSuccess) configured = true;
  return e;
}

template <int SF, int W, int RP, bool TAIL>
hipError_t launch_fp8_cfg(const Fp8Cfg &c, const uint8_t *codes, const void *scale, float single, uint32_t bs_log2,
                          const uint16_t *x, uint16_t *y, uint32_t N, uint32_t K, hipStream_t stream) {
  static bool configured = false;
  auto kern = k_fp8_gemv<SF, W, RP, kFp8LoadsPerBlock / RP, TAIL>;
  hipError_t e = lds_cap(kern, configured);
  if (e != hipSuccess) return e;
  const size_t lds = fp8_lds_bytes(c);
  hipLaunchKernelGGL(kern, dim3(c.blocks), dim3(64 * W), lds, stream, codes, scale, single, x, y, N, K, bs_log2,
                     c.ct, c.max_rows);
  return hipGetLastError();
}

template <int SF>
hipError_t launch_fp8_sf(const Fp8Cfg &c, const uint8_t *codes, const void *scale, float single, uint32_t bs_log2,
                         const uint16_t *x, uint16_t *y, uint32_t N, uint32_t K, hipStream_t stream) {
  if (c.waves == 8 && c.rp == 1 && K % 1024u == 0 && K >= 1024u && K <= 4096u)
    return launch_fp8_rx<SF>(c, codes, scale, single, bs_log2, x, y, N, K, stream);
  if (c.waves == 16) {
    if (c.rp == 2)
      return c.tail ? launch_fp8_cfg<SF, 16, 2, true>(c, codes, scale, single, bs_log2, x, y, N, K, stream)
                    : launch_fp8_cfg<SF, 16, 2, false>(c, codes, scale, single, bs_log2, x, y, N, K, stream);
    return c.tail ? launch_fp8_cfg<SF, 16, 1, true>(c, codes, scale, single, bs_log2, x, y, N, K, stream)
                  : launch_fp8_cfg<SF, 16, 1, false>(c, codes, scale, single, bs_log2, x, y, N, K, stream);
  }
  return c.tail ? launch_fp8_cfg<SF, 8, 1, true>(c, codes, scale, single, bs_log2, x, y, N, K, stream)
                : launch_fp8_cfg<SF, 8, 1, false>(c, codes, scale, single, bs_log2, x, y, N, K, stream);
}

// Launch shape, as for the int8 gemv: 8-wave workgroups; short rows (K <=
// 8192) two per CU above 16384 rows and one per CU below; long rows two per
// CU, one row at a time (4096 x 14336 with 128 x 128 BF16 block scales: 12.0
// against 12.5 us with one 16-wave workgroup per CU; per-row scales 11.0
// either way; graph-timed).
Fp8Cfg choose_fp8_cfg(uint32_t N, uint32_t K, bool block, uint32_t bs_log2) {
  const uint32_t cus = (uint32_t)device_cu_count();
  Fp8Cfg c{};
  c.waves = 8;
  const uint32_t per_cu = N > 16384u || K > 8192u ? 2u : 1u;
  const uint32_t W = (uint32_t)c.waves;
  c.blocks = per_cu * cus;
  const uint32_t need = (N + W - 1) / W;
  const uint32_t enough = (N + W * kFp8MaxRowsPerWave - 1) / (W * kFp8MaxRowsPerWave);
  if (c.blocks > need) c.blocks = need;
  if (c.blocks < enough) c.blocks = enough;
  const uint32_t tw = c.blocks * W;
  c.max_rows = (N + tw - 1) / tw;
  c.rp = 1;
  const uint32_t cpr = K / 16u;
  const size_t budget = kFp8LdsPerCu / per_cu;
  for (uint32_t ntiles = (cpr + kFp8TileRunsMax - 1) / kFp8TileRunsMax;; ++ntiles) {
    c.ct = ((cpr + ntiles - 1) / ntiles + 63u) / 64u * 64u;
    if (fp8_lds_bytes(c) <= budget || c.ct == 64u) break;
  }
  c.tail = (cpr % 64u) != 0;
  return c;
}

}  // namespace

hipError_t launch_fp8_gemv(const uint8_t *codes, const void *scale, Fp8ScaleKind kind, uint32_t block_size,
                           float single, uint32_t N, uint32_t K, const uint16_t *x, uint16_t *y, hipStream_t stream) {
  const bool block = kind == kFp8BlockBf16 || kind == kFp8BlockF32;
  const uint32_t bs_log2 = block ? (uint32_t)__builtin_ctz(block_size) : 10u;
  const Fp8Cfg c = choose_fp8_cfg(N, K, block, bs_log2);
  switch (kind) {
    case kFp8BlockBf16: return launch_fp8_sf<kSfBlockBf16>(c, codes, scale, single, bs_log2, x, y, N, K, stream);
    case kFp8BlockF32: return launch_fp8_sf<kSfBlockF32>(c, codes, scale, single, bs_log2, x, y, N, K, stream);
    default:  // per-row (scale [N]) or one global value (scale NULL)
      return launch_fp8_sf<kSfRow>(c, codes, kind == kFp8PerRow ? scale : nullptr, single, bs_log2, x, y, N, K,
                                   stream);
  }
}

}  // namespace int8w
