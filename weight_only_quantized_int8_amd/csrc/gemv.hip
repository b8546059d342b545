// gemv.hip -- m = 1 products for gfx950 (rustdoc page "MlxInt8Weight",
// methods gemv, gemv_silu_gate and gemv_silu_gate_resid):
//   gemv                  y[n] = sum_k w[n,k] x[k]
//   gemv_silu_gate        y[n] = sum_k w[n,k] silu(gate[k]) up[k]
//   gemv_silu_gate_resid  y[n] = x_resid[n] + sum_k w[n,k] silu(gate[k]) up[k]
// with w[n,k] = q[n,k] * s[n, k/gs] + b[n, k/gs].
//
// HBM-bound (the codes are ~94% of the bytes at gs = 64).  Design:
//  * Activation.  a[k] (x, or silu(gate)*up in fp32) is formed once per
//    workgroup and K-tile into LDS, with the sum of each run of 16
//    activations.  The gated product therefore never leaves the chip, and its
//    exp/divide cost is shared by every row the workgroup streams.
//  * Codes.  A lane owns runs of 16 consecutive codes (one 16-byte load), so a
//    wave-wide load streams 1 KiB of a row ("segment").  Each wave streams a
//    balanced, contiguous range of rows, RP rows side by side (the LDS reads
//    of a segment's activation serve all RP rows).  All loads go through
//    bounded buffer resources with the wave-uniform part of the offset in a
//    scalar register; past the wave's last row a load re-reads its last item.
//  * Arithmetic.  A run never straddles a group (gs is a multiple of 16), so
//    the affine terms factor out of the run:
//        sum_k (q_k s + b) a_k = s * sum_k q_k a_k + b * sum_k a_k.
//    Codes become binary16 (1024 + q) with one byte permute per two codes and
//    multiply through v_fma_mix_f32 (f16 x f32 -> f32, exact products); the
//    1024 offset folds into the bias: s*P' + (b - 1024 s)*S with
//    P' = sum (1024 + q) a and S = sum a.  Per code: half a permute and one
//    FMA.  (scale, bias - 1024 scale) pairs are staged per wave in LDS as fp32.
//  * Pipeline.  Loads run two blocks of U items ahead (the next block is
//    issued before the current one is consumed); the first block goes out
//    right after the activation and scale/bias loads, so the staging hides
//    under its latency without waiting for it.
//  * Reduction.  A row's lane partials are summed with a fixed DPP sequence as
//    soon as its last segment is consumed; with several K-tiles the partials
//    meet in LDS in tile order.  No atomics: results are deterministic.
//  * fp32 accumulation throughout; the residual is added in fp32 before the
//    one rounding to BF16.
//  * Short rows (in_features = 1024..4096, a multiple of 1024, plain x): a
//    lane's activations (16 per 1 KiB segment, at most 64) stay in its
//    registers instead of LDS, and each segment's (scale, bias) of the lane's
//    group is loaded with the codes.  A wave then needs no LDS, no barrier and
//    no staging before its first block (one block = one row), so it starts
//    streaming as a plain copy does; this form takes the 8B-shaped projections
//    from 70 to 74 % of HBM peak.
#include "common.h"
#include "launch.h"

namespace int8w {

namespace {

constexpr uint32_t kTileRunsMax = 1024;    // 16384 activations per LDS tile (staged scales)
constexpr uint32_t kTileRunsInline = 2048; // 32768 per tile when the scales come with the codes
constexpr int kLoadsPerBlock = 4;          // 1 KiB wave loads per pipeline block (U items x RP rows)
constexpr uint32_t kMaxRowsPerWave = 16;   // rows a wave may own
constexpr size_t kLdsPerCu = 156 * 1024;   // dynamic LDS budget of one CU
constexpr int kSbPerLane = 8;              // scale/bias entries a lane prefetches per tile

struct GemvCfg {
  int waves;           // waves per workgroup (8 or 16)
  int rp;              // rows each wave carries side by side (1 or 2)
  uint32_t blocks;     // workgroups
  uint32_t ct;         // 16-code runs per LDS tile (multiple of 64)
  uint32_t max_rows;   // most rows any wave owns
  bool tail;           // in_features not a multiple of 1024
  bool sbi;            // scales and biases loaded with the codes, not staged in LDS
};

// LDS bytes of one workgroup (layout in gemv_wave).
size_t lds_bytes(const GemvCfg &c, uint32_t gs) {
  const size_t tg = c.sbi ? 0u : (size_t)c.ct * 16u / gs;
  return (size_t)c.ct * 68u + (size_t)c.waves * c.max_rows * tg * 8u + (size_t)c.waves * c.max_rows * 4u;
}

// binary16 pair (1024 + q0, 1024 + q1) from bytes 0/1 (sel 0x04010400) or
// 2/3 (sel 0x04030402) of a code word: byte 0x64 over each code is the
// binary16 pattern of 1024 + q, exact for q in 0..255.
__device__ __forceinline__ uint32_t f16_pair(uint32_t word, uint32_t sel) {
  return __builtin_amdgcn_perm(0x64646464u, word, sel);
}

// sum_i (1024 + q_i) a_i over one lane's 16 codes.
__device__ __forceinline__ float run_dot(const u32x4 &w, const float4 &a0, const float4 &a1, const float4 &a2,
                                         const float4 &a3) {
  const uint32_t words[4] = {w.x, w.y, w.z, w.w};
  const float av[16] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w,
                        a2.x, a2.y, a2.z, a2.w, a3.x, a3.y, a3.z, a3.w};
  float p = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const f16x2 lo = __builtin_bit_cast(f16x2, f16_pair(words[i], 0x04010400u));
    const f16x2 hi = __builtin_bit_cast(f16x2, f16_pair(words[i], 0x04030402u));
    p = __builtin_fmaf((float)lo.x, av[4 * i + 0], p);
    p = __builtin_fmaf((float)lo.y, av[4 * i + 1], p);
    p = __builtin_fmaf((float)hi.x, av[4 * i + 2], p);
    p = __builtin_fmaf((float)hi.y, av[4 * i + 3], p);
  }
  return p;
}

// Sum over the 64 lanes of a wave in a fixed order (row-wise shifts, then row
// broadcasts); the total lands in lane 63.
__device__ __forceinline__ float wave_sum_lane63(float v) {
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x111, 0xf, 0xf, true));
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x112, 0xf, 0xf, true));
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x114, 0xf, 0xf, true));
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x118, 0xf, 0xf, true));
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x142, 0xa, 0xf, false));
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x143, 0xc, 0xf, false));
  return v;
}

__device__ __forceinline__ uint32_t uniform(uint32_t v) { return __builtin_amdgcn_readfirstlane(v); }

// The weights one launch streams: one for gemv and the gated variants, up to
// kMaxTargets sharing one activation for gemv_multi (same in_features and
// group size).  Passed by value as a kernel argument.
constexpr int kMaxTargets = 4;
struct GemvTargets {
  const uint8_t *codes[kMaxTargets];
  const uint16_t *scales[kMaxTargets];
  const uint16_t *biases[kMaxTargets];
  uint16_t *y[kMaxTargets];
  uint32_t n[kMaxTargets];         // rows of each weight
  uint32_t wave_end[kMaxTargets];  // waves [wave_end[i-1], wave_end[i]) stream weight i
  uint32_t count;
};

template <int U, int RP>
struct Block {
  u32x4 q[U][RP];
  uint16_t s[U][RP], b[U][RP];  // BF16 bits of the lane's group scale and bias (SBI only)
};

// LDS layout of one workgroup (dynamic):
//   act   [NSEG][4][64] float4   activation of lane l's 16 codes in segment s
//   ssum  [NSEG][64] float       their sum
//   sb    [W][max_rows][TG] float2   each wave's (scale, bias - 1024 scale); not with SBI
//   part  [W][max_rows] float        row partial sums across K-tiles
// SBI: each item's scale and bias (of the lane's group) are loaded with its
// codes instead of being staged per tile, which frees the LDS for a tile of
// up to 32768 activations: the long rows of a 16-wave workgroup (in_features
// 16385..32768) then run as one tile, with no drain and second prologue in
// the middle of the stream.  Same arithmetic per run; for shapes the staged
// form also covers in one tile, the same bits.
template <int EPI, int W, int RP, int U, bool TAIL, bool SBI>
__device__ __forceinline__ void gemv_wave(const uint8_t *__restrict__ codes, const uint16_t *__restrict__ scales,
                                          const uint16_t *__restrict__ biases, uint16_t *y, uint32_t N,
                                          uint32_t lw, uint32_t TW, const uint16_t *__restrict__ xg,
                                          const uint16_t *__restrict__ up, const uint16_t *resid, uint32_t K,
                                          uint32_t gs_log2, uint32_t tile_runs, uint32_t max_rows) {
  // This wave is wave lw of the TW waves that stream the N rows of one
  // weight.  y may be resid itself (in-place residual): each output element
  // reads its own residual before it is written, by the same lane.
  constexpr int kThreads = 64 * W;
  constexpr uint32_t kRunsMax = SBI ? kTileRunsInline : kTileRunsMax;
  constexpr int kStage = (int)(kRunsMax + kThreads - 1) / kThreads;  // runs staged per thread
  extern __shared__ float4 lds4[];
  const uint32_t CT = tile_runs;
  const uint32_t NSEG = CT >> 6;
  const uint32_t TG = SBI ? 0u : (CT << 4) >> gs_log2;
  float4 *act = lds4;
  float *ssum = reinterpret_cast<float *>(lds4 + NSEG * 256);
  float2 *sb_all = reinterpret_cast<float2 *>(ssum + NSEG * 64);
  float *part_all = reinterpret_cast<float *>(sb_all + W * max_rows * TG);

  const uint32_t tid = threadIdx.x;
  const uint32_t lane = tid & 63u;
  const uint32_t wave = uniform(tid >> 6);
  const uint32_t rq = N / TW, rr = N % TW;  // the first rr waves own rq + 1 rows
  const uint32_t rbeg = lw * rq + (lw < rr ? lw : rr);
  const uint32_t nr = lw < TW ? rq + (lw < rr ? 1u : 0u) : 0u;
  const uint32_t ngrp = (nr + RP - 1) / RP;  // row groups of RP rows
  const uint32_t cpr = K >> 4;
  const uint32_t G = K >> gs_log2;
  const uint32_t gps = 1024u >> gs_log2;  // groups per segment
  const uint32_t seg_sb = gps << 1;         // scale bytes per segment (SBI)

  const auto rw = make_rsrc(codes + (size_t)rbeg * K, nr * K);
  const auto rx = make_rsrc(xg, K * 2u);
  const auto ru = make_rsrc(EPI != kEpiNone ? up : xg, K * 2u);
  // a wave without rows still issues its (unused) scale/bias loads: point
  // them at the weight's first row
  const uint16_t *srow = scales + (size_t)(nr ? rbeg : 0u) * G;
  const uint16_t *brow = biases + (size_t)(nr ? rbeg : 0u) * G;
  const auto rsc = make_rsrc(scales + (size_t)rbeg * G, SBI ? nr * G * 2u : 0u);
  const auto rbi = make_rsrc(biases + (size_t)rbeg * G, SBI ? nr * G * 2u : 0u);
  const uint32_t v_sg = ((lane << 4) >> gs_log2) << 1;  // the lane's group in a segment, bytes (SBI)
  float2 *sb = sb_all + wave * max_rows * TG;
  float *part = part_all + wave * max_rows;

  // per-lane offsets; everything else is wave-uniform
  const uint32_t vo_w = lane << 4;
  const uint32_t lane_grp = (lane << 4) >> gs_log2;
  const uint32_t v_act = lane << 4;
  const uint32_t v_s = lane << 2;
  const uint32_t v_sb = lane_grp << 3;

  float acc[RP];
#pragma unroll
  for (int r = 0; r < RP; ++r) acc[r] = 0.f;
  Block<U, RP> A, B;

  for (uint32_t t0 = 0; t0 < cpr; t0 += CT) {
    const uint32_t ct = (cpr - t0) < CT ? (cpr - t0) : CT;
    const bool last_tile = t0 + ct == cpr;
    const uint32_t nseg = (ct + 63u) >> 6;
    const uint32_t nitems = ngrp * nseg;
    const uint32_t nblk = (nitems + U - 1) / U;
    const uint32_t tg = (ct << 4) >> gs_log2;
    const uint32_t g0 = (t0 << 4) >> gs_log2;
    const uint32_t last_lanes = ct - ((nseg - 1u) << 6);
    // lanes past the end of a partial last segment load nothing and read a
    // staged (finite) scale/bias entry; their activations are zero
    const uint32_t vo_w_last = TAIL && lane >= last_lanes ? kOutOfRange : vo_w;
    const uint32_t v_sb_last = TAIL && lane >= last_lanes ? 0u : v_sb;
    const uint32_t v_sg_last = TAIL && lane >= last_lanes ? kOutOfRange : v_sg;  // reads zero
    const uint32_t grp_skip = RP * K - (nseg << 10);  // to the next row group (mod 2^32)
    const uint32_t grp_skip_s = RP * G * 2u - nseg * seg_sb;
    const uint32_t last_off = (nr ? nr - 1u : 0u) * K + (t0 << 4) + ((nseg - 1u) << 10);
    const uint32_t last_soff = (nr ? nr - 1u : 0u) * G * 2u + (g0 << 1) + (nseg - 1u) * seg_sb;

    uint32_t i_off = t0 << 4, i_soff = g0 << 1, i_seg = 0, i_grp = 0;
    auto issue = [&](Block<U, RP> &blk) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        uint32_t vw = vo_w, vs = v_sg;
        if constexpr (TAIL) {
          vw = (i_seg == nseg - 1u) ? vo_w_last : vo_w;
          vs = (i_seg == nseg - 1u) ? v_sg_last : v_sg;
        }
#pragma unroll
        for (int r = 0; r < RP; ++r) {
          // past the wave's rows a load re-reads the last segment of its last
          // row (last_off), with that segment's lane mask
          const bool live = i_grp < ngrp && i_grp * RP + r < nr;
          const uint32_t sw = uniform(live ? i_off + r * K : last_off);
          const uint32_t vwr = live ? vw : vo_w_last;
          blk.q[u][r] = __builtin_amdgcn_raw_buffer_load_b128(rw, (int)vwr, (int)sw, kAuxNontemporal);
          if constexpr (SBI) {
            const uint32_t ss = uniform(live ? i_soff + r * G * 2u : last_soff);
            const uint32_t vsr = live ? vs : v_sg_last;
            blk.s[u][r] = __builtin_amdgcn_raw_buffer_load_b16(rsc, (int)vsr, (int)ss, 0);
            blk.b[u][r] = __builtin_amdgcn_raw_buffer_load_b16(rbi, (int)vsr, (int)ss, 0);
          }
        }
        i_off += 1024u;
        if constexpr (SBI) i_soff += seg_sb;
        if (++i_seg == nseg) {
          i_seg = 0;
          ++i_grp;
          i_off += grp_skip;
          if constexpr (SBI) i_soff += grp_skip_s;
        }
      }
    };
    uint32_t c_grp = 0, c_seg = 0;
    auto consume = [&](const Block<U, RP> &blk) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (c_grp < ngrp) {
          const float4 *ap = reinterpret_cast<const float4 *>(reinterpret_cast<const char *>(act) +
                                                              uniform(c_seg << 12) + v_act);
          const float4 a0 = ap[0], a1 = ap[64], a2 = ap[128], a3 = ap[192];
          const float S = *reinterpret_cast<const float *>(reinterpret_cast<const char *>(ssum) +
                                                           uniform(c_seg << 8) + v_s);
          uint32_t vs = v_sb;
          if constexpr (TAIL && !SBI) vs = (c_seg == nseg - 1u) ? v_sb_last : v_sb;
#pragma unroll
          for (int r = 0; r < RP; ++r) {
            float2 sbv;
            if constexpr (SBI) {
              sbv.x = bf16_bits_to_f32(blk.s[u][r]);
              sbv.y = __builtin_fmaf(-1024.f, sbv.x, bf16_bits_to_f32(blk.b[u][r]));
            } else {
              const uint32_t row = c_grp * RP + r;
              const uint32_t rs = row < nr ? row : 0u;
              sbv = *reinterpret_cast<const float2 *>(reinterpret_cast<const char *>(sb) +
                                                      uniform((rs * tg + c_seg * gps) << 3) + vs);
            }
            const float p = run_dot(blk.q[u][r], a0, a1, a2, a3);
            acc[r] = __builtin_fmaf(sbv.x, p, __builtin_fmaf(sbv.y, S, acc[r]));
          }
          if (c_seg == nseg - 1u) {  // the group's rows are done for this tile
#pragma unroll
            for (int r = 0; r < RP; ++r) {
              const uint32_t row = c_grp * RP + r;
              if (row < nr) {
                const float tot = wave_sum_lane63(acc[r]);
                if (lane == 63u) {
                  float v = t0 ? part[row] + tot : tot;
                  if (last_tile) {
                    if constexpr (EPI == kEpiSiluGateResid) v += bf16_bits_to_f32(resid[rbeg + row]);
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

    // 1. activation loads, then this wave's scales and biases for the tile
    //    (staged form), then the first weight block: all in flight together
    u32x4 xv[kStage][2], uv[kStage][2];
#pragma unroll
    for (int s = 0; s < kStage; ++s) {
      const uint32_t e = tid + s * kThreads;
      const uint32_t off = e < ct ? (t0 + e) * 32u : kOutOfRange;
      xv[s][0] = buf_load_b128(rx, off);
      xv[s][1] = buf_load_b128(rx, off + 16u);
      if constexpr (EPI != kEpiNone) {
        uv[s][0] = buf_load_b128(ru, off);
        uv[s][1] = buf_load_b128(ru, off + 16u);
      }
    }
    const uint32_t nsb = nr * tg;
    const uint32_t tg_inv = (uint32_t)(0xFFFFFFFFu / tg) + 1u;  // e / tg == umulhi(e, tg_inv) for e < 2^16
    uint16_t sv[kSbPerLane], bv[kSbPerLane];
    if constexpr (!SBI) {
#pragma unroll
      for (int j = 0; j < kSbPerLane; ++j) {
        const uint32_t e = lane + 64u * j;
        const uint32_t r = __umulhi(e, tg_inv), g = e - r * tg;
        const uint32_t src = e < nsb ? r * G + g0 + g : 0u;
        sv[j] = srow[src];
        bv[j] = brow[src];
      }
    }
    // the first weight block goes out after the small loads and unconditionally
    // (a wave without items loads out of range): vmcnt counts in order, so
    // waiting for the activation and the scales then never waits for it
    issue(A);
    if (t0) __syncthreads();  // everyone is done with the previous tile's activation
    // 2. form the activation tile; runs past the end are written as zeros
#pragma unroll
    for (int s = 0; s < kStage; ++s) {
      const uint32_t e = tid + s * kThreads;
      if (e < (nseg << 6)) {
        const uint32_t wv[8] = {xv[s][0].x, xv[s][0].y, xv[s][0].z, xv[s][0].w,
                                xv[s][1].x, xv[s][1].y, xv[s][1].z, xv[s][1].w};
        uint32_t uw[8];
        if constexpr (EPI != kEpiNone) {
          uw[0] = uv[s][0].x; uw[1] = uv[s][0].y; uw[2] = uv[s][0].z; uw[3] = uv[s][0].w;
          uw[4] = uv[s][1].x; uw[5] = uv[s][1].y; uw[6] = uv[s][1].z; uw[7] = uv[s][1].w;
        }
        float4 *dst = act + (e >> 6) * 256u + (e & 63u);
        float sum = 0.f;
#pragma unroll
        for (int f = 0; f < 4; ++f) {  // four activations (one float4) at a time
          float a0 = bf16_lo(wv[2 * f]), a1 = bf16_hi(wv[2 * f]);
          float a2 = bf16_lo(wv[2 * f + 1]), a3 = bf16_hi(wv[2 * f + 1]);
          if constexpr (EPI != kEpiNone) {
            a0 = silu_mul(a0, bf16_lo(uw[2 * f]));
            a1 = silu_mul(a1, bf16_hi(uw[2 * f]));
            a2 = silu_mul(a2, bf16_lo(uw[2 * f + 1]));
            a3 = silu_mul(a3, bf16_hi(uw[2 * f + 1]));
          }
          sum += a0; sum += a1; sum += a2; sum += a3;
          dst[f * 64] = make_float4(a0, a1, a2, a3);
        }
        ssum[e] = sum;
      }
    }
    __syncthreads();
    if constexpr (!SBI) {
      // this wave's private (scale, bias - 1024 scale) slice: only this wave
      // reads it, after writing it, and its previous tile is consumed
#pragma unroll
      for (int j = 0; j < kSbPerLane; ++j) {
        const uint32_t e = lane + 64u * j;
        if (e < nsb) {
          const float sc = bf16_bits_to_f32(sv[j]);
          sb[e] = make_float2(sc, __builtin_fmaf(-1024.f, sc, bf16_bits_to_f32(bv[j])));
        }
      }
      for (uint32_t e0 = 64u * kSbPerLane; e0 < nsb; e0 += 64u * kSbPerLane) {  // rows beyond the prefetch
#pragma unroll
        for (int j = 0; j < kSbPerLane; ++j) {
          const uint32_t e = e0 + lane + 64u * j;
          const uint32_t r = __umulhi(e, tg_inv), g = e - r * tg;
          const uint32_t src = e < nsb ? r * G + g0 + g : 0u;
          sv[j] = srow[src];
          bv[j] = brow[src];
        }
#pragma unroll
        for (int j = 0; j < kSbPerLane; ++j) {
          const uint32_t e = e0 + lane + 64u * j;
          if (e < nsb) {
            const float sc = bf16_bits_to_f32(sv[j]);
            sb[e] = make_float2(sc, __builtin_fmaf(-1024.f, sc, bf16_bits_to_f32(bv[j])));
          }
        }
      }
    }
    // 3. two-stage pipeline, two blocks per iteration and the rest after
    //    the loop.  The loop has a single exit: with an exit after every
    //    block, the compiler's wait counts at the loop head also covered the
    //    paths that leave, and it waited there for the block just issued.
    //    After each consume the other block's loads (U RP items, each its
    //    codes, and with SBI its scale and bias) may still be in flight, and
    //    nothing older: said explicitly, because a consume whose items are
    //    past the wave's rows reads nothing and so waits for nothing, and the
    //    compiler would otherwise wait for every load before reusing the
    //    consumed block's registers.
    constexpr int kBlk = (SBI ? 3 : 1) * U * RP;
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

// The register-resident form for in_features = NS * 1024 (NS = 1..4), plain
// activation.  Same row partition, arithmetic and reduction as gemv_wave; a
// pipeline block is one row (NS segments), two rows in flight.
template <int NS>
__device__ __forceinline__ void gemv_wave_rx(const uint8_t *__restrict__ codes, const uint16_t *__restrict__ scales,
                                             const uint16_t *__restrict__ biases, uint16_t *y, uint32_t N,
                                             uint32_t lw, uint32_t TW, const uint16_t *__restrict__ xg,
                                             uint32_t gs_log2) {
  constexpr uint32_t K = NS * 1024u;
  const uint32_t lane = threadIdx.x & 63u;
  const uint32_t rq = N / TW, rr = N % TW;
  const uint32_t rbeg = lw * rq + (lw < rr ? lw : rr);
  const uint32_t nr = lw < TW ? rq + (lw < rr ? 1u : 0u) : 0u;
  const uint32_t G = K >> gs_log2;
  const uint32_t seg_sb = (1024u >> gs_log2) << 1;      // scale bytes per segment
  const auto rw = make_rsrc(codes + (size_t)rbeg * K, nr * K);
  const auto rx = make_rsrc(xg, K * 2u);
  const auto rsc = make_rsrc(scales + (size_t)rbeg * G, nr * G * 2u);
  const auto rbi = make_rsrc(biases + (size_t)rbeg * G, nr * G * 2u);
  const uint32_t vo_w = lane << 4;
  const uint32_t v_sg = ((lane << 4) >> gs_log2) << 1;  // the lane's group in a segment, bytes

  struct RowBlock {
    u32x4 q[NS];
    uint16_t s[NS], b[NS];  // BF16 bits of the lane's group scale and bias
  };
  // the activation loads go out first: waiting for them never waits for codes
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
      const uint32_t sw = uniform(row * K + (u << 10));
      const uint32_t ss = uniform(row * G * 2u + u * seg_sb);
      blk.q[u] = __builtin_amdgcn_raw_buffer_load_b128(rw, (int)vo_w, (int)sw, kAuxNontemporal);
      blk.s[u] = __builtin_amdgcn_raw_buffer_load_b16(rsc, (int)v_sg, (int)ss, 0);
      blk.b[u] = __builtin_amdgcn_raw_buffer_load_b16(rbi, (int)v_sg, (int)ss, 0);
    }
    ++i_row;
  };
  RowBlock A, B;
  issue(A);
  float a[NS][16], S[NS];
#pragma unroll
  for (int u = 0; u < NS; ++u) {
    const uint32_t wv[8] = {xw[u][0].x, xw[u][0].y, xw[u][0].z, xw[u][0].w,
                            xw[u][1].x, xw[u][1].y, xw[u][1].z, xw[u][1].w};
    float sum = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      a[u][2 * i] = bf16_lo(wv[i]);
      a[u][2 * i + 1] = bf16_hi(wv[i]);
      sum += a[u][2 * i];
      sum += a[u][2 * i + 1];
    }
    S[u] = sum;
  }
  uint32_t c_row = 0;
  auto consume = [&](const RowBlock &blk) {
    float acc = 0.f;
#pragma unroll
    for (int u = 0; u < NS; ++u) {
      const float sc = bf16_bits_to_f32(blk.s[u]);
      const float bb = __builtin_fmaf(-1024.f, sc, bf16_bits_to_f32(blk.b[u]));
      const float p = run_dot(blk.q[u], make_float4(a[u][0], a[u][1], a[u][2], a[u][3]),
                              make_float4(a[u][4], a[u][5], a[u][6], a[u][7]),
                              make_float4(a[u][8], a[u][9], a[u][10], a[u][11]),
                              make_float4(a[u][12], a[u][13], a[u][14], a[u][15]));
      acc = __builtin_fmaf(sc, p, __builtin_fmaf(bb, S[u], acc));
    }
    const float tot = wave_sum_lane63(acc);
    if (lane == 63u) y[rbeg + c_row] = to_bf16_bits(tot);
    ++c_row;
  };
  // two-stage pipeline in a loop with a single exit (see gemv_wave); the
  // scale and bias stay 16-bit values until they are used, so that no
  // arithmetic on a block just requested is placed at the loop's end
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

// MR = 2..4 rows of X (gemm with a few rows) on the register-resident
// shapes: the m = 1 form above, with each run of 16 codes converted once to
// BF16 pairs (exact: a code has at most 8 significant bits) and multiplied
// into every row's activations, which the lane holds as the BF16 pairs it
// loaded, by v_dot2c_f32_bf16 (two exact products per operation).  The affine
// terms factor out of the run as in gemv_wave: s * sum q x + b * sum x, per
// row.  Per code: 1.5 operations to convert, 0.5 per row to multiply.
template <int NS, int MR>
__device__ __forceinline__ void gemv_wave_rxm(const uint8_t *__restrict__ codes, const uint16_t *__restrict__ scales,
                                              const uint16_t *__restrict__ biases, uint16_t *Y, uint32_t N,
                                              uint32_t lw, uint32_t TW, const uint16_t *__restrict__ X,
                                              uint32_t gs_log2) {
  constexpr uint32_t K = NS * 1024u;
  const uint32_t lane = threadIdx.x & 63u;
  const uint32_t rq = N / TW, rr = N % TW;
  const uint32_t rbeg = lw * rq + (lw < rr ? lw : rr);
  const uint32_t nr = lw < TW ? rq + (lw < rr ? 1u : 0u) : 0u;
  const uint32_t G = K >> gs_log2;
  const uint32_t seg_sb = (1024u >> gs_log2) << 1;      // scale bytes per segment
  const auto rw = make_rsrc(codes + (size_t)rbeg * K, nr * K);
  const auto rx = make_rsrc(X, MR * K * 2u);
  const auto rsc = make_rsrc(scales + (size_t)rbeg * G, nr * G * 2u);
  const auto rbi = make_rsrc(biases + (size_t)rbeg * G, nr * G * 2u);
  const uint32_t vo_w = lane << 4;
  const uint32_t v_sg = ((lane << 4) >> gs_log2) << 1;  // the lane's group in a segment, bytes

  struct RowBlock {
    u32x4 q[NS];
    uint16_t s[NS], b[NS];  // BF16 bits of the lane's group scale and bias
  };
  // the activation loads go out first: waiting for them never waits for codes
  u32x4 xw[MR][NS][2];
#pragma unroll
  for (int r = 0; r < MR; ++r)
#pragma unroll
    for (int u = 0; u < NS; ++u) {
      xw[r][u][0] = buf_load_b128(rx, r * (K * 2u) + (u << 11) + (lane << 5));
      xw[r][u][1] = buf_load_b128(rx, r * (K * 2u) + (u << 11) + (lane << 5) + 16u);
    }
  uint32_t i_row = 0;
  auto issue = [&](RowBlock &blk) {
    // past the wave's rows a block re-reads its last row
    const uint32_t row = i_row < nr ? i_row : (nr ? nr - 1u : 0u);
#pragma unroll
    for (int u = 0; u < NS; ++u) {
      const uint32_t sw = uniform(row * K + (u << 10));
      const uint32_t ss = uniform(row * G * 2u + u * seg_sb);
      blk.q[u] = __builtin_amdgcn_raw_buffer_load_b128(rw, (int)vo_w, (int)sw, kAuxNontemporal);
      blk.s[u] = __builtin_amdgcn_raw_buffer_load_b16(rsc, (int)v_sg, (int)ss, 0);
      blk.b[u] = __builtin_amdgcn_raw_buffer_load_b16(rbi, (int)v_sg, (int)ss, 0);
    }
    ++i_row;
  };
  RowBlock A, B;
  issue(A);
  float S[MR][NS];  // the sum of the lane's 16 activations of each row and segment
#pragma unroll
  for (int r = 0; r < MR; ++r)
#pragma unroll
    for (int u = 0; u < NS; ++u) {
      const uint32_t wv[8] = {xw[r][u][0].x, xw[r][u][0].y, xw[r][u][0].z, xw[r][u][0].w,
                              xw[r][u][1].x, xw[r][u][1].y, xw[r][u][1].z, xw[r][u][1].w};
      float sum = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        sum += bf16_lo(wv[i]);
        sum += bf16_hi(wv[i]);
      }
      S[r][u] = sum;
    }
  uint32_t c_row = 0;
  auto consume = [&](const RowBlock &blk) {
    float acc[MR];
#pragma unroll
    for (int r = 0; r < MR; ++r) acc[r] = 0.f;
#pragma unroll
    for (int u = 0; u < NS; ++u) {
      const float sc = bf16_bits_to_f32(blk.s[u]);
      const float bi = bf16_bits_to_f32(blk.b[u]);
      // codes 2i, 2i + 1 of the run as a BF16 pair (the fp32 value of a code
      // has zero low halves, so its high half is the BF16 value)
      const uint32_t words[4] = {blk.q[u].x, blk.q[u].y, blk.q[u].z, blk.q[u].w};
      uint32_t cb[8];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t f0 = __builtin_bit_cast(uint32_t, code_f32(words[j], 0));
        const uint32_t f1 = __builtin_bit_cast(uint32_t, code_f32(words[j], 1));
        const uint32_t f2 = __builtin_bit_cast(uint32_t, code_f32(words[j], 2));
        const uint32_t f3 = __builtin_bit_cast(uint32_t, code_f32(words[j], 3));
        cb[2 * j] = __builtin_amdgcn_perm(f1, f0, 0x07060302u);
        cb[2 * j + 1] = __builtin_amdgcn_perm(f3, f2, 0x07060302u);
      }
#pragma unroll
      for (int r = 0; r < MR; ++r) {
        const uint32_t xv[8] = {xw[r][u][0].x, xw[r][u][0].y, xw[r][u][0].z, xw[r][u][0].w,
                                xw[r][u][1].x, xw[r][u][1].y, xw[r][u][1].z, xw[r][u][1].w};
        float p = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i)
          p = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, cb[i]), __builtin_bit_cast(bf16x2, xv[i]), p,
                                              false);
        acc[r] = __builtin_fmaf(sc, p, __builtin_fmaf(bi, S[r][u], acc[r]));
      }
    }
#pragma unroll
    for (int r = 0; r < MR; ++r) {
      const float tot = wave_sum_lane63(acc[r]);
      if (lane == 63u) Y[(size_t)r * N + rbeg + c_row] = to_bf16_bits(tot);
    }
    ++c_row;
  };
  // the same two-stage pipeline as gemv_wave_rx
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

// gemm for m = MR rows on the register-resident shapes: one 8-wave workgroup
// per CU (the activations of four rows take up to 128 registers a lane).
template <int NS, int MR>
__global__ __launch_bounds__(512) void k_gemv_rows(const uint8_t *__restrict__ codes,
                                                    const uint16_t *__restrict__ scales,
                                                    const uint16_t *__restrict__ biases, const uint16_t *__restrict__ X,
                                                    uint16_t *Y, uint32_t N, uint32_t gs_log2) {
  const uint32_t gw = blockIdx.x * 8u + uniform(threadIdx.x >> 6);
  gemv_wave_rxm<NS, MR>(codes, scales, biases, Y, N, gw, gridDim.x * 8u, X, gs_log2);
}

// gemm with MR rows of X (two, where it is used) on long rows (in_features
// above 4096, a multiple of 1024): the arithmetic of gemv_wave_rxm (codes converted once
// per run to BF16 pairs, v_dot2c_f32_bf16 into every row, s * sum q x +
// b * sum x per run, the same reduction), with X kept in LDS instead of
// registers.  The workgroup copies X's BF16 rows into LDS once (exact: no
// conversion), each run's two 16-byte halves placed 1 KiB apart so that a
// wave's reads of one half are contiguous, with the fp32 sum of each run's
// 16 activations beside them; the waves then stream their rows in blocks of U
// segments, scale and bias loaded with each segment's codes, two blocks in
// flight.
// LDS: xt [MR][K] BF16 (segment s of row r at r*2K + 2048 s: lane l's first
// half at + 16 l, its second at + 1024 + 16 l), then ssum [MR][K/16] fp32.
constexpr uint32_t kRowsLdsMaxMK = 65536;  // MR * in_features: 147 KiB of LDS

template <int MR>
__global__ __launch_bounds__(1024) void k_gemv_rows_lds(const uint8_t *__restrict__ codes,
                                                        const uint16_t *__restrict__ scales,
                                                        const uint16_t *__restrict__ biases,
                                                        const uint16_t *__restrict__ X, uint16_t *Y, uint32_t N,
                                                        uint32_t K, uint32_t gs_log2) {
  constexpr int W = 16, U = 4;
  constexpr uint32_t kThreads = 64u * W;
  constexpr int kXRuns = (int)((kRowsLdsMaxMK / 16u + kThreads - 1u) / kThreads);  // X runs per thread
  extern __shared__ u32x4 ldsx[];
  uint8_t *xt = reinterpret_cast<uint8_t *>(ldsx);
  const uint32_t runs = K >> 4;  // runs of 16 codes per row
  float *ssum = reinterpret_cast<float *>(xt + MR * K * 2u);

  const uint32_t tid = threadIdx.x;
  const uint32_t lane = tid & 63u;
  const uint32_t lw = blockIdx.x * W + uniform(tid >> 6);
  const uint32_t TW = gridDim.x * W;
  const uint32_t rq = N / TW, rr = N % TW;
  const uint32_t rbeg = lw * rq + (lw < rr ? lw : rr);
  const uint32_t nr = lw < TW ? rq + (lw < rr ? 1u : 0u) : 0u;
  const uint32_t nseg = K >> 10;
  const uint32_t G = K >> gs_log2;
  const uint32_t seg_sb = (1024u >> gs_log2) << 1;  // scale bytes per segment
  const auto rw = make_rsrc(codes + (size_t)rbeg * K, nr * K);
  const auto rsc = make_rsrc(scales + (size_t)rbeg * G, nr * G * 2u);
  const auto rbi = make_rsrc(biases + (size_t)rbeg * G, nr * G * 2u);
  const auto rx = make_rsrc(X, MR * K * 2u);
  const uint32_t vo_w = lane << 4;
  const uint32_t v_sg = ((lane << 4) >> gs_log2) << 1;  // the lane's group in a segment, bytes
  const uint32_t last_off = (nr ? nr - 1u : 0u) * K + ((nseg - 1u) << 10);
  const uint32_t last_soff = (nr ? nr - 1u : 0u) * G * 2u + (nseg - 1u) * seg_sb;

  // 1. X's runs (32 bytes each), then the first code block: waiting for the
  //    former never waits for the latter
  const uint32_t xruns = MR * runs;
  u32x4 xv[kXRuns][2];
#pragma unroll
  for (int j = 0; j < kXRuns; ++j) {
    const uint32_t e = tid + (uint32_t)j * kThreads;
    const uint32_t off = e < xruns ? e * 32u : kOutOfRange;
    xv[j][0] = buf_load_b128(rx, off);
    xv[j][1] = buf_load_b128(rx, off + 16u);
  }
  Block<U, 1> A, B;
  uint32_t i_off = 0, i_soff = 0, i_seg = 0, i_grp = 0;
  auto issue = [&](Block<U, 1> &blk) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      // past the wave's rows a load re-reads the last segment of its last row
      const bool live = i_grp < nr;
      const uint32_t sw = uniform(live ? i_off : last_off);
      const uint32_t ss = uniform(live ? i_soff : last_soff);
      blk.q[u][0] = __builtin_amdgcn_raw_buffer_load_b128(rw, (int)vo_w, (int)sw, kAuxNontemporal);
      blk.s[u][0] = __builtin_amdgcn_raw_buffer_load_b16(rsc, (int)v_sg, (int)ss, 0);
      blk.b[u][0] = __builtin_amdgcn_raw_buffer_load_b16(rbi, (int)v_sg, (int)ss, 0);
      i_off += 1024u;
      i_soff += seg_sb;
      if (++i_seg == nseg) {
        i_seg = 0;
        ++i_grp;
      }
    }
  };
  issue(A);

  // 2. X into LDS, with each run's sum (in the order gemv_wave_rxm sums)
#pragma unroll
  for (int j = 0; j < kXRuns; ++j) {
    const uint32_t e = tid + (uint32_t)j * kThreads;
    if (e < xruns) {
      const uint32_t r = e / runs, t = e - r * runs;  // row, run within the row
      uint8_t *dst = xt + r * K * 2u + ((t >> 6) << 11) + ((t & 63u) << 4);
      *reinterpret_cast<u32x4 *>(dst) = xv[j][0];
      *reinterpret_cast<u32x4 *>(dst + 1024u) = xv[j][1];
      const uint32_t wv[8] = {xv[j][0].x, xv[j][0].y, xv[j][0].z, xv[j][0].w,
                              xv[j][1].x, xv[j][1].y, xv[j][1].z, xv[j][1].w};
      float sum = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        sum += bf16_lo(wv[i]);
        sum += bf16_hi(wv[i]);
      }
      ssum[e] = sum;
    }
  }
  __syncthreads();

  float acc[MR];
#pragma unroll
  for (int r = 0; r < MR; ++r) acc[r] = 0.f;
  uint32_t c_grp = 0, c_seg = 0;
  auto consume = [&](const Block<U, 1> &blk) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (c_grp < nr) {
        const float sc = bf16_bits_to_f32(blk.s[u][0]);
        const float bi = bf16_bits_to_f32(blk.b[u][0]);
        const uint32_t words[4] = {blk.q[u][0].x, blk.q[u][0].y, blk.q[u][0].z, blk.q[u][0].w};
        uint32_t cb[8];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint32_t f0 = __builtin_bit_cast(uint32_t, code_f32(words[j], 0));
          const uint32_t f1 = __builtin_bit_cast(uint32_t, code_f32(words[j], 1));
          const uint32_t f2 = __builtin_bit_cast(uint32_t, code_f32(words[j], 2));
          const uint32_t f3 = __builtin_bit_cast(uint32_t, code_f32(words[j], 3));
          cb[2 * j] = __builtin_amdgcn_perm(f1, f0, 0x07060302u);
          cb[2 * j + 1] = __builtin_amdgcn_perm(f3, f2, 0x07060302u);
        }
        const uint32_t seg_off = uniform(c_seg << 11) + (lane << 4);
#pragma unroll
        for (int r = 0; r < MR; ++r) {
          const uint8_t *src = xt + r * K * 2u + seg_off;
          const u32x4 h0 = *reinterpret_cast<const u32x4 *>(src);
          const u32x4 h1 = *reinterpret_cast<const u32x4 *>(src + 1024u);
          const uint32_t xw[8] = {h0.x, h0.y, h0.z, h0.w, h1.x, h1.y, h1.z, h1.w};
          const float S = ssum[r * runs + (c_seg << 6) + lane];
          float p = 0.f;
#pragma unroll
          for (int i = 0; i < 8; ++i)
            p = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, cb[i]), __builtin_bit_cast(bf16x2, xw[i]),
                                                p, false);
          acc[r] = __builtin_fmaf(sc, p, __builtin_fmaf(bi, S, acc[r]));
        }
        if (c_seg == nseg - 1u) {  // the row's last segment
#pragma unroll
          for (int r = 0; r < MR; ++r) {
            const float tot = wave_sum_lane63(acc[r]);
            if (lane == 63u) Y[(size_t)r * N + rbeg + c_grp] = to_bf16_bits(tot);
            acc[r] = 0.f;
          }
        }
      }
      if (++c_seg == nseg) { c_seg = 0; ++c_grp; }
    }
  };
  // 3. the pipeline of gemv_wave (two blocks in flight, a single exit); after
  //    each consume only the other block's loads (codes, scale and bias of U
  //    items) may still be in flight
  const uint32_t nblk = (nr * nseg + U - 1u) / U;
  constexpr int kBlk = 3 * U;
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

// The wave body of a launch: the register-resident form (NS > 0) or the
// LDS-tiled one (NS == 0).
template <int NS, int EPI, int W, int RP, int U, bool TAIL, bool SBI>
__device__ __forceinline__ void gemv_body(const uint8_t *codes, const uint16_t *scales, const uint16_t *biases,
                                          uint16_t *y, uint32_t N, uint32_t lw, uint32_t TW, const uint16_t *xg,
                                          const uint16_t *up, const uint16_t *resid, uint32_t K, uint32_t gs_log2,
                                          uint32_t tile_runs, uint32_t max_rows) {
  if constexpr (NS > 0)
    gemv_wave_rx<NS>(codes, scales, biases, y, N, lw, TW, xg, gs_log2);
  else
    gemv_wave<EPI, W, RP, U, TAIL, SBI>(codes, scales, biases, y, N, lw, TW, xg, up, resid, K, gs_log2, tile_runs,
                                   max_rows);
}

// gemv, gemv_silu_gate, gemv_silu_gate_resid: one weight, all waves.
template <int NS, int EPI, int W, int RP, int U, bool TAIL, bool SBI>
__global__ __launch_bounds__(64 * W) void k_gemv(const uint8_t *__restrict__ codes,
                                                 const uint16_t *__restrict__ scales,
                                                 const uint16_t *__restrict__ biases, const uint16_t *__restrict__ xg,
                                                 const uint16_t *__restrict__ up, const uint16_t *resid, uint16_t *y,
                                                 uint32_t N, uint32_t K, uint32_t gs_log2, uint32_t tile_runs,
                                                 uint32_t max_rows) {
  const uint32_t gw = blockIdx.x * W + uniform(threadIdx.x >> 6);
  gemv_body<NS, EPI, W, RP, U, TAIL, SBI>(codes, scales, biases, y, N, gw, gridDim.x * W, xg, up, resid, K, gs_log2,
                                     tile_runs, max_rows);
}

// gemv_multi: the waves are dealt to the weights of the launch in proportion
// to their rows; each wave streams its share of one weight.
template <int NS, int W, int RP, int U, bool TAIL, bool SBI>
__global__ __launch_bounds__(64 * W) void k_gemv_multi(GemvTargets t, const uint16_t *__restrict__ xg, uint32_t K,
                                                       uint32_t gs_log2, uint32_t tile_runs, uint32_t max_rows) {
  const uint32_t gw = blockIdx.x * W + uniform(threadIdx.x >> 6);
  uint32_t j = 0;
#pragma unroll
  for (int i = 0; i + 1 < kMaxTargets; ++i) j += (i + 1 < (int)t.count && gw >= t.wave_end[i]) ? 1u : 0u;
  const uint8_t *codes = t.codes[0];
  const uint16_t *scales = t.scales[0], *biases = t.biases[0];
  uint16_t *y = t.y[0];
  uint32_t N = t.n[0], wb = 0, we = t.wave_end[0];
#pragma unroll
  for (int i = 1; i < kMaxTargets; ++i) {
    if (j == (uint32_t)i) {
      codes = t.codes[i]; scales = t.scales[i]; biases = t.biases[i]; y = t.y[i];
      N = t.n[i]; wb = t.wave_end[i - 1]; we = t.wave_end[i];
    }
  }
  // waves past the last weight's share (the grid is whole workgroups) own no rows
  gemv_body<NS, kEpiNone, W, RP, U, TAIL, SBI>(codes, scales, biases, y, N, gw - wb, we - wb, xg, xg, nullptr, K,
                                          gs_log2, tile_runs, max_rows);
}

// Expert-indexed gemv (the DynQuantizedStorage trait page, provided method
// indexed_moe_forward): slot p of tokens x topk takes the weight of expert
// ids[p] (rows ids[p]*N .. +N-1 of the stacked codes) and its token's input
// row (or its own, x_rows == topk).  Workgroup b serves slot b % slots, part
// b / slots of that slot's rows: every slot gets the same share of the GPU,
// and each slot streams its expert once, so an expert named by several slots
// is streamed once per slot.  A slot whose id is not below E writes NaN and
// reads no weight.
template <int NS, int W, int RP, int U, bool TAIL, bool SBI>
__global__ __launch_bounds__(64 * W) void k_moe_gemv(const uint8_t *__restrict__ codes,
                                                     const uint16_t *__restrict__ scales,
                                                     const uint16_t *__restrict__ biases,
                                                     const uint16_t *__restrict__ x, const uint32_t *__restrict__ ids,
                                                     uint16_t *y, uint32_t N, uint32_t E, uint32_t topk,
                                                     uint32_t x_rows, uint32_t slots, uint32_t K, uint32_t gs_log2,
                                                     uint32_t tile_runs, uint32_t max_rows) {
  const uint32_t p = blockIdx.x % slots;
  const uint32_t part = blockIdx.x / slots;
  const uint32_t TW = (gridDim.x / slots) * W;
  const uint32_t lw = part * W + uniform(threadIdx.x >> 6);
  const uint32_t e = uniform(ids[p]);
  uint16_t *yp = y + (size_t)p * N;
  if (e >= E) {
    const uint32_t rq = N / TW, rr = N % TW;
    const uint32_t rbeg = lw * rq + (lw < rr ? lw : rr);
    const uint32_t nr = rq + (lw < rr ? 1u : 0u);
    for (uint32_t r = threadIdx.x & 63u; r < nr; r += 64u) yp[rbeg + r] = 0x7FC0u;
    return;
  }
  const uint32_t t = p / topk, j = p - t * topk;
  const uint16_t *xp = x + ((size_t)t * x_rows + (x_rows == 1u ? 0u : j)) * K;
  const size_t G = K >> gs_log2;
  gemv_body<NS, kEpiNone, W, RP, U, TAIL, SBI>(codes + (size_t)e * N * K, scales + (size_t)e * N * G,
                                          biases + (size_t)e * N * G, yp, N, lw, TW, xp, xp, nullptr, K, gs_log2,
                                          tile_runs, max_rows);
}

// Expert-grouped form of the expert-indexed gemv, for several tokens and
// in_features = NS * 1024: every expert that some slot names is streamed
// once, against the activations of all slots that name it (up to kGrpC per
// pass).  Each workgroup derives the same routing from ids in LDS: the set
// of named experts (rank r = the r-th named expert in ascending order), then
// work items (expert rank, part of its rows) dealt over the grid, then for
// its item the slots naming the expert in ascending order.  The per-slot
// arithmetic is the register-resident gemv's, so every output is bit-identical
// to that of int8_gemv on the expert's rows.  Slots whose id is not below E
// get NaN, written by all workgroups over their share of the rows.
constexpr uint32_t kGrpMaxSlots = 256;
constexpr uint32_t kGrpMaxExperts = 512;
constexpr int kGrpC = 4;

template <int NS>
__global__ __launch_bounds__(512) void k_moe_grouped(const uint8_t *__restrict__ codes,
                                                     const uint16_t *__restrict__ scales,
                                                     const uint16_t *__restrict__ biases,
                                                     const uint16_t *__restrict__ x, const uint32_t *__restrict__ ids,
                                                     uint16_t *y, uint32_t N, uint32_t E, uint32_t topk,
                                                     uint32_t x_rows, uint32_t slots, uint32_t gs_log2) {
  constexpr uint32_t K = NS * 1024u;
  constexpr uint32_t W = 8;
  __shared__ uint32_t s_ids[kGrpMaxSlots];
  __shared__ unsigned long long s_mask[kGrpMaxExperts / 64];
  __shared__ uint32_t s_table[kGrpMaxSlots];  // expert of each rank
  __shared__ uint32_t s_list[kGrpMaxSlots];   // slots naming the item's expert
  __shared__ uint32_t s_meta[2];              // named experts, slots of the item's expert
  extern __shared__ float4 grp_act[];         // [kGrpC][NS][4][64] float4, then [kGrpC][NS][64] sums
  float *grp_sum = reinterpret_cast<float *>(grp_act + kGrpC * NS * 256);

  const uint32_t tid = threadIdx.x, lane = tid & 63u, wave = uniform(tid >> 6);
  const uint32_t G = K >> gs_log2;

  // 1. the named experts, in ascending order
  if (tid < kGrpMaxExperts / 64) s_mask[tid] = 0ull;
  if (tid < slots) s_ids[tid] = ids[tid];
  __syncthreads();
  if (tid < slots && s_ids[tid] < E) atomicOr(&s_mask[s_ids[tid] >> 6], 1ull << (s_ids[tid] & 63u));
  __syncthreads();
  if (wave == 0) {
    uint32_t base = 0;
    for (uint32_t wd = 0; wd < (E + 63u) / 64u; ++wd) {
      const unsigned long long msk = s_mask[wd];
      if ((msk >> lane) & 1ull) s_table[base + __popcll(msk & ((1ull << lane) - 1ull))] = wd * 64u + lane;
      base += __popcll(msk);
    }
    if (lane == 0) s_meta[0] = base;
  }
  __syncthreads();
  const uint32_t D = s_meta[0];

  // 2. slots without an expert: NaN over this workgroup's share of the rows
  {
    const uint32_t gq = N / gridDim.x, gr = N % gridDim.x, b = blockIdx.x;
    const uint32_t r0 = b * gq + (b < gr ? b : gr), rn = gq + (b < gr ? 1u : 0u);
    for (uint32_t j = 0; j < slots; ++j)
      if (s_ids[j] >= E)
        for (uint32_t r = tid; r < rn; r += 512u) y[(size_t)j * N + r0 + r] = 0x7FC0u;
  }
  if (D == 0) return;

  // 3. work items: (expert rank, part of its rows)
  const uint32_t P = gridDim.x >= D ? gridDim.x / D : 1u;
  const uint32_t seg_sb = (1024u >> gs_log2) << 1;
  const uint32_t v_sg = ((lane << 4) >> gs_log2) << 1;
  for (uint32_t item = blockIdx.x; item < D * P; item += gridDim.x) {
    const uint32_t e = s_table[item / P], part = item % P;
    __syncthreads();  // the previous item is done with s_list and the activations
    if (wave == 0) {
      uint32_t base = 0;
      for (uint32_t j0 = 0; j0 < slots; j0 += 64u) {
        const uint32_t j = j0 + lane;
        const bool hit = j < slots && s_ids[j] == e;
        const unsigned long long msk = __ballot(hit);
        if (hit) s_list[base + __popcll(msk & ((1ull << lane) - 1ull))] = j;
        base += __popcll(msk);
      }
      if (lane == 0) s_meta[1] = base;
    }
    __syncthreads();
    const uint32_t cnt = s_meta[1];
    // this wave's rows of the part
    const uint32_t pq = N / P, pr = N % P;
    const uint32_t pbeg = part * pq + (part < pr ? part : pr), pn = pq + (part < pr ? 1u : 0u);
    const uint32_t rq = pn / W, rr = pn % W;
    const uint32_t rbeg = pbeg + wave * rq + (wave < rr ? wave : rr);
    const uint32_t nr = rq + (wave < rr ? 1u : 0u);
    const auto rw = make_rsrc(codes + ((size_t)e * N + rbeg) * K, nr * K);
    const auto rsc = make_rsrc(scales + ((size_t)e * N + rbeg) * G, nr * G * 2u);
    const auto rbi = make_rsrc(biases + ((size_t)e * N + rbeg) * G, nr * G * 2u);

    for (uint32_t c0 = 0; c0 < cnt; c0 += kGrpC) {
      const uint32_t cs = cnt - c0 < (uint32_t)kGrpC ? cnt - c0 : (uint32_t)kGrpC;
      // stage the activations of slots s_list[c0 .. c0 + cs)
      if (c0) __syncthreads();  // the previous pass is done with them
      for (uint32_t q = tid; q < cs * NS * 64u; q += 512u) {
        const uint32_t c = q / (NS * 64u), run = q - c * (NS * 64u);
        const uint32_t slot = s_list[c0 + c];
        const uint32_t t = slot / topk, j = slot - t * topk;
        const uint4 *src = reinterpret_cast<const uint4 *>(x + ((size_t)t * x_rows + (x_rows == 1u ? 0u : j)) * K) +
                           2u * run;
        const uint4 v0 = src[0], v1 = src[1];
        const uint32_t wv[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
        float4 *dst = grp_act + ((c * NS + (run >> 6)) * 4u) * 64u + (run & 63u);
        float sum = 0.f;
#pragma unroll
        for (int f = 0; f < 4; ++f) {
          const float a0 = bf16_lo(wv[2 * f]), a1 = bf16_hi(wv[2 * f]);
          const float a2 = bf16_lo(wv[2 * f + 1]), a3 = bf16_hi(wv[2 * f + 1]);
          sum += a0; sum += a1; sum += a2; sum += a3;
          dst[f * 64] = make_float4(a0, a1, a2, a3);
        }
        grp_sum[(c * NS + (run >> 6)) * 64u + (run & 63u)] = sum;
      }
      __syncthreads();

      struct RowBlock {
        u32x4 q[NS];
        uint16_t s[NS], b[NS];
      };
      uint32_t i_row = 0;
      auto issue = [&](RowBlock &blk) {
        const uint32_t row = i_row < nr ? i_row : (nr ? nr - 1u : 0u);
#pragma unroll
        for (int u = 0; u < NS; ++u) {
          const uint32_t sw = uniform(row * K + (u << 10));
          const uint32_t ss = uniform(row * G * 2u + u * seg_sb);
          blk.q[u] = __builtin_amdgcn_raw_buffer_load_b128(rw, (int)(lane << 4), (int)sw, kAuxNontemporal);
          blk.s[u] = __builtin_amdgcn_raw_buffer_load_b16(rsc, (int)v_sg, (int)ss, 0);
          blk.b[u] = __builtin_amdgcn_raw_buffer_load_b16(rbi, (int)v_sg, (int)ss, 0);
        }
        ++i_row;
      };
      uint32_t c_row = 0;
      auto consume = [&](const RowBlock &blk) {
        // one slot at a time (not unrolled: keeps one slot's activations live)
#pragma unroll 1
        for (uint32_t c = 0; c < cs; ++c) {
          float acc = 0.f;
#pragma unroll
          for (int u = 0; u < NS; ++u) {
            const float sc = bf16_bits_to_f32(blk.s[u]);
            const float bb = __builtin_fmaf(-1024.f, sc, bf16_bits_to_f32(blk.b[u]));
            const float4 *ap = grp_act + ((c * NS + u) * 4u) * 64u + lane;
            const float p = run_dot(blk.q[u], ap[0], ap[64], ap[128], ap[192]);
            const float S = grp_sum[(c * NS + u) * 64u + lane];
            acc = __builtin_fmaf(sc, p, __builtin_fmaf(bb, S, acc));
          }
          const float tot = wave_sum_lane63(acc);
          if (lane == 63u) y[(size_t)s_list[c0 + c] * N + rbeg + c_row] = to_bf16_bits(tot);
        }
        ++c_row;
      };
      RowBlock A, B;
      issue(A);
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
  }
}

template <typename Kern>
hipError_t raise_lds_cap(Kern kern, bool &configured, int bytes = 160 * 1024) {
  if (configured) return hipSuccess;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e == hipSuccess) configured = true;
  return e;
}

template <int EPI, int W, int RP, bool TAIL, int NS = 0, bool SBI = false>
hipError_t launch_cfg(const GemvCfg &cfg, const GemvTargets &t, uint32_t K, uint32_t gs, const uint16_t *xg,
                      const uint16_t *up, const uint16_t *resid, hipStream_t stream) {
  static bool configured = false;  // raise the dynamic-LDS cap once per instantiation
  const uint32_t gs_log2 = (uint32_t)__builtin_ctz(gs);
  const size_t lds = NS ? 0u : lds_bytes(cfg, gs);  // the register-resident form uses no LDS
  if (t.count == 1) {
    auto kern = k_gemv<NS, EPI, W, RP, kLoadsPerBlock / RP, TAIL, SBI>;
    hipError_t e = raise_lds_cap(kern, configured);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, dim3(cfg.blocks), dim3(64 * W), lds, stream, t.codes[0], t.scales[0], t.biases[0], xg,
                       up, resid, t.y[0], t.n[0], K, gs_log2, cfg.ct, cfg.max_rows);
  } else {
    static bool configured_multi = false;
    auto kern = k_gemv_multi<NS, W, RP, kLoadsPerBlock / RP, TAIL, SBI>;
    hipError_t e = raise_lds_cap(kern, configured_multi);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, dim3(cfg.blocks), dim3(64 * W), lds, stream, t, xg, K, gs_log2, cfg.ct, cfg.max_rows);
  }
  return hipGetLastError();
}

// The register-resident form applies to a plain activation of 1024..4096
// values (a multiple of 1024) on the 8-wave, one-row-at-a-time shape.
bool rx_form(const GemvCfg &cfg, uint32_t K, GemvEpilogue epi) {
  return epi == kEpiNone && cfg.waves == 8 && cfg.rp == 1 && K % 1024u == 0 && K >= 1024u && K <= 4096u;
}

template <int EPI, bool TAIL>
hipError_t launch_shape(const GemvCfg &cfg, const GemvTargets &t, uint32_t K, uint32_t gs, const uint16_t *xg,
                        const uint16_t *up, const uint16_t *resid, hipStream_t stream) {
  if (cfg.waves == 16) {
    if constexpr (!TAIL) {
      if (cfg.sbi)
        return cfg.rp == 2 ? launch_cfg<EPI, 16, 2, false, 0, true>(cfg, t, K, gs, xg, up, resid, stream)
                           : launch_cfg<EPI, 16, 1, false, 0, true>(cfg, t, K, gs, xg, up, resid, stream);
    }
    return cfg.rp == 2 ? launch_cfg<EPI, 16, 2, TAIL>(cfg, t, K, gs, xg, up, resid, stream)
                       : launch_cfg<EPI, 16, 1, TAIL>(cfg, t, K, gs, xg, up, resid, stream);
  }
  return cfg.rp == 2 ? launch_cfg<EPI, 8, 2, TAIL>(cfg, t, K, gs, xg, up, resid, stream)
                     : launch_cfg<EPI, 8, 1, TAIL>(cfg, t, K, gs, xg, up, resid, stream);
}

// The activation tile of the LDS form: the whole row in one tile with
// staged scales when that fits the LDS budget; else, for 16-wave workgroups
// and in_features a multiple of 1024 up to 32768, one tile with the scales
// loaded per item (sbi); else several staged tiles.  One tile saves a drain
// of the stream, a barrier and a second prologue per extra tile: 8192 x 28672
// gs128 silu_gate_resid 41.9 -> 40.3 us (graph-timed, interleaved).  Where
// one staged tile fits, the staged form stays (per-item scale loads measured
// 0-4 % slower on 4096 x 14336).
void pick_tile(GemvCfg &c, uint32_t K, uint32_t gs, size_t budget) {
  const uint32_t cpr = K / 16u;
  c.tail = (cpr % 64u) != 0;
  c.sbi = false;
  uint32_t ntiles = (cpr + kTileRunsMax - 1) / kTileRunsMax;
  for (;; ++ntiles) {
    c.ct = ((cpr + ntiles - 1) / ntiles + 63u) / 64u * 64u;
    if (lds_bytes(c, gs) <= budget || c.ct == 64u) break;
  }
  if (ntiles > 1u && c.waves == 16 && !c.tail && cpr <= kTileRunsInline) {
    GemvCfg one = c;
    one.sbi = true;
    one.ct = cpr;  // a multiple of 64 runs: in_features is a multiple of 1024
    if (lds_bytes(one, gs) <= budget) c = one;
  }
}

// Deal the launch's waves to its weights in proportion to their rows (every
// weight at least one wave, none more waves than rows); returns the most
// rows any wave owns.
uint32_t deal_waves(uint32_t tw, const uint32_t *n, uint32_t count, uint32_t *wave_end) {
  uint64_t total = 0;
  for (uint32_t i = 0; i < count; ++i) total += n[i];
  uint32_t share[kMaxTargets], used = 0;
  for (uint32_t i = 0; i < count; ++i) {
    share[i] = (uint32_t)((uint64_t)tw * n[i] / total);
    if (share[i] == 0) share[i] = 1;
    used += share[i];
  }
  while (used < tw) {  // leftover waves to the weight with the most rows per wave
    uint32_t best = 0;
    for (uint32_t i = 1; i < count; ++i)
      if ((uint64_t)n[i] * share[best] > (uint64_t)n[best] * share[i]) best = i;
    ++share[best];
    ++used;
  }
  uint32_t acc = 0, max_rows = 0;
  for (uint32_t i = 0; i < count; ++i) {
    if (share[i] > n[i]) share[i] = n[i];
    acc += share[i];
    wave_end[i] = acc;
    const uint32_t r = (n[i] + share[i] - 1) / share[i];
    if (r > max_rows) max_rows = r;
  }
  for (uint32_t i = count; i < kMaxTargets; ++i) wave_end[i] = acc;
  return max_rows;
}

// Launch shape (measured on MI355X): short rows (K <= 8192) run 8-wave
// workgroups, two per CU when the launch has more than 16384 rows and one
// per CU otherwise (a small launch is latency-bound: fewer waves with two
// rows each beat more waves with one); long rows one 16-wave workgroup per
// CU, so one activation tile serves 16 waves, with two rows side by side
// when every wave owns at least two.
GemvCfg choose_cfg(const uint32_t *n, uint32_t count, uint32_t K, uint32_t gs, uint32_t *wave_end, int waves = 0,
                   int rp = 0, uint32_t wg_per_cu = 0) {
  const uint32_t cus = (uint32_t)device_cu_count();
  uint32_t N = 0;
  for (uint32_t i = 0; i < count; ++i) N += n[i];
  GemvCfg c{};
  c.waves = waves ? waves : (K <= 8192u ? 8 : 16);
  const uint32_t per_cu = wg_per_cu ? wg_per_cu : (c.waves == 8 && N > 16384u ? 2u : 1u);
  const uint32_t W = (uint32_t)c.waves;
  c.blocks = per_cu * cus;
  const uint32_t need = (N + W - 1) / W;
  if (c.blocks > need) c.blocks = need;
  const uint32_t enough = (N + W * kMaxRowsPerWave - 1) / (W * kMaxRowsPerWave);
  if (c.blocks < enough) c.blocks = enough;
  for (;; ++c.blocks) {  // a weight's share of waves is rounded: keep every wave within kMaxRowsPerWave rows
    c.max_rows = deal_waves(c.blocks * W, n, count, wave_end);
    if (c.max_rows <= kMaxRowsPerWave) break;
  }
  const uint32_t tw = c.blocks * W;
  c.blocks = (wave_end[count - 1] + W - 1) / W;  // no workgroup of idle waves only
  c.rp = rp ? rp : (c.waves == 16 && N / tw >= 2u ? 2 : 1);
  pick_tile(c, K, gs, kLdsPerCu / per_cu);
  return c;
}

hipError_t launch_targets(const GemvCfg &cfg, const GemvTargets &t, uint32_t K, uint32_t gs, GemvEpilogue epi,
                          const uint16_t *x_or_gate, const uint16_t *up, const uint16_t *x_resid,
                          hipStream_t stream) {
  if (rx_form(cfg, K, epi)) {
    switch (K / 1024u) {
      case 1: return launch_cfg<kEpiNone, 8, 1, false, 1>(cfg, t, K, gs, x_or_gate, nullptr, nullptr, stream);
      case 2: return launch_cfg<kEpiNone, 8, 1, false, 2>(cfg, t, K, gs, x_or_gate, nullptr, nullptr, stream);
      case 3: return launch_cfg<kEpiNone, 8, 1, false, 3>(cfg, t, K, gs, x_or_gate, nullptr, nullptr, stream);
      default: return launch_cfg<kEpiNone, 8, 1, false, 4>(cfg, t, K, gs, x_or_gate, nullptr, nullptr, stream);
    }
  }
  if (cfg.tail) {
    switch (epi) {
      case kEpiNone: return launch_shape<kEpiNone, true>(cfg, t, K, gs, x_or_gate, nullptr, nullptr, stream);
      case kEpiSiluGate: return launch_shape<kEpiSiluGate, true>(cfg, t, K, gs, x_or_gate, up, nullptr, stream);
      default: return launch_shape<kEpiSiluGateResid, true>(cfg, t, K, gs, x_or_gate, up, x_resid, stream);
    }
  }
  switch (epi) {
    case kEpiNone: return launch_shape<kEpiNone, false>(cfg, t, K, gs, x_or_gate, nullptr, nullptr, stream);
    case kEpiSiluGate: return launch_shape<kEpiSiluGate, false>(cfg, t, K, gs, x_or_gate, up, nullptr, stream);
    default: return launch_shape<kEpiSiluGateResid, false>(cfg, t, K, gs, x_or_gate, up, x_resid, stream);
  }
}

GemvTargets make_targets(const WeightView *w, uint16_t *const *y, uint32_t count) {
  GemvTargets t{};
  for (uint32_t i = 0; i < kMaxTargets; ++i) {
    const uint32_t s = i < count ? i : 0u;  // unused slots repeat the first weight
    t.codes[i] = reinterpret_cast<const uint8_t *>(w[s].packed);
    t.scales[i] = w[s].scales;
    t.biases[i] = w[s].biases;
    t.y[i] = y[s];
    t.n[i] = w[s].N;
  }
  t.count = count;
  return t;
}

// One launch over `count` weights with the same K and group size.
hipError_t launch_gemv_list(const WeightView *w, uint16_t *const *y, uint32_t count, GemvEpilogue epi,
                            const uint16_t *x_or_gate, const uint16_t *up, const uint16_t *x_resid,
                            hipStream_t stream) {
  GemvTargets t = make_targets(w, y, count);
  const GemvCfg cfg = choose_cfg(t.n, count, w[0].K, w[0].gs, t.wave_end);
  return launch_targets(cfg, t, w[0].K, w[0].gs, epi, x_or_gate, up, x_resid, stream);
}

template <int W, int RP, bool TAIL, int NS = 0, bool SBI = false>
hipError_t launch_moe_cfg(const GemvCfg &cfg, const WeightView &w, uint32_t E, const uint16_t *x, uint32_t x_rows,
                          const uint32_t *ids, uint32_t topk, uint32_t slots, uint16_t *y, hipStream_t stream) {
  static bool configured = false;
  auto kern = k_moe_gemv<NS, W, RP, kLoadsPerBlock / RP, TAIL, SBI>;
  hipError_t e = raise_lds_cap(kern, configured);
  if (e != hipSuccess) return e;
  const uint32_t gs_log2 = (uint32_t)__builtin_ctz(w.gs);
  const size_t lds = NS ? 0u : lds_bytes(cfg, w.gs);
  hipLaunchKernelGGL(kern, dim3(cfg.blocks), dim3(64 * W), lds, stream, reinterpret_cast<const uint8_t *>(w.packed),
                     w.scales, w.biases, x, ids, y, w.N / E, E, topk, x_rows, slots, w.K, gs_log2, cfg.ct,
                     cfg.max_rows);
  return hipGetLastError();
}

// Launch shape of the expert-indexed gemv: every slot gets the same number
// of workgroups (the gemv's wave shape), enough for all slots together to
// fill the GPU and for no wave to own more than kMaxRowsPerWave rows.
GemvCfg choose_moe_cfg(uint32_t N, uint32_t K, uint32_t gs, uint32_t slots) {
  const uint32_t cus = (uint32_t)device_cu_count();
  GemvCfg c{};
  c.waves = K <= 8192u ? 8 : 16;
  const uint32_t per_cu = c.waves == 8 && (uint64_t)N * slots > 16384u ? 2u : 1u;  // as choose_cfg
  const uint32_t W = (uint32_t)c.waves;
  uint32_t per_slot = (per_cu * cus + slots - 1) / slots;
  const uint32_t most = (N + W - 1) / W;                                  // no more waves than rows
  const uint32_t least = (N + W * kMaxRowsPerWave - 1) / (W * kMaxRowsPerWave);
  if (per_slot > most) per_slot = most;
  if (per_slot < least) per_slot = least;
  const uint32_t tw = per_slot * W;
  c.blocks = per_slot * slots;
  c.max_rows = (N + tw - 1) / tw;
  c.rp = c.waves == 16 && N / tw >= 2u ? 2 : 1;
  pick_tile(c, K, gs, kLdsPerCu / per_cu);
  return c;
}

}  // namespace

hipError_t launch_gemv(const WeightView &w, GemvEpilogue epi, const uint16_t *x_or_gate,
                       const uint16_t *up, const uint16_t *x_resid, uint16_t *y,
                       hipStream_t stream) {
  return launch_gemv_list(&w, &y, 1, epi, x_or_gate, up, x_resid, stream);
}

bool gemv_rows_supported(uint32_t K, uint32_t m) {
  return m >= 2u && m <= 4u && K % 1024u == 0 && K >= 1024u && K <= 4096u;
}

namespace {

template <int NS, int MR>
void launch_rows_cfg(const WeightView &w, const uint16_t *X, uint16_t *Y, uint32_t blocks, hipStream_t stream) {
  hipLaunchKernelGGL((k_gemv_rows<NS, MR>), dim3(blocks), dim3(512), 0, stream,
                     reinterpret_cast<const uint8_t *>(w.packed), w.scales, w.biases, X, Y, w.N,
                     (uint32_t)__builtin_ctz(w.gs));
}

template <int MR>
void launch_rows_ns(const WeightView &w, const uint16_t *X, uint16_t *Y, uint32_t blocks, hipStream_t stream) {
  switch (w.K / 1024u) {
    case 1: launch_rows_cfg<1, MR>(w, X, Y, blocks, stream); break;
    case 2: launch_rows_cfg<2, MR>(w, X, Y, blocks, stream); break;
    case 3: launch_rows_cfg<3, MR>(w, X, Y, blocks, stream); break;
    default: launch_rows_cfg<4, MR>(w, X, Y, blocks, stream); break;
  }
}

}  // namespace

hipError_t launch_gemv_rows(const WeightView &w, const uint16_t *X, uint16_t *Y, uint32_t m, hipStream_t stream) {
  if (!gemv_rows_supported(w.K, m)) return hipErrorInvalidValue;
  uint32_t blocks = (uint32_t)device_cu_count();
  const uint32_t need = (w.N + 7u) / 8u;  // no workgroup without rows
  if (blocks > need) blocks = need;
  switch (m) {
    case 2: launch_rows_ns<2>(w, X, Y, blocks, stream); break;
    case 3: launch_rows_ns<3>(w, X, Y, blocks, stream); break;
    default: launch_rows_ns<4>(w, X, Y, blocks, stream); break;
  }
  return hipGetLastError();
}

// Measured against the small-m matrix-core kernel (graph-timed, rotated
// weights): m = 2 on 4096 x 14336 gs32 16.5 against 18.5 us, on 8192 x 28672
// gs128 45.3 against 53.3 us; but 4096 x 14336 gs64 m = 2 16.5 against 14.6
// us, and m = 3 or 4 slower on every shape tried (up to 20.6 against 14.7 us):
// the dot products of several rows cost more vector work per code than the
// stream hides.  So two rows, where the small-m kernel is weakest: group size
// 32 (a rescale every 32 codes) or rows longer than 16384.
bool gemv_rows_lds_supported(uint32_t K, uint32_t gs, uint32_t m) {
  return m == 2u && K > 4096u && K % 1024u == 0 && (uint64_t)m * K <= kRowsLdsMaxMK && (gs == 32u || K > 16384u);
}

namespace {

template <int MR>
hipError_t launch_rows_lds_cfg(const WeightView &w, const uint16_t *X, uint16_t *Y, hipStream_t stream) {
  static bool configured = false;
  auto kern = k_gemv_rows_lds<MR>;
  hipError_t e = raise_lds_cap(kern, configured);
  if (e != hipSuccess) return e;
  uint32_t blocks = (uint32_t)device_cu_count();
  const uint32_t need = (w.N + 15u) / 16u;  // no workgroup without rows
  if (blocks > need) blocks = need;
  const size_t lds = (size_t)MR * w.K * 2u + (size_t)MR * (w.K / 16u) * 4u;
  hipLaunchKernelGGL(kern, dim3(blocks), dim3(1024), lds, stream, reinterpret_cast<const uint8_t *>(w.packed),
                     w.scales, w.biases, X, Y, w.N, w.K, (uint32_t)__builtin_ctz(w.gs));
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemv_rows_lds(const WeightView &w, const uint16_t *X, uint16_t *Y, uint32_t m,
                                hipStream_t stream) {
  if (!gemv_rows_lds_supported(w.K, w.gs, m)) return hipErrorInvalidValue;
  return launch_rows_lds_cfg<2>(w, X, Y, stream);
}

hipError_t launch_gemv_multi(const WeightView *w, uint16_t *const *y, uint32_t count, const uint16_t *x,
                             hipStream_t stream) {
  return launch_gemv_list(w, y, count, kEpiNone, x, nullptr, nullptr, stream);
}

namespace {

template <int NS>
hipError_t launch_moe_grouped(const WeightView &w, uint32_t E, const uint16_t *x, uint32_t x_rows,
                              const uint32_t *ids, uint32_t topk, uint32_t slots, uint16_t *y, hipStream_t stream) {
  static bool configured = false;
  auto kern = k_moe_grouped<NS>;
  const size_t lds = (size_t)kGrpC * NS * (256u * 16u + 64u * 4u);
  // the kernel also holds a few KiB of static LDS: ask for the dynamic part only
  hipError_t e = raise_lds_cap(kern, configured, (int)lds);
  if (e != hipSuccess) return e;
  const uint32_t blocks = 2u * (uint32_t)device_cu_count();  // two 8-wave workgroups per CU
  hipLaunchKernelGGL(kern, dim3(blocks), dim3(512), lds, stream, reinterpret_cast<const uint8_t *>(w.packed),
                     w.scales, w.biases, x, ids, y, w.N / E, E, topk, x_rows, slots,
                     (uint32_t)__builtin_ctz(w.gs));
  return hipGetLastError();
}

}  // namespace

hipError_t launch_moe_gemv(const WeightView &w, uint32_t E, const uint16_t *x, uint32_t x_rows, const uint32_t *ids,
                           uint32_t tokens, uint32_t topk, uint16_t *y, hipStream_t stream) {
  const uint32_t slots = tokens * topk;
  // when the slots outnumber the experts, experts repeat: stream each named
  // expert once (measured: 8 experts, top-2, 4 tokens 77 -> 73 us, 8 tokens
  // 150 -> 112 us; at 2 tokens the per-slot form stays faster)
  if (tokens > 1u && slots >= E && slots <= kGrpMaxSlots && E <= kGrpMaxExperts && w.K % 1024u == 0 &&
      w.K >= 1024u && w.K <= 4096u) {
    switch (w.K / 1024u) {
      case 1: return launch_moe_grouped<1>(w, E, x, x_rows, ids, topk, slots, y, stream);
      case 2: return launch_moe_grouped<2>(w, E, x, x_rows, ids, topk, slots, y, stream);
      case 3: return launch_moe_grouped<3>(w, E, x, x_rows, ids, topk, slots, y, stream);
      default: return launch_moe_grouped<4>(w, E, x, x_rows, ids, topk, slots, y, stream);
    }
  }
  const GemvCfg cfg = choose_moe_cfg(w.N / E, w.K, w.gs, slots);
  if (rx_form(cfg, w.K, kEpiNone)) {
    switch (w.K / 1024u) {
      case 1: return launch_moe_cfg<8, 1, false, 1>(cfg, w, E, x, x_rows, ids, topk, slots, y, stream);
      case 2: return launch_moe_cfg<8, 1, false, 2>(cfg, w, E, x, x_rows, ids, topk, slots, y, stream);
      case 3: return launch_moe_cfg<8, 1, false, 3>(cfg, w, E, x, x_rows, ids, topk, slots, y, stream);
      default: return launch_moe_cfg<8, 1, false, 4>(cfg, w, E, x, x_rows, ids, topk, slots, y, stream);
    }
  }
  if (cfg.waves == 16) {
    if (cfg.sbi)
      return cfg.rp == 2 ? launch_moe_cfg<16, 2, false, 0, true>(cfg, w, E, x, x_rows, ids, topk, slots, y, stream)
                         : launch_moe_cfg<16, 1, false, 0, true>(cfg, w, E, x, x_rows, ids, topk, slots, y, stream);
    if (cfg.rp == 2)
      return cfg.tail ? launch_moe_cfg<16, 2, true>(cfg, w, E, x, x_rows, ids, topk, slots, y, stream)
                      : launch_moe_cfg<16, 2, false>(cfg, w, E, x, x_rows, ids, topk, slots, y, stream);
    return cfg.tail ? launch_moe_cfg<16, 1, true>(cfg, w, E, x, x_rows, ids, topk, slots, y, stream)
                    : launch_moe_cfg<16, 1, false>(cfg, w, E, x, x_rows, ids, topk, slots, y, stream);
  }
  return cfg.tail ? launch_moe_cfg<8, 1, true>(cfg, w, E, x, x_rows, ids, topk, slots, y, stream)
                  : launch_moe_cfg<8, 1, false>(cfg, w, E, x, x_rows, ids, topk, slots, y, stream);
}

}  // namespace int8w
