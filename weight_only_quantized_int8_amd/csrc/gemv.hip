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
//    the R rows).  Its loads run as a two-stage software pipeline of blocks of
//    U runs per row: block j+1 is in flight while block j is consumed, and the
//    first block is issued before the activation staging, so the staging hides
//    under the first HBM round trip.  Loads go through bounded buffer
//    resources, so the code is branch-free: past-the-end loads return zero
//    without touching memory.
//  * Waves of a workgroup may also split K (WK-way) for short, wide matrices;
//    partial sums meet in LDS.  Lane partials are summed with cross-lane
//    shuffles; there are no atomics, so results are deterministic.
//  * fp32 accumulation throughout; the residual is added in fp32 before the
//    one rounding to BF16.
#include "common.h"
#include "launch.h"

namespace int8w {

namespace {

constexpr int kGemvThreads = 512;          // 8 waves
constexpr int kWaves = kGemvThreads / 64;
constexpr uint32_t kTileRunsMax = 1024;    // 16384 activations per LDS tile
constexpr int kStagePerThread = kTileRunsMax / kGemvThreads;
constexpr int kU = 4;                      // 1 KiB wave loads per pipeline block
constexpr uint32_t kMaxRowsPerWave = 16;   // rows a wave may own
constexpr size_t kLdsBudget = 150 * 1024;  // dynamic LDS per workgroup
constexpr int kSbPerLane = 8;              // scale/bias elements a lane prefetches per tile

struct GemvCfg {
  uint32_t blocks;     // workgroups (8 waves each)
  uint32_t ct;         // 16-code runs per LDS tile (multiple of 64)
  uint32_t max_rows;   // most rows any wave owns
  bool tail;           // in_features not a multiple of 1024
};

size_t lds_bytes(const GemvCfg &c, uint32_t gs) {
  const size_t tg = (size_t)c.ct * 16u / gs;
  return (size_t)c.ct * 68u + (size_t)kWaves * 2u * c.max_rows * tg * 2u + (size_t)kWaves * c.max_rows * 4u;
}

template <int U>
struct Block {
  u32x4 q[U];
};

// f16 pair (1024 + q0, 1024 + q1) from bytes 0/1 (sel 0x04010400) or 2/3
// (sel 0x04030402) of a code word: byte 0x64 over each code is the binary16
// pattern of 1024 + q, exact for q in 0..255.
__device__ __forceinline__ uint32_t f16_pair(uint32_t word, uint32_t sel) {
  return __builtin_amdgcn_perm(0x64646464u, word, sel);
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

// LDS layout of one workgroup (dynamic):
//   act   [NSEG][4][64] float4   activation of the tile, run-interleaved
//   ssum  [NSEG][64]    float    per-run activation sums
//   sb    [kWaves][2][max_rows][tg_max] u16   each wave's scales / biases for the tile
//   part  [kWaves][max_rows] float            row partial sums across tiles
template <int EPI, int U, bool TAIL>
__global__ __launch_bounds__(kGemvThreads) void k_gemv(
    const uint8_t *__restrict__ codes, const uint16_t *__restrict__ scales,
    const uint16_t *__restrict__ biases, const uint16_t *__restrict__ xg,
    const uint16_t *__restrict__ up, const uint16_t *resid, uint16_t *y, uint32_t N, uint32_t K,
    uint32_t gs_log2, uint32_t tile_runs, uint32_t max_rows) {
  // y may be resid itself (in-place residual): each output element reads its
  // own residual before it is written, by the same lane.
  extern __shared__ float4 lds4[];
  const uint32_t CT = tile_runs;              // multiple of 64
  const uint32_t NSEG = CT >> 6;              // 1 KiB segments per tile row
  const uint32_t TG = (CT << 4) >> gs_log2;   // groups per tile row
  float4 *act = lds4;
  float *ssum = reinterpret_cast<float *>(lds4 + NSEG * 256);
  uint16_t *sb_all = reinterpret_cast<uint16_t *>(ssum + NSEG * 64);
  float *part_all = reinterpret_cast<float *>(sb_all + kWaves * 2 * max_rows * TG);

  const uint32_t tid = threadIdx.x;
  const uint32_t lane = tid & 63u;
  const uint32_t wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const uint32_t gw = blockIdx.x * kWaves + wave;
  const uint32_t TW = gridDim.x * kWaves;
  // this wave's rows: a balanced contiguous range
  const uint32_t rq = N / TW, rr = N % TW;  // the first rr waves own rq + 1 rows
  const uint32_t rbeg = gw * rq + (gw < rr ? gw : rr);
  const uint32_t nr = rq + (gw < rr ? 1u : 0u);
  const uint32_t cpr = K >> 4;      // 16-code runs per row
  const uint32_t G = K >> gs_log2;  // groups per row

  const auto rw = make_rsrc(codes + (size_t)rbeg * K, nr * K);
  const auto rx = make_rsrc(xg, K * 2u);
  const auto ru = make_rsrc(EPI != kEpiNone ? up : xg, K * 2u);
  const uint16_t *srow = scales + (size_t)rbeg * G;
  const uint16_t *brow = biases + (size_t)rbeg * G;

  uint16_t *sbs = sb_all + wave * 2 * max_rows * TG;  // this wave's scales; biases follow
  uint16_t *sbb = sbs + max_rows * TG;
  float *part = part_all + wave * max_rows;

  // per-lane parts of the offsets; everything else is wave-uniform
  const uint32_t vo_w = lane << 4;
  const uint32_t lane_grp = (lane << 4) >> gs_log2;  // group of this lane within a 1 KiB segment

  float acc = 0.f;
  Block<U> A, B;

  for (uint32_t t0 = 0; t0 < cpr; t0 += CT) {
    const uint32_t ct = (cpr - t0) < CT ? (cpr - t0) : CT;
    const bool last_tile = t0 + ct == cpr;
    const uint32_t nseg = (ct + 63u) >> 6;
    const uint32_t nitems = nr * nseg;
    const uint32_t nblk = (nitems + U - 1) / U;  // blocks of this wave in this tile
    const uint32_t tg = (ct << 4) >> gs_log2;    // groups of this tile
    const uint32_t g0 = (t0 << 4) >> gs_log2;    // first group of this tile
    const uint32_t last_lanes = ct - ((nseg - 1u) << 6);
    const uint32_t vo_w_last = TAIL && lane >= last_lanes ? kOutOfRange : vo_w;
    // lanes past the end of a partial last segment read a staged (finite)
    // scale/bias entry; their codes and activations are zero
    const uint32_t lane_grp_last = TAIL && lane >= last_lanes ? 0u : lane_grp;
    const uint32_t seg_bytes0 = t0 << 4;

    // item (row, seg) iterators, wave-uniform
    uint32_t i_row = 0, i_seg = 0;
    // Issue one block of U items.  Only the wave's final block can hold items
    // past its last row; those are marked out of range in the per-lane offset
    // (what the buffer bound is checked against), so the code stays
    // branch-free.  The wave-uniform part of each offset is the scalar offset.
    auto issue = [&](Block<U> &blk) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const bool live = i_row < nr;
        const uint32_t sw = live ? i_row * K + seg_bytes0 + (i_seg << 10) : 0u;
        const uint32_t dead = live ? 0u : kOutOfRange;
        const bool last = TAIL && i_seg == nseg - 1u;
        const uint32_t vw = (last ? vo_w_last : vo_w) | dead;
        blk.q[u] = __builtin_amdgcn_raw_buffer_load_b128(rw, (int)vw, (int)sw, kAuxNontemporal);
        if (++i_seg == nseg) { i_seg = 0; ++i_row; }
      }
    };
    uint32_t c_row = 0, c_seg = 0;
    auto consume = [&](const Block<U> &blk) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (c_row < nr) {
          const float4 *ap = act + (c_seg << 8) + lane;
          const float4 a0 = ap[0], a1 = ap[64], a2 = ap[128], a3 = ap[192];
          const float S = ssum[(c_seg << 6) + lane];
          const bool lastseg = TAIL && c_seg == nseg - 1u;
          const uint32_t gi = c_row * tg + ((c_seg << 10) >> gs_log2) + (lastseg ? lane_grp_last : lane_grp);
          const float sc = bf16_bits_to_f32(sbs[gi]);
          const float bi = __builtin_fmaf(-1024.f, sc, bf16_bits_to_f32(sbb[gi]));
          const u32x4 w = blk.q[u];
          // P' = sum (1024 + q) a over the lane's 16 codes (f16 codes, fp32 FMA)
          float p = 0.f;
          const uint32_t words[4] = {w.x, w.y, w.z, w.w};
          const float av[16] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w,
                                a2.x, a2.y, a2.z, a2.w, a3.x, a3.y, a3.z, a3.w};
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const f16x2 lo = __builtin_bit_cast(f16x2, f16_pair(words[i], 0x04010400u));
            const f16x2 hi = __builtin_bit_cast(f16x2, f16_pair(words[i], 0x04030402u));
            p = __builtin_fmaf((float)lo.x, av[4 * i + 0], p);
            p = __builtin_fmaf((float)lo.y, av[4 * i + 1], p);
            p = __builtin_fmaf((float)hi.x, av[4 * i + 2], p);
            p = __builtin_fmaf((float)hi.y, av[4 * i + 3], p);
          }
          // sum (q s + b) a = s P' + (b - 1024 s) S
          acc = __builtin_fmaf(sc, p, __builtin_fmaf(bi, S, acc));
          if (c_seg == nseg - 1u) {  // this row's part of the tile is done
            const float tot = wave_sum_lane63(acc);
            if (lane == 63u) {
              float v = t0 ? part[c_row] + tot : tot;
              if (last_tile) {
                if constexpr (EPI == kEpiSiluGateResid) v += bf16_bits_to_f32(resid[rbeg + c_row]);
                y[rbeg + c_row] = to_bf16_bits(v);
              } else {
                part[c_row] = v;
              }
            }
            acc = 0.f;
          }
        }
        if (++c_seg == nseg) { c_seg = 0; ++c_row; }
      }
    };

    // 1. activation loads for this tile, this wave's scales and biases for
    //    the tile, then the first weight block: all in flight together
    u32x4 xv[kStagePerThread][2], uv[kStagePerThread][2];
#pragma unroll
    for (int s = 0; s < kStagePerThread; ++s) {
      const uint32_t e = tid + s * kGemvThreads;
      const uint32_t off = e < ct ? (t0 + e) * 32u : kOutOfRange;
      xv[s][0] = buf_load_b128(rx, off);
      xv[s][1] = buf_load_b128(rx, off + 16u);
      if constexpr (EPI != kEpiNone) {
        uv[s][0] = buf_load_b128(ru, off);
        uv[s][1] = buf_load_b128(ru, off + 16u);
      }
    }
    if (nblk) issue(A);
    // this wave's scales and biases for the tile: element e = (row, group)
    // of the nr x tg slice, loaded up front (kSbPerLane per lane at a time)
    const uint32_t nsb = nr * tg;
    uint16_t sv[kSbPerLane], bv[kSbPerLane];
#pragma unroll
    for (int j = 0; j < kSbPerLane; ++j) {
      const uint32_t e = lane + 64u * j;
      const uint32_t r = e / tg, g = e - r * tg;
      const uint32_t src = e < nsb ? r * G + g0 + g : 0u;
      sv[j] = srow[src];
      bv[j] = brow[src];
    }
    if (t0) __syncthreads();  // everyone is done with the previous tile's activation
    // 2. form the activation tile: [seg][4][64] float4 plus per-run sums;
    //    runs past the end are written as zeros
#pragma unroll
    for (int s = 0; s < kStagePerThread; ++s) {
      const uint32_t e = tid + s * kGemvThreads;
      if (e < (nseg << 6)) {
        const uint32_t wv[8] = {xv[s][0].x, xv[s][0].y, xv[s][0].z, xv[s][0].w,
                                xv[s][1].x, xv[s][1].y, xv[s][1].z, xv[s][1].w};
        float a[16];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          a[2 * i] = bf16_lo(wv[i]);
          a[2 * i + 1] = bf16_hi(wv[i]);
        }
        if constexpr (EPI != kEpiNone) {
          const uint32_t uw[8] = {uv[s][0].x, uv[s][0].y, uv[s][0].z, uv[s][0].w,
                                  uv[s][1].x, uv[s][1].y, uv[s][1].z, uv[s][1].w};
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            a[2 * i] = silu_mul(a[2 * i], bf16_lo(uw[i]));
            a[2 * i + 1] = silu_mul(a[2 * i + 1], bf16_hi(uw[i]));
          }
        }
        float sum = 0.f;
#pragma unroll
        for (int i = 0; i < 16; ++i) sum += a[i];
        float4 *dst = act + ((e >> 6) << 8) + (e & 63u);
#pragma unroll
        for (int f = 0; f < 4; ++f) dst[f * 64] = make_float4(a[4 * f], a[4 * f + 1], a[4 * f + 2], a[4 * f + 3]);
        ssum[e] = sum;
      }
    }
    __syncthreads();
    // this wave's private scale/bias slice (no barrier needed: only this wave
    // reads it, after writing it, and its previous tile is consumed)
#pragma unroll
    for (int j = 0; j < kSbPerLane; ++j) {
      const uint32_t e = lane + 64u * j;
      if (e < nsb) {
        sbs[e] = sv[j];
        sbb[e] = bv[j];
      }
    }
    for (uint32_t e = lane + 64u * kSbPerLane; e < nsb; e += 64u) {  // slices beyond kSbPerLane*64
      const uint32_t r = e / tg, g = e - r * tg;
      sbs[e] = srow[r * G + g0 + g];
      sbb[e] = brow[r * G + g0 + g];
    }
    // 3. two-stage pipeline: the next block is issued before the current one
    //    is consumed; the only branches are the loop exits, so every issued
    //    block is a live one
    for (uint32_t b = 0; b < nblk;) {
      if (b + 1 >= nblk) { consume(A); break; }
      issue(B);
      consume(A);
      ++b;
      if (b + 1 >= nblk) { consume(B); break; }
      issue(A);
      consume(B);
      ++b;
    }
  }
}

template <int EPI, bool TAIL>
hipError_t launch_cfg(const GemvCfg &cfg, hipStream_t stream, const WeightView &w, const uint16_t *xg,
                      const uint16_t *up, const uint16_t *resid, uint16_t *y) {
  auto kern = k_gemv<EPI, kU, TAIL>;
  static bool configured = false;  // raise the dynamic-LDS cap once per instantiation
  if (!configured) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
    if (e != hipSuccess) return e;
    configured = true;
  }
  const size_t lds = lds_bytes(cfg, w.gs);
  hipLaunchKernelGGL(kern, dim3(cfg.blocks), dim3(kGemvThreads), lds, stream,
                     reinterpret_cast<const uint8_t *>(w.packed), w.scales, w.biases, xg, up, resid, y, w.N,
                     w.K, (uint32_t)__builtin_ctz(w.gs), cfg.ct, cfg.max_rows);
  return hipGetLastError();
}

GemvCfg choose_cfg(uint32_t N, uint32_t K, uint32_t gs, uint32_t blocks_override = 0) {
  const uint32_t cus = (uint32_t)device_cu_count();
  GemvCfg c{};
  // One workgroup of 8 waves per CU; every wave streams a contiguous range of rows.
  c.blocks = blocks_override ? blocks_override : cus;
  const uint32_t need = (N + kWaves - 1) / kWaves;
  if (c.blocks > need) c.blocks = need;
  const uint32_t enough = (N + kWaves * kMaxRowsPerWave - 1) / (kWaves * kMaxRowsPerWave);
  if (c.blocks < enough) c.blocks = enough;  // at most kMaxRowsPerWave rows per wave
  const uint32_t tw = c.blocks * kWaves;
  c.max_rows = (N + tw - 1) / tw;
  const uint32_t cpr = K / 16u;
  // Tile K so that the activation tile and the waves' scale/bias slices fit.
  for (uint32_t ntiles = (cpr + kTileRunsMax - 1) / kTileRunsMax;; ++ntiles) {
    c.ct = ((cpr + ntiles - 1) / ntiles + 63u) / 64u * 64u;
    if (lds_bytes(c, gs) <= kLdsBudget || c.ct == 64u) break;
  }
  c.tail = (cpr % 64u) != 0;
  return c;
}

hipError_t launch_gemv_with(const GemvCfg &cfg, const WeightView &w, GemvEpilogue epi, const uint16_t *x_or_gate,
                            const uint16_t *up, const uint16_t *x_resid, uint16_t *y, hipStream_t stream) {
  if (cfg.tail) {
    switch (epi) {
      case kEpiNone: return launch_cfg<kEpiNone, true>(cfg, stream, w, x_or_gate, nullptr, nullptr, y);
      case kEpiSiluGate: return launch_cfg<kEpiSiluGate, true>(cfg, stream, w, x_or_gate, up, nullptr, y);
      default: return launch_cfg<kEpiSiluGateResid, true>(cfg, stream, w, x_or_gate, up, x_resid, y);
    }
  }
  switch (epi) {
    case kEpiNone: return launch_cfg<kEpiNone, false>(cfg, stream, w, x_or_gate, nullptr, nullptr, y);
    case kEpiSiluGate: return launch_cfg<kEpiSiluGate, false>(cfg, stream, w, x_or_gate, up, nullptr, y);
    default: return launch_cfg<kEpiSiluGateResid, false>(cfg, stream, w, x_or_gate, up, x_resid, y);
  }
}

}  // namespace

hipError_t launch_gemv(const WeightView &w, GemvEpilogue epi, const uint16_t *x_or_gate,
                       const uint16_t *up, const uint16_t *x_resid, uint16_t *y,
                       hipStream_t stream) {
  return launch_gemv_with(choose_cfg(w.N, w.K, w.gs), w, epi, x_or_gate, up, x_resid, y, stream);
}

}  // namespace int8w
