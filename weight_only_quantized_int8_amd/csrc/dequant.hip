// dequant.hip -- dequantize_to for gfx950: the full BF16 weight from the
// packed codes (rustdoc page "MlxInt8Weight", method dequantize_to).
//
//   out[n, k] = RNE_bf16(q[n,k] * scale + bias), row-major [N, K].
//
// HBM-bound streaming kernel.  Algorithmic traffic per weight: 1 + 4/gs
// bytes read, 2 bytes written.
//  * Each row is cut into 1 KiB segments (64 runs of 16 codes, one run per
//    lane); the (row, segment) items of the whole matrix are split evenly over
//    all waves, each wave streaming a contiguous stretch.
//  * Loads go through bounded buffer resources with the wave-uniform offset in
//    a scalar register; two blocks of U items are in flight.  A run never
//    straddles a group (gs is a multiple of 16), so each lane needs one
//    (scale, bias) pair per run.  Lanes past the end of a row's last, partial
//    segment load and store nothing.
//  * Output goes out as two 16-byte stores per lane with the default cache
//    policy, eight 8-wave workgroups per CU.  Measured on 28672 x 8192 gs128
//    (graph-timed): 153 us at eight per CU, 156 at four, 157 at two;
//    non-temporal stores (flat or buffer) 2-6 % slower at two and four, equal
//    at eight.  That is 99 % of the rate of the plain streaming expand of
//    measure.hip (one byte read, two written per element, no arithmetic).
//  * The fp32 value q*s + b is one fused multiply-add; q*s is exact in fp32
//    (8-bit by 8-bit significands), so this equals the separately rounded
//    product-then-sum.  Rounding to BF16 is the hardware nearest-even convert.
#include "common.h"
#include "launch.h"

namespace int8w {

namespace {

constexpr int kDqThreads = 512;  // 8 waves
constexpr int kDqWaves = kDqThreads / 64;
constexpr int kDqU = 4;          // items per pipeline block

__device__ __forceinline__ uint32_t uniform_u32(uint32_t v) { return __builtin_amdgcn_readfirstlane(v); }

template <int U>
struct DqBlock {
  u32x4 q[U];
  uint16_t s[U], b[U];
};

template <int U>
__global__ __launch_bounds__(kDqThreads) void k_dequant(const uint8_t *__restrict__ codes,
                                                        const uint16_t *__restrict__ scales,
                                                        const uint16_t *__restrict__ biases,
                                                        uint16_t *__restrict__ out, uint32_t N, uint32_t K,
                                                        uint32_t gs_log2) {
  const uint32_t lane = threadIdx.x & 63u;
  const uint32_t gw = blockIdx.x * kDqWaves + uniform_u32(threadIdx.x >> 6);
  const uint32_t TW = gridDim.x * kDqWaves;
  const uint32_t rpr = K >> 4;                // runs per row
  const uint32_t nseg = (rpr + 63u) >> 6;     // segments per row
  const uint32_t G = K >> gs_log2;
  const uint32_t gps = 1024u >> gs_log2;      // groups per segment
  const uint32_t items = N * nseg;
  const uint32_t iq = items / TW, ir = items % TW;
  const uint32_t ibeg = gw * iq + (gw < ir ? gw : ir);
  const uint32_t nit = iq + (gw < ir ? 1u : 0u);
  const uint32_t last_lanes = rpr - ((nseg - 1u) << 6);

  // issue and consume iterators over (row, segment), wave-uniform
  const uint32_t row0 = nit ? ibeg / nseg : 0u;
  const uint32_t seg0 = nit ? ibeg - row0 * nseg : 0u;
  const uint32_t row_end = nit ? (ibeg + nit - 1u) / nseg + 1u : row0;  // past this wave's last row
  // bounded views of this wave's rows (offsets are relative to row0 and
  // stay far below 2^31, where the out-of-range marker lives)
  const auto rc = make_rsrc(codes + (size_t)row0 * K, (row_end - row0) * K);
  const auto rs = make_rsrc(scales + (size_t)row0 * G, (row_end - row0) * G * 2u);
  const auto rb = make_rsrc(biases + (size_t)row0 * G, (row_end - row0) * G * 2u);
  const uint32_t vo_w = lane << 4;
  const uint32_t vo_s = ((lane << 4) >> gs_log2) << 1;
  const uint32_t vo_w_last = lane < last_lanes ? vo_w : kOutOfRange;
  const uint32_t vo_s_last = lane < last_lanes ? vo_s : kOutOfRange;

  uint32_t i_row = 0, i_seg = seg0, i_left = nit;  // rows relative to row0
  uint32_t c_row = row0, c_seg = seg0, c_left = nit;

  auto issue = [&](DqBlock<U> &blk) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const bool live = i_left != 0;
      const bool last = i_seg == nseg - 1u;
      const uint32_t vw = live ? (last ? vo_w_last : vo_w) : kOutOfRange;
      const uint32_t vs = live ? (last ? vo_s_last : vo_s) : kOutOfRange;
      const uint32_t sw = uniform_u32(live ? i_row * K + (i_seg << 10) : 0u);
      const uint32_t ss = uniform_u32(live ? (i_row * G + i_seg * gps) << 1 : 0u);
      blk.q[u] = __builtin_amdgcn_raw_buffer_load_b128(rc, (int)vw, (int)sw, kAuxNontemporal);
      blk.s[u] = __builtin_amdgcn_raw_buffer_load_b16(rs, (int)vs, (int)ss, 0);
      blk.b[u] = __builtin_amdgcn_raw_buffer_load_b16(rb, (int)vs, (int)ss, 0);
      i_left -= live ? 1u : 0u;
      if (++i_seg == nseg) { i_seg = 0; ++i_row; }
    }
  };
  auto consume = [&](const DqBlock<U> &blk) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (c_left) {
        const bool ok = c_seg != nseg - 1u || lane < last_lanes;
        if (ok) {
          const float s = bf16_bits_to_f32(blk.s[u]), b = bf16_bits_to_f32(blk.b[u]);
          const u32x4 q = blk.q[u];
          const uint32_t w[4] = {q.x, q.y, q.z, q.w};
          uint32_t o[8];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            o[2 * i] = pack_bf16x2(__builtin_fmaf(code_f32(w[i], 0), s, b), __builtin_fmaf(code_f32(w[i], 1), s, b));
            o[2 * i + 1] =
                pack_bf16x2(__builtin_fmaf(code_f32(w[i], 2), s, b), __builtin_fmaf(code_f32(w[i], 3), s, b));
          }
          uint4 *dst = reinterpret_cast<uint4 *>(out + (size_t)c_row * K + (c_seg << 10)) + 2u * lane;
          dst[0] = make_uint4(o[0], o[1], o[2], o[3]);
          dst[1] = make_uint4(o[4], o[5], o[6], o[7]);
        }
        --c_left;
        if (++c_seg == nseg) { c_seg = 0; ++c_row; }
      }
    }
  };

  DqBlock<U> A, B;
  const uint32_t nblk = (nit + U - 1) / U;
  if (nblk) issue(A);
  // two blocks per iteration and the rest after the loop: a single exit,
  // so that the compiler's wait counts at the loop head do not also cover
  // the paths that leave (with them it waited for the block just issued)
  uint32_t b = 0;
  for (; b + 2u < nblk; b += 2u) {
    issue(B);
    consume(A);
    issue(A);
    consume(B);
  }
  if (b + 1u < nblk) {
    issue(B);
    consume(A);
    consume(B);
  } else if (b < nblk) {
    consume(A);
  }
}

}  // namespace

hipError_t launch_dequant(const WeightView &w, uint16_t *out, hipStream_t stream) {
  const uint32_t nseg = (w.K / 16u + 63u) / 64u;
  const uint32_t items = w.N * nseg;
  uint32_t blocks = 8u * (uint32_t)device_cu_count();  // eight 8-wave workgroups per CU
  const uint32_t need = (items + kDqWaves - 1) / kDqWaves;
  if (blocks > need) blocks = need;
  if (blocks == 0) blocks = 1;
  hipLaunchKernelGGL(k_dequant<kDqU>, dim3(blocks), dim3(kDqThreads), 0, stream,
                     reinterpret_cast<const uint8_t *>(w.packed), w.scales, w.biases, out, w.N, w.K,
                     (uint32_t)__builtin_ctz(w.gs));
  return hipGetLastError();
}

}  // namespace int8w
