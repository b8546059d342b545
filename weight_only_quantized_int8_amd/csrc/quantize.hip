// quantize.hip -- BF16 weight -> 8-bit affine codes, scales and biases for
// gfx950 (rustdoc page of the DynQuantizedStorage trait, method quantize; the
// target layout is the MlxInt8Weight page's packed / scales / biases fields).
//
// The pages give no formula; this is the plain affine min/max reading, in
// fp32, one operation at a time (the CPU oracle takes the same steps, so the
// codes agree bit for bit):
//   per group of gs consecutive values v of a row:
//     lo = min v, hi = max v                    (a zero extreme, -0 or +0, is +0)
//     s  = RNE_bf16((hi - lo) / 255)            (fp32 subtraction, IEEE division)
//     b  = lo                                   (a BF16 value already)
//     q  = clamp(rint((v - b) / s), 0, 255)     (IEEE division, ties to even)
//   and q = 0 for a group whose s is zero.  Inputs must be finite.
//
// HBM-bound streaming kernel: 2 bytes read and 1 + 4/gs bytes written per
// value.  The matrix is a flat run of 16-byte chunks (8 values); a group is
// gs/8 consecutive chunks and never crosses a row (gs divides K), so a wave
// handles 64 consecutive chunks (1 KiB) per item and its lanes meet per group
// with cross-lane min/max.  Waves stream contiguous, balanced item ranges
// through bounded buffer resources, two blocks of items in flight.
#include "common.h"
#include "launch.h"

namespace int8w {

namespace {

constexpr int kQThreads = 512;  // 8 waves
constexpr int kQWaves = kQThreads / 64;
constexpr int kQU = 4;          // items per pipeline block

__device__ __forceinline__ uint32_t uniform_q(uint32_t v) { return __builtin_amdgcn_readfirstlane(v); }

// (hi - lo) / 255 correctly rounded without the division sequence: the
// product with RN(1/255), then one FMA correction from the exact residual.
// Equal to the IEEE quotient for every non-negative finite fp32 (denormals
// included, which these kernels keep), checked exhaustively on the host by
// tests/test_div255.py.
__device__ __forceinline__ float div255(float x) {
  constexpr float r = 1.0f / 255.0f;
  const float q0 = x * r;
  const float e = __builtin_fmaf(-q0, 255.0f, x);
  return __builtin_fmaf(e, r, q0);
}

// one code, in the order of the definition above
__device__ __forceinline__ uint32_t quant_code(float v, float b, float s) {
  if (s == 0.0f) return 0u;
  const float t = __fdiv_rn(v - b, s);
  float r = __builtin_rintf(t);
  r = r < 0.0f ? 0.0f : r;
  r = r > 255.0f ? 255.0f : r;
  return (uint32_t)r;
}

// The same eight codes without a division per code.  The quotient only
// matters through rint, whose decision points are the half-integers, so
// t = (v - b) * rcp(s) serves where it is clearly on one side of one: rcp is
// within 1 ulp and the product within half an ulp, so for quotients below 256
// t is within 2^-14 of the correctly rounded quotient, and a t farther than
// 2^-13 from every half-integer gives the same code.  near[i] is set for the
// codes that need the IEEE division (t near a half-integer, or not finite);
// as booleans they stay lane masks in scalar registers.  v - b >= 0 (b is
// the group's minimum), so codes are only clamped at 255: v_cvt_pk_u8_f32
// saturates to 0..255 (measured on gfx950: 256, 300 and +inf give 255;
// it rounds to nearest even, so on the integer-valued r it is exact), which
// is the clamp.  A NaN quotient (only with s == 0) gives 0, and those codes
// are zeroed by the caller anyway.
__device__ __forceinline__ void quant_codes_fast(const float (&f)[8], float b, float s, uint32_t &q0, uint32_t &q1,
                                                 bool (&near)[8]) {
  const float rs = __builtin_amdgcn_rcpf(s);
  const bool live = s != 0.0f;
  uint32_t w[2] = {0u, 0u};
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float t = (f[i] - b) * rs;
    const float r = __builtin_rintf(t);
    near[i] = live && !(__builtin_fabsf(t - r) < 0.5f - 0x1p-13f);
    w[i >> 2] = __builtin_amdgcn_cvt_pk_u8_f32(r, i & 3, w[i >> 2]);
  }
  q0 = w[0];
  q1 = w[1];
}

// Cross-lane min / max over the LPG lanes of a group (aligned runs of 4, 8 or
// 16 lanes) by row-local DPP moves: swap neighbours, swap pairs, then mirror
// the half row and the row.  Each step combines two disjoint halves of the
// lanes seen so far, so every lane ends with the group's extreme; min and max
// do not depend on the order.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xf, 0xf, false));
}
template <int LPG>
__device__ __forceinline__ void group_min_max(float &lo, float &hi) {
  lo = fminf(lo, dpp_mov<0xB1>(lo));  // quad_perm [1,0,3,2]
  hi = fmaxf(hi, dpp_mov<0xB1>(hi));
  lo = fminf(lo, dpp_mov<0x4E>(lo));  // quad_perm [2,3,0,1]
  hi = fmaxf(hi, dpp_mov<0x4E>(hi));
  if constexpr (LPG >= 8) {
    lo = fminf(lo, dpp_mov<0x141>(lo));  // row_half_mirror
    hi = fmaxf(hi, dpp_mov<0x141>(hi));
  }
  if constexpr (LPG >= 16) {
    lo = fminf(lo, dpp_mov<0x140>(lo));  // row_mirror
    hi = fmaxf(hi, dpp_mov<0x140>(hi));
  }
}

template <int U>
struct QBlock {
  u32x4 v[U];
};

// LPG = lanes per group = gs / 8
template <int U, int LPG>
__global__ __launch_bounds__(kQThreads) void k_quantize(const uint16_t *__restrict__ w, uint8_t *__restrict__ codes,
                                                        uint16_t *__restrict__ scales, uint16_t *__restrict__ biases,
                                                        uint64_t chunks) {
  const uint32_t lane = threadIdx.x & 63u;
  const uint64_t gw = (uint64_t)blockIdx.x * kQWaves + uniform_q(threadIdx.x >> 6);
  const uint64_t TW = (uint64_t)gridDim.x * kQWaves;
  const uint64_t items = (chunks + 63u) >> 6;
  const uint64_t iq = items / TW, ir = items % TW;
  const uint64_t ibeg = gw * iq + (gw < ir ? gw : ir);
  const uint32_t nit = (uint32_t)(iq + (gw < ir ? 1u : 0u));

  // this wave's window of the input: items [ibeg, ibeg + nit), 1 KiB each
  const uint64_t c0 = ibeg << 6;  // first chunk
  const uint64_t cend = (ibeg + nit) << 6 < chunks ? (ibeg + nit) << 6 : chunks;
  const auto rw = make_rsrc(w + (c0 << 3), (uint32_t)((cend > c0 ? cend - c0 : 0u) << 4));
  const uint32_t vo = lane << 4;
  // the same window of the codes (8 bytes per chunk): stores past it are dropped
  const auto rc = make_rsrc(codes + (c0 << 3), (uint32_t)((cend > c0 ? cend - c0 : 0u) << 3));

  uint32_t i_item = 0, i_left = nit;
  auto issue = [&](QBlock<U> &blk) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const bool live = i_left != 0u;
      const uint32_t so = uniform_q(live ? i_item << 10 : 0u);
      blk.v[u] = __builtin_amdgcn_raw_buffer_load_b128(rw, (int)(live ? vo : kOutOfRange), (int)so, kAuxNontemporal);
      i_left -= live ? 1u : 0u;
      ++i_item;
    }
  };
  uint32_t c_item = 0, c_left = nit;
  auto consume = [&](const QBlock<U> &blk) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (c_left) {
        const uint64_t c = c0 + ((uint64_t)c_item << 6) + lane;  // this lane's chunk
        const bool mine = c < chunks;
        const uint32_t wv[4] = {blk.v[u].x, blk.v[u].y, blk.v[u].z, blk.v[u].w};
        float f[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          f[2 * i] = bf16_lo(wv[i]);
          f[2 * i + 1] = bf16_hi(wv[i]);
        }
        float lo = f[0], hi = f[0];
#pragma unroll
        for (int i = 1; i < 8; ++i) {
          lo = fminf(lo, f[i]);
          hi = fmaxf(hi, f[i]);
        }
        // lanes past the end hold zeros; they sit in their own (unwritten)
        // groups, since chunks is a whole number of groups
        group_min_max<LPG>(lo, hi);
        // A zero extreme is +0: the cross-lane min/max do not follow element
        // order, so which signed zero survives is arbitrary; normalising both
        // makes an all-zero group's scale and bias +0 whatever the order.
        if (lo == 0.0f) lo = 0.0f;
        if (hi == 0.0f) hi = 0.0f;
        const float sf = div255(hi - lo);
        const uint16_t s_bits = to_bf16_bits(sf);
        const uint16_t b_bits = to_bf16_bits(lo);  // exact
        const float s = bf16_bits_to_f32(s_bits), b = bf16_bits_to_f32(b_bits);
        uint32_t q0, q1;
        bool near[8];
        quant_codes_fast(f, b, s, q0, q1, near);
        if (s == 0.0f) q0 = q1 = 0u;
        // The IEEE division, per code position, only where some lane of the
        // wave needs it there (each test is wave-uniform; usually none does,
        // and when one does it is usually one position of one lane).
        if (__builtin_amdgcn_ballot_w64(near[0] || near[1] || near[2] || near[3] || near[4] || near[5] ||
                                        near[6] || near[7]) != 0u) {
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const bool here = near[i];
            if (__builtin_amdgcn_ballot_w64(here) != 0u) {
              if (here) {
                const uint32_t c = quant_code(f[i], b, s) << (8 * (i & 3));
                const uint32_t keep = ~(0xFFu << (8 * (i & 3)));
                if (i < 4)
                  q0 = (q0 & keep) | c;
                else
                  q1 = (q1 & keep) | c;
              }
            }
          }
        }
        // the item's 512 bytes of codes: one non-temporal buffer store
        __builtin_amdgcn_raw_buffer_store_b64(u32x2{q0, q1}, rc, (int)(mine ? lane << 3 : kOutOfRange),
                                              (int)uniform_q(c_item << 9), kAuxNontemporal);
        if (mine) {
          if ((lane & (LPG - 1)) == 0u) {
            const uint64_t grp = c / LPG;
            scales[grp] = s_bits;
            biases[grp] = b_bits;
          }
        }
        --c_left;
        ++c_item;
      }
    }
  };

  QBlock<U> A, B;
  const uint32_t nblk = (nit + U - 1) / U;
  if (nblk) issue(A);
  // two blocks per iteration and the rest after the loop: a single exit,
  // so that the compiler's wait counts at the loop head do not also cover
  // the paths that leave (with them it waited for the block just issued)
  uint32_t bl = 0;
  for (; bl + 2u < nblk; bl += 2u) {
    issue(B);
    consume(A);
    issue(A);
    consume(B);
  }
  if (bl + 1u < nblk) {
    issue(B);
    consume(A);
    consume(B);
  } else if (bl < nblk) {
    consume(A);
  }
}

template <int LPG>
hipError_t launch_lpg(const uint16_t *w, uint64_t chunks, uint32_t *packed, uint16_t *scales, uint16_t *biases,
                      hipStream_t stream) {
  const uint64_t items = (chunks + 63u) / 64u;
  // eight 8-wave workgroups per CU and non-temporal code stores: 14336 x 4096
  // gs64 in 43.1 us against 45.1 with four per CU and default stores, 48.3
  // with two (graph-timed); two or eight loads per block were no better
  uint64_t blocks = 8u * (uint64_t)device_cu_count();
  const uint64_t need = (items + kQWaves - 1) / kQWaves;
  if (blocks > need) blocks = need;
  if (blocks == 0) blocks = 1;
  hipLaunchKernelGGL((k_quantize<kQU, LPG>), dim3((uint32_t)blocks), dim3(kQThreads), 0, stream, w,
                     reinterpret_cast<uint8_t *>(packed), scales, biases, chunks);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_quantize(const uint16_t *w, uint32_t N, uint32_t K, uint32_t gs, uint32_t *packed, uint16_t *scales,
                           uint16_t *biases, hipStream_t stream) {
  const uint64_t chunks = (uint64_t)N * K / 8u;
  switch (gs) {
    case 32: return launch_lpg<4>(w, chunks, packed, scales, biases, stream);
    case 64: return launch_lpg<8>(w, chunks, packed, scales, biases, stream);
    default: return launch_lpg<16>(w, chunks, packed, scales, biases, stream);
  }
}

}  // namespace int8w
