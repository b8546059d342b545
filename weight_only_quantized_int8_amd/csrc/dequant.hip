// dequant.hip -- dequantize_to for gfx950: the full BF16 weight from the
// packed codes (rustdoc page "MlxInt8Weight", method dequantize_to).
//
// out[n, k] = RNE_bf16(q[n,k] * scale + bias), row-major [N, K].
//
// HBM-bound streaming kernel: per 16 codes it reads one 16-byte code vector
// (non-temporal: read once) plus a 2-byte scale and bias (shared by the
// gs/16 neighbouring threads of the group, so they hit in cache) and writes
// 32 bytes of BF16.  Algorithmic traffic per weight: 1 + 4/gs bytes read,
// 2 bytes written.  The fp32 value q*s + b is formed with one fused
// multiply-add; q*s is exact in fp32, so this equals the separately rounded
// product-then-sum.  Rounding to BF16 uses the hardware nearest-even convert.
#include "common.h"
#include "launch.h"

namespace int8w {

namespace {

__device__ __forceinline__ void dequant_chunk(uint4 q, float s, float b, uint4 *dst) {
  const uint32_t w[4] = {q.x, q.y, q.z, q.w};
  uint32_t o[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float v0 = __builtin_fmaf(code_f32(w[i], 0), s, b);
    float v1 = __builtin_fmaf(code_f32(w[i], 1), s, b);
    float v2 = __builtin_fmaf(code_f32(w[i], 2), s, b);
    float v3 = __builtin_fmaf(code_f32(w[i], 3), s, b);
    o[2 * i] = pack_bf16x2(v0, v1);
    o[2 * i + 1] = pack_bf16x2(v2, v3);
  }
  store_nt(make_uint4(o[0], o[1], o[2], o[3]), dst);
  store_nt(make_uint4(o[4], o[5], o[6], o[7]), dst + 1);
}

// One thread handles 16 consecutive codes (one uint4 of packed words) per
// step; a grid-stride loop with two steps in flight covers all N*K/16 chunks.
__global__ __launch_bounds__(256) void k_dequant(const uint4 *__restrict__ packed,
                                                 const uint16_t *__restrict__ scales,
                                                 const uint16_t *__restrict__ biases,
                                                 uint4 *__restrict__ out, uint32_t chunks_per_row,
                                                 uint32_t total_chunks, uint32_t groups_per_row,
                                                 uint32_t gs_log2) {
  const uint32_t stride = gridDim.x * blockDim.x;
  for (uint32_t c = blockIdx.x * blockDim.x + threadIdx.x; c < total_chunks; c += 2 * stride) {
    const uint32_t c1 = c + stride;
    const bool has1 = c1 < total_chunks;
    uint4 q0 = load_nt(packed + c);
    uint4 q1 = has1 ? load_nt(packed + c1) : make_uint4(0, 0, 0, 0);
    uint32_t n0 = c / chunks_per_row;
    uint32_t g0 = n0 * groups_per_row + (((c - n0 * chunks_per_row) * 16u) >> gs_log2);
    float s0 = bf16_bits_to_f32(scales[g0]);
    float b0 = bf16_bits_to_f32(biases[g0]);
    float s1 = 0.f, b1 = 0.f;
    if (has1) {
      uint32_t n1 = c1 / chunks_per_row;
      uint32_t g1 = n1 * groups_per_row + (((c1 - n1 * chunks_per_row) * 16u) >> gs_log2);
      s1 = bf16_bits_to_f32(scales[g1]);
      b1 = bf16_bits_to_f32(biases[g1]);
    }
    dequant_chunk(q0, s0, b0, out + 2 * (size_t)c);
    if (has1) dequant_chunk(q1, s1, b1, out + 2 * (size_t)c1);
  }
}

}  // namespace

hipError_t launch_dequant(const WeightView &w, uint16_t *out, hipStream_t stream) {
  const uint32_t chunks_per_row = w.K / 16u;
  const uint32_t total = w.N * chunks_per_row;
  const uint32_t gs_log2 = (uint32_t)__builtin_ctz(w.gs);
  const int threads = 256;
  uint32_t want = (total + 2u * threads - 1u) / (2u * threads);
  uint32_t cap = (uint32_t)device_cu_count() * 8u;  // 8 workgroups of 4 waves per CU
  uint32_t blocks = want < cap ? want : cap;
  if (blocks == 0) blocks = 1;
  hipLaunchKernelGGL(k_dequant, dim3(blocks), dim3(threads), 0, stream,
                     reinterpret_cast<const uint4 *>(w.packed), w.scales, w.biases,
                     reinterpret_cast<uint4 *>(out), chunks_per_row, total, w.K / w.gs, gs_log2);
  return hipGetLastError();
}

}  // namespace int8w
