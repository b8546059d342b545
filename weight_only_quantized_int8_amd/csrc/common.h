// common.h -- device helpers shared by the gfx950 kernels of libint8w.
//
// Weight encoding (rustdoc page "MlxInt8Weight", field sections packed /
// scales / biases): uint32 words holding four unsigned 8-bit codes, code k of
// a row in byte k%4 of word k/4 (least significant byte first); one BF16
// scale and one BF16 bias per group of group_size codes; w = q*scale + bias.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace int8w {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

// BF16 bit pattern -> fp32 (exact: BF16 is the upper half of binary32).
__device__ __forceinline__ float bf16_lo(uint32_t word) { return __uint_as_float(word << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t word) { return __uint_as_float(word & 0xFFFF0000u); }
__device__ __forceinline__ float bf16_bits_to_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// Two fp32 -> packed BF16 pair, round to nearest even (gfx950 v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2 p = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, p);
}
__device__ __forceinline__ uint16_t to_bf16_bits(float v) {
  return __builtin_bit_cast(uint16_t, (__bf16)v);
}

// Byte b (0..3) of a code word as fp32; the backend selects v_cvt_f32_ubyte{b}.
__device__ __forceinline__ float code_f32(uint32_t word, int b) {
  return (float)((word >> (8 * b)) & 0xFFu);
}

// silu(g) * u in fp32; silu(g) = g / (1 + e^-g), with the hardware
// reciprocal of 1 + e^-g (within 1 ulp) instead of an IEEE division, whose
// scale-and-fixup sequence cost about nine more operations per value.  For
// g -> -inf, e^-g overflows to +inf, its reciprocal is +0 and the product
// -0, the limit of silu there; for g -> +inf it is g.
__device__ __forceinline__ float silu_mul(float g, float u) {
  const float e = __expf(-g);
  return g * __builtin_amdgcn_rcpf(1.0f + e) * u;
}

// Sum over the 64 lanes of a wave; every lane receives the total.
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Streaming (read-once) loads and write-once stores: non-temporal hint.
__device__ __forceinline__ uint4 load_nt(const uint4 *p) {
  u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint2 load_nt(const uint2 *p) {
  u32x2 v = __builtin_nontemporal_load(reinterpret_cast<const u32x2 *>(p));
  return make_uint2(v.x, v.y);
}
__device__ __forceinline__ void store_nt(uint4 v, uint4 *p) {
  u32x4 t = {v.x, v.y, v.z, v.w};
  __builtin_nontemporal_store(t, reinterpret_cast<u32x4 *>(p));
}

// ---- buffer loads.  A raw buffer resource bounds every access: a load whose
// byte offset (plus its size) exceeds num_records returns zero and touches no
// memory, so a pipeline can issue its loads unconditionally and mark the ones
// past the end with an out-of-range offset instead of branching.
constexpr uint32_t kOutOfRange = 0x80000000u;
constexpr int kBufferDword3 = 0x00020000;  // raw (untyped) buffer, 32-bit data format
constexpr int kAuxNontemporal = 2;          // nt: streamed once

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t num_bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)num_bytes, kBufferDword3);
}
template <int AUX = 0>
__device__ __forceinline__ u32x4 buf_load_b128(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, AUX);
}
template <int AUX = 0>
__device__ __forceinline__ u32x2 buf_load_b64(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, AUX);
}
__device__ __forceinline__ uint16_t buf_load_b16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b16(r, (int)off, 0, 0);
}

}  // namespace int8w
