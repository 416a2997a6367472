// Device helpers of the 1x128 E4M3 quantisers (token rows, the SiLU-mul activation, the fused
// add-RMSNorm): BF16 unpacking and the per-block quantise-and-store of a 16-lane team.
//
// The 1x128 quantiser takes scale = amax/448 and code = E4M3_RNE(x / scale) with IEEE FP32
// division, so that its decisions are reproducible; a block of zeros gets scale 1. Each 128-wide
// block is handled by 16 lanes holding 8 consecutive elements (16-byte loads), and its amax is a
// 16-lane butterfly reduction.
#pragma once
#include "internal.h"

namespace fp8g {
namespace kernels {

constexpr float kE4M3Max = 448.0f;

__device__ __forceinline__ float bf16_bits_to_float(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

__device__ __forceinline__ void unpack_bf16x8(const uint4 raw, float v[8]) {
  const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = bf16_bits_to_float(w[i] & 0xFFFFu);
    v[2 * i + 1] = bf16_bits_to_float(w[i] >> 16);
  }
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  const bf16x2 v = {(__bf16)a, (__bf16)b};  // round-to-nearest-even (v_cvt_pk_bf16_f32)
  return __builtin_bit_cast(uint32_t, v);
}

typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t pack_f16x2(float a, float b) {
  const f16x2_t v = {(_Float16)a, (_Float16)b};  // round-to-nearest-even
  return __builtin_bit_cast(uint32_t, v);
}

// Quantise the 8 values a lane holds, given the amax of its 16-lane team; writes 8 codes + scale.
__device__ __forceinline__ void quant_store_8(const float v[8], float amax, uint8_t* codes_out, float* scale_out,
                                              bool write_scale) {
  const float s = amax > 0.0f ? __fdiv_rn(amax, kE4M3Max) : 1.0f;
  float q[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) q[i] = __fdiv_rn(v[i], s);
  int lo = __builtin_amdgcn_cvt_pk_fp8_f32(q[0], q[1], 0, false);
  lo = __builtin_amdgcn_cvt_pk_fp8_f32(q[2], q[3], lo, true);
  int hi = __builtin_amdgcn_cvt_pk_fp8_f32(q[4], q[5], 0, false);
  hi = __builtin_amdgcn_cvt_pk_fp8_f32(q[6], q[7], hi, true);
  *reinterpret_cast<uint2*>(codes_out) = make_uint2((uint32_t)lo, (uint32_t)hi);
  if (write_scale) *scale_out = s;
}

__device__ __forceinline__ float team16_max(float v) {
#pragma unroll
  for (int off = 8; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 16));
  return v;
}

}  // namespace kernels
}  // namespace fp8g
