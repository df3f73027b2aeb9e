// Shared device helpers for the NVFP4 MoE kernels (gfx950 / CDNA4 only).
//
// Element decoding follows the NVFP4 format: E2M1 codes (two per byte, element 2j in
// the low nibble), one FP8 E4M3 (OCP "FN") scale per 16 inputs, one FP32 global scale
// per expert tensor ("Strata NVFP4" README, "How it differs from upstream Strata";
// TensorFold pull 906 for the E4M3 scale bytes and the 16-input groups).
//
// gfx950 facts these helpers rely on (each checked against the CPU oracle by the
// bit-exact dequantization tests):
//   * v_cvt_scalef32_pk_{f32,f16,bf16}_fp4 decode the two E2M1 codes of one byte, low
//     nibble first, and multiply by 2^exponent(scale): only the scale's exponent is
//     used (an E8M0 scale), never its mantissa.
//   * v_cvt_f32_fp8 decodes the OCP E4M3 "FN" format (0x7F/0xFF NaN, max 448).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef int i32x4_t __attribute__((ext_vector_type(4)));
typedef int i32x16_t __attribute__((ext_vector_type(16)));

namespace nvfp4 {

constexpr int kGroup = 16;

// ---------------------------------------------------------------- scalar codecs
// E4M3 byte SEL of `word` -> fp32 (exact).
template <int SEL>
__device__ __forceinline__ float e4m3_f32(uint32_t word) {
  return __builtin_amdgcn_cvt_f32_fp8((int)word, SEL);
}

// The two E2M1 codes of byte SEL of `word` as exact fp32 values (low nibble -> [0]).
template <int SEL>
__device__ __forceinline__ f32x2_t e2m1x2_f32(uint32_t word) {
  return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(word, 1.0f, SEL);
}

// The two E2M1 codes of byte SEL as exact bf16 values.
template <int SEL>
__device__ __forceinline__ bf16x2_t e2m1x2_bf16(uint32_t word) {
  return __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(word, 1.0f, SEL);
}

// Two E4M3 scale bytes (bytes 2*HI and 2*HI+1 of `word`) as fp16. Every E4M3 value,
// subnormals and NaN included, is an fp16 value, so the convert is exact.
template <bool HI>
__device__ __forceinline__ f16x2_t e4m3x2_f16(uint32_t word) {
  return __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(word, 1.0f, HI);
}

// Byte SEL of `word` -> two weights e2m1 * s in fp16. The E2M1 convert is exact; the
// product has at most 5 significant bits (1 from the code, 4 from the scale) and
// magnitude 2^-10 .. 2688, so the fp16 multiply is exact too. A NaN scale gives NaN.
template <int SEL>
__device__ __forceinline__ f16x2_t e2m1x2_f16_scaled(uint32_t word, _Float16 s) {
  const f16x2_t v = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(word, 1.0f, SEL);
  return v * f16x2_t{s, s};
}

// Four bytes (8 codes) -> 8 exact fp16 weights, element order = k order.
__device__ __forceinline__ void unpack8_f16(uint32_t word, _Float16 s, f16x2_t out[4]) {
  out[0] = e2m1x2_f16_scaled<0>(word, s);
  out[1] = e2m1x2_f16_scaled<1>(word, s);
  out[2] = e2m1x2_f16_scaled<2>(word, s);
  out[3] = e2m1x2_f16_scaled<3>(word, s);
}

// ---------------------------------------------------------------- bf16 helpers
__device__ __forceinline__ float bf16_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t v) { return __uint_as_float(v & 0xFFFF0000u); }

__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  __bf16 b = (__bf16)f;  // round to nearest even
  return __builtin_bit_cast(uint16_t, b);
}

__device__ __forceinline__ uint16_t f32_to_f16_bits(float f) {
  _Float16 h = (_Float16)f;  // round to nearest even
  return __builtin_bit_cast(uint16_t, h);
}

__device__ __forceinline__ float silu(float z) { return z / (1.0f + __expf(-z)); }

// ---------------------------------------------------------------- wave reductions
// Sum over groups of 16 consecutive lanes (every lane of the group gets the total).
// Sum over each row of 16 lanes (lanes 16r .. 16r+15), the result in all 16 lanes, with
// DPP moves (VALU only, no LDS crossbar): swap neighbours, swap pairs, then rotate the
// row by 4 and by 8 lanes.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float sum16(float v) {
  v += dpp_mov<0xB1>(v);   // quad_perm [1,0,3,2]
  v += dpp_mov<0x4E>(v);   // quad_perm [2,3,0,1]
  v += dpp_mov<0x124>(v);  // row_ror:4
  v += dpp_mov<0x128>(v);  // row_ror:8
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

}  // namespace nvfp4
