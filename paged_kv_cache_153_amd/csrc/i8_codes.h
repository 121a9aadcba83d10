// i8_codes.h — exact conversions of INT8 KV-cache codes to the 16-bit matrix
// operand types, and the rounded bf16 packing of weights, shared by the INT8
// decode and prefill kernels.
//
// Codes are integers in [-127, 127]: fp16 holds them exactly (11 significant
// bits) and so does bf16 (8), so the matrix cores see the codes themselves
// and the row scales are applied outside the products.
#pragma once

#include "device_common.h"

namespace pa {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float float2_t __attribute__((ext_vector_type(2)));

// bf16(a) | bf16(b) << 16, rounded to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16_rne(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(float2_t{a, b}, bf16x2_t));
}

// Four signed codes (one dword) -> two half2 words holding them exactly.
__device__ __forceinline__ void codes_to_half(uint32_t w, uint32_t& lo, uint32_t& hi) {
  const uint32_t u = w ^ 0x80808080u;  // code + 128, as unsigned bytes
  // half bits 0x64uu = 1024 + uu; bytes 4..7 of the pair are the 0x64s
  const uint32_t l16 = __builtin_amdgcn_perm(0x64646464u, u, 0x04010400u);
  const uint32_t h16 = __builtin_amdgcn_perm(0x64646464u, u, 0x04030402u);
  const half2_t bias = {(half_t)1152.f, (half_t)1152.f};
  lo = __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2_t, l16) - bias);
  hi = __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2_t, h16) - bias);
}

// High 16 bits of two floats packed: bf16(a) | bf16(b) << 16 by truncation,
// exact for floats with at most 8 significant bits such as the codes.
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  return __builtin_amdgcn_perm(__builtin_bit_cast(uint32_t, b), __builtin_bit_cast(uint32_t, a),
                               0x07060302u);
}

// Byte K of w as a signed code, in float (exact).
template <int K>
__device__ __forceinline__ float byte_f32(uint32_t w) {
  return (float)((int32_t)(w << (24 - 8 * K)) >> 24);
}

// Four signed codes (one dword) -> two bf16x2 words holding them exactly.
__device__ __forceinline__ void codes_to_bf16(uint32_t w, uint32_t& lo, uint32_t& hi) {
  lo = pack_bf16(byte_f32<0>(w), byte_f32<1>(w));
  hi = pack_bf16(byte_f32<2>(w), byte_f32<3>(w));
}

}  // namespace pa
