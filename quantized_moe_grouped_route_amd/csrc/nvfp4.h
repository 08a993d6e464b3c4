// NVFP4 weight decode shared by the NVFP4 schedules.
//
// An E2M1 code times its UE4M3 block scale is always a bf16 value (every
// product of the 16 E2M1 values and the 127 non-negative finite e4m3 values
// fits in 8 significant bits), so dequantization is exact: each byte (two
// E2M1 codes, element 2b in the low nibble) is widened to two fp32 values by
// the gfx950 conversion (scale operand 2^0), multiplied by the block scale
// in fp32 (exact) and packed to bf16 (exact, no rounding happens).
#pragma once

#include "common.h"

namespace moeq {

// Two E2M1 codes in byte `sel` of `word` -> fp32 pair (low nibble first).
template <int SEL>
__device__ __forceinline__ v2f e2m1x2_f32(u32 word) {
  return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(word, 1.0f, SEL);
}

// Two floats -> packed bf16 pair (one v_cvt_pk_bf16_f32, nearest even).
__device__ __forceinline__ u32 pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(u32, __builtin_convertvector(v2f{lo, hi}, v2bf));
}

// 8 E2M1 codes (one 32-bit word, elements 0..7) times `scale` -> 8 bf16 as
// four packed 32-bit words, in element order.
__device__ __forceinline__ u32x4 dequant8_bf16(u32 word, float scale) {
  const v2f p0 = e2m1x2_f32<0>(word), p1 = e2m1x2_f32<1>(word);
  const v2f p2 = e2m1x2_f32<2>(word), p3 = e2m1x2_f32<3>(word);
  return u32x4{pack_bf16x2(p0.x * scale, p0.y * scale), pack_bf16x2(p1.x * scale, p1.y * scale),
               pack_bf16x2(p2.x * scale, p2.y * scale), pack_bf16x2(p3.x * scale, p3.y * scale)};
}

// The same 8 bf16 values packed by taking the high halves of the fp32
// products with one byte permute per pair: the products are exact bf16
// values, so their low halves are zero and no rounding is skipped.  The
// products are formed as scalars and only scalars are bit-cast: this
// compiler keeps just element 0 when elements of a vector are bit-cast one
// by one.
__device__ __forceinline__ u32 hi_halves(float lo, float hi) {
  // v_perm_b32: selector bytes 0-3 pick from the second operand
  return __builtin_amdgcn_perm(__builtin_bit_cast(u32, hi), __builtin_bit_cast(u32, lo), 0x07060302u);
}
__device__ __forceinline__ u32x4 dequant8_bf16_hi(u32 word, float scale) {
  const v2f p0 = e2m1x2_f32<0>(word), p1 = e2m1x2_f32<1>(word);
  const v2f p2 = e2m1x2_f32<2>(word), p3 = e2m1x2_f32<3>(word);
  return u32x4{hi_halves(p0.x * scale, p0.y * scale), hi_halves(p1.x * scale, p1.y * scale),
               hi_halves(p2.x * scale, p2.y * scale), hi_halves(p3.x * scale, p3.y * scale)};
}

// binary16 form, for binary16 activations.  Every E2M1 x UE4M3 product is
// also a binary16 value (at most 6 significant bits, magnitudes in
// [2^-10, 2688]), so the packed fp16 multiply is exact too; it halves the
// VALU work of the fp32 form: per 8 codes, 4 conversions and 4 packed
// multiplies.
// Two UE4M3 scale bytes (bytes 0 and 1 of `two`) -> their binary16 values.
__device__ __forceinline__ v2h ue4m3x2_f16(u32 two) {
  return __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(two, 1.0f, false);
}
template <int SEL>
__device__ __forceinline__ u32 e2m1x2_times(u32 word, v2h s2) {
  const v2h p = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(word, 1.0f, SEL) * s2;
  return __builtin_bit_cast(u32, p);
}
// 8 E2M1 codes (one word, elements 0..7) times the scale held twice in s2.
__device__ __forceinline__ u32x4 dequant8_f16(u32 word, v2h s2) {
  return u32x4{e2m1x2_times<0>(word, s2), e2m1x2_times<1>(word, s2), e2m1x2_times<2>(word, s2),
               e2m1x2_times<3>(word, s2)};
}

// Packed pair of output elements of kind KIND (bf16 or f16) from two floats.
template <int KIND>
__device__ __forceinline__ u32 pack2(float lo, float hi) {
  if (KIND == OUT_BF16) return pack_bf16x2(lo, hi);
  return (u32)f32_to_f16_bits(lo) | ((u32)f32_to_f16_bits(hi) << 16);
}

}  // namespace moeq
