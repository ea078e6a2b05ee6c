// mxq_device.h -- gfx950 device-side types and codec helpers shared by the
// library's kernels.  (The CPU oracle has its own, independent code.)
//
// Formats: E2M1 elements (magnitudes {0,.5,1,1.5,2,3,4,6}), E8M0 block
// scales 2^(c-127), E4M3 block scales with max 448 and NaN only
// ["4.5 FP8 and NVFP4/MXFP4" (infra-guide), sec. 1.2, 3.1, 4.1].
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mxq {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

// DPP control words (quad_perm): read the value of lane (i ^ 1) / (i ^ 2)
// inside each group of four lanes.
constexpr int kDppQuadXor1 = 0xB1;  // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;  // quad_perm [2,3,0,1]

__device__ __forceinline__ unsigned dpp_quad_xor1(unsigned v) {
  return (unsigned)__builtin_amdgcn_update_dpp(0, (int)v, kDppQuadXor1, 0xF, 0xF, false);
}
__device__ __forceinline__ unsigned dpp_quad_xor2(unsigned v) {
  return (unsigned)__builtin_amdgcn_update_dpp(0, (int)v, kDppQuadXor2, 0xF, 0xF, false);
}

// Largest |x| of the two bf16 values packed in a dword, as bf16 magnitude
// bits (non-negative floats order like their bit patterns).
__device__ __forceinline__ unsigned bf16x2_absmax_bits(unsigned a, unsigned b) {
  u16x2 ua = __builtin_bit_cast(u16x2, a & 0x7FFF7FFFu);
  u16x2 ub = __builtin_bit_cast(u16x2, b & 0x7FFF7FFFu);
  u16x2 m = __builtin_elementwise_max(ua, ub);
  return __builtin_bit_cast(unsigned, m);
}

// E8M0 code for a block whose largest magnitude has exponent field `ef`
// (the biased fp32/bf16 exponent): floor(log2 amax) - 2 clamped at -127,
// i.e. max(ef - 2, 0).  Subnormal amax has ef == 0 and gets code 0.
__device__ __forceinline__ unsigned e8m0_code_from_expfield(unsigned ef) {
  return ef > 2u ? ef - 2u : 0u;
}

// The fp32 whose exponent field is the E8M0 code; the gfx950 scaled convert
// instructions use exactly this exponent (code 0 is read as 2^-127).
__device__ __forceinline__ float e8m0_as_scale(unsigned code) {
  return __uint_as_float(code << 23);
}

// 2^(code - 127) as an fp32 value for arithmetic (code 0 is the subnormal
// 2^-127, which e8m0_as_scale cannot express as a plain multiplier).
__device__ __forceinline__ float e8m0_value(unsigned code) {
  return code ? __uint_as_float(code << 23) : 0x1p-127f;
}

// E4M3 (OCP FP8) value of a code: S EEEE MMM, bias 7, subnormals for
// E = 0 (m/8 * 2^-6), and S 1111 111 is NaN.  gfx950's fp8 convert decodes
// exactly this format (OCP, not the FNUZ variant of earlier CDNA parts) in
// one instruction; the exhaustive dequantize test holds it to the oracle's
// field decode for every code.  B selects byte B of the word.
template <int B = 0>
__device__ __forceinline__ float e4m3_value_b(unsigned w) {
  return __builtin_amdgcn_cvt_f32_fp8((int)w, B);
}
__device__ __forceinline__ float e4m3_value(unsigned c) { return e4m3_value_b<0>(c); }

// E4M3 encode of r >= 0 (finite or +Inf): round to nearest, ties to even
// mantissa, saturate at 448, underflow to 0.
__device__ __forceinline__ unsigned e4m3_encode_nonneg(float r) {
  if (!(r < 448.0f)) return 0x7Eu;
  if (r < 0x1p-6f) {
    // subnormal range: quantum 2^-9; code == number of quanta (8 == 2^-6)
    return (unsigned)__builtin_rintf(r * 512.0f);
  }
  unsigned b = __float_as_uint(r);
  unsigned rounded = b + 0x7FFFFu + ((b >> 20) & 1u);  // RNE to 3 mantissa bits
  return (rounded >> 20) - (120u << 3);
}

// Round an fp32 to bf16 (nearest, ties to even); finite inputs.
__device__ __forceinline__ unsigned short f32_to_bf16_rne(float f) {
  unsigned u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (unsigned short)(u >> 16);
}

// bf16 rounding of the exact value p + err, where p = fl32(a*b) and
// err = a*b - p exactly (|err| <= ulp(p)/2): a single correct rounding.
__device__ __forceinline__ unsigned short bf16_rne_of_sum(float p, float err) {
  unsigned u = __float_as_uint(p);
  unsigned low = u & 0xFFFFu;
  if (low == 0x8000u && err != 0.0f) {
    // p sits exactly on a bf16 midpoint: the residual decides.
    bool up = (err > 0.0f) == ((u >> 31) == 0u);  // away from zero if same sign
    unsigned t = u >> 16;
    return (unsigned short)(up ? t + 1u : t);
  }
  return f32_to_bf16_rne(p);
}

// MXFP4 of one lane's 8 consecutive bf16 values, four lanes (a DPP quad,
// all of it active) forming one 32-element block: block absmax as an integer
// max of magnitude bits shared over the quad, E8M0 code = max(expfield - 2,
// 0), then the scaled convert (round to nearest even, saturation at 6,
// signed zeros).  Returns the 8 codes packed, element 2j in the low nibble
// of byte j, and sets *code to the block's E8M0 code.  Every MXFP4
// quantizer of bf16 data in the library goes through this function.
__device__ __forceinline__ unsigned mx_quantize_quad_bf16(bf16x8 xb, unsigned* code) {
  // The convert's bf16 pairs are built from bf16x8 elements: feeding it a
  // bit_cast<bf16x2>(uint) miscompiled (every call got the first dword).
  const u32x4 v = __builtin_bit_cast(u32x4, xb);
  unsigned m = bf16x2_absmax_bits(bf16x2_absmax_bits(v.x, v.y), bf16x2_absmax_bits(v.z, v.w));
  m = max(m & 0xFFFFu, m >> 16);
  m = max(m, dpp_quad_xor1(m));
  m = max(m, dpp_quad_xor2(m));
  const unsigned c = e8m0_code_from_expfield(m >> 7);
  const float scale = e8m0_as_scale(c);
  unsigned out = 0;
  out = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(out, (bf16x2){xb[0], xb[1]}, scale, 0);
  out = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(out, (bf16x2){xb[2], xb[3]}, scale, 1);
  out = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(out, (bf16x2){xb[4], xb[5]}, scale, 2);
  out = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(out, (bf16x2){xb[6], xb[7]}, scale, 3);
  *code = c;
  return out;
}

// The same quantizer with one lane holding the whole block: elements
// 8j .. 8j+7 in xb[j].  The block absmax, E8M0 code and converts are those
// of mx_quantize_quad_bf16, so codes and scale are bit-identical to it.
// Returns the 16 code bytes (element 2j in the low nibble of byte j).
__device__ __forceinline__ u32x4 mx_quantize_lane_bf16(const bf16x8 (&xb)[4], unsigned* code) {
  unsigned m = 0;
#pragma unroll
  for (int j = 0; j < 4; j++) {
    const u32x4 v = __builtin_bit_cast(u32x4, xb[j]);
    m = bf16x2_absmax_bits(m, bf16x2_absmax_bits(bf16x2_absmax_bits(v.x, v.y), bf16x2_absmax_bits(v.z, v.w)));
  }
  m = max(m & 0xFFFFu, m >> 16);
  const unsigned c = e8m0_code_from_expfield(m >> 7);
  const float scale = e8m0_as_scale(c);
  unsigned o[4];
#pragma unroll
  for (int j = 0; j < 4; j++) {
    unsigned out = 0;
    out = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(out, (bf16x2){xb[j][0], xb[j][1]}, scale, 0);
    out = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(out, (bf16x2){xb[j][2], xb[j][3]}, scale, 1);
    out = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(out, (bf16x2){xb[j][4], xb[j][5]}, scale, 2);
    out = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(out, (bf16x2){xb[j][6], xb[j][7]}, scale, 3);
    o[j] = out;
  }
  *code = c;
  return (u32x4){o[0], o[1], o[2], o[3]};
}

// MXFP8 (E4M3 elements, E8M0 scale per 32) [infra-guide sec. 4.2, mxfp8;
// sec. 1.2, E4M3 max 448].  Block code from the bf16 exponent field of the
// block amax by the MXFP4 rule with E4M3's top exponent: max(ef - 8, 0), so
// the largest magnitude scales into [256, 512).
__device__ __forceinline__ unsigned e8m0_code_e4m3(unsigned ef) { return ef > 8u ? ef - 8u : 0u; }

// E4M3 codes of 8 bf16 values under block code `code`: every magnitude is
// clamped to 448 * 2^e first (the gfx950 scaled fp8 convert gives the NaN
// code for scaled values past 448 instead of saturating; the clamp is exact:
// 448 * 2^e is a bf16 value), then the scaled convert rounds to nearest
// even.  Byte i of the result is element i.  Every MXFP8 quantizer of bf16
// data in the library goes through this function.
__device__ __forceinline__ u32x2 mx8_encode8_bf16(bf16x8 xb, unsigned code) {
  typedef short s16x2 __attribute__((ext_vector_type(2)));
  const float scale = e8m0_as_scale(code);
  const unsigned lim = ((code + 8u) << 7) | 0x60u;  // bf16 bits of 448 * 2^e
  const u16x2 lim2 = {(unsigned short)lim, (unsigned short)lim};
  const u32x4 v = __builtin_bit_cast(u32x4, xb);
  u32x4 cl;
#pragma unroll
  for (int i = 0; i < 4; i++) {
    const unsigned w = v[i];
    const u16x2 mg = __builtin_bit_cast(u16x2, w & 0x7FFF7FFFu);
    cl[i] = __builtin_bit_cast(unsigned, __builtin_elementwise_min(mg, lim2)) | (w & 0x80008000u);
  }
  const bf16x8 xc = __builtin_bit_cast(bf16x8, cl);
  s16x2 lo = {0, 0}, hi = {0, 0};
  lo = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(lo, (bf16x2){xc[0], xc[1]}, scale, false);
  lo = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(lo, (bf16x2){xc[2], xc[3]}, scale, true);
  hi = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(hi, (bf16x2){xc[4], xc[5]}, scale, false);
  hi = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(hi, (bf16x2){xc[6], xc[7]}, scale, true);
  return (u32x2){__builtin_bit_cast(unsigned, lo), __builtin_bit_cast(unsigned, hi)};
}

// Largest |x| of 8 bf16 values as bf16 magnitude bits.
__device__ __forceinline__ unsigned bf16x8_absmax_bits(bf16x8 xb) {
  const u32x4 v = __builtin_bit_cast(u32x4, xb);
  const unsigned m = bf16x2_absmax_bits(bf16x2_absmax_bits(v.x, v.y), bf16x2_absmax_bits(v.z, v.w));
  return max(m & 0xFFFFu, m >> 16);
}

// MXFP8 of one 32-element block held by one lane (elements 8j .. 8j+7 in
// xb[j]): the block code and the 32 code bytes (element i in byte i).
__device__ __forceinline__ void mx8_quantize_lane_bf16(const bf16x8 (&xb)[4], unsigned* code, u32x2 (&out)[4]) {
  unsigned m = 0;
#pragma unroll
  for (int j = 0; j < 4; j++) m = max(m, bf16x8_absmax_bits(xb[j]));
  const unsigned c = e8m0_code_e4m3(m >> 7);
#pragma unroll
  for (int j = 0; j < 4; j++) out[j] = mx8_encode8_bf16(xb[j], c);
  *code = c;
}

}  // namespace mxq
