// Device helpers shared by the gfx950 kernels: NVFP4 decode to exact BF16 operands,
// the bit-exact E4M3 / E2M1 encoders of the quantizer, and thin MFMA wrappers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nvfp4 {

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------------------------------
// Decode. An element is e2m1(code) * e4m3(scale): at most 2 + 4 significant bits and a
// magnitude in [2^-10, 2688], so it is exactly a BF16 value. gfx950's scaled FP4
// conversion applies only the exponent of its f32 scale, so it runs with scale 1.0 (exact
// E2M1 values in f32); the E4M3 scale multiplies in f32 (exact), and the BF16 pattern is
// the high half of the f32 product (exact, nothing is rounded away).
// ---------------------------------------------------------------------------------------

// E4M3 byte `sel` (0..3) of a dword -> f32 (OCP E4M3FN, exact; 0x7F/0xFF give NaN)
template <int SEL>
__device__ __forceinline__ float e4m3_to_f32(uint32_t four_bytes) {
  return __builtin_amdgcn_cvt_f32_fp8(four_bytes, SEL);
}

// two nibbles of byte SEL of `codes` times s -> packed bf16x2 (low nibble in low half)
template <int SEL>
__device__ __forceinline__ uint32_t decode_pair(uint32_t codes, float s) {
  f32x2 v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, 1.0f, SEL);
  float p0 = v[0] * s;
  float p1 = v[1] * s;
  return __builtin_amdgcn_perm(__float_as_uint(p1), __float_as_uint(p0), 0x07060302u);
}

// 8 codes (one dword, k ascending from the low nibble) times one scale -> 8 bf16 (16 B)
__device__ __forceinline__ u32x4 decode8(uint32_t codes, float s) {
  u32x4 r;
  r[0] = decode_pair<0>(codes, s);
  r[1] = decode_pair<1>(codes, s);
  r[2] = decode_pair<2>(codes, s);
  r[3] = decode_pair<3>(codes, s);
  return r;
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// 4x4 transpose of dwords across the four 16-lane rows of a wave: lane (c, g) = c + 16g
// enters holding dword j of 16-byte chunk g in v[j] and leaves holding dword g of chunk j
// in v[j]. Two butterfly stages: v_permlane32_swap exchanges the upper lanes (rows 2, 3)
// of its first operand with the lower lanes (rows 0, 1) of its second; v_permlane16_swap
// exchanges odd rows of its first operand with even rows of its second.
__device__ __forceinline__ void transpose4(u32x4& v) {
  const auto a = __builtin_amdgcn_permlane32_swap(v[0], v[2], false, false);
  const auto b = __builtin_amdgcn_permlane32_swap(v[1], v[3], false, false);
  const auto c = __builtin_amdgcn_permlane16_swap(a[0], b[0], false, false);
  const auto d = __builtin_amdgcn_permlane16_swap(a[1], b[1], false, false);
  v[0] = c[0];
  v[1] = c[1];
  v[2] = d[0];
  v[3] = d[1];
}

// ---------------------------------------------------------------------------------------
// MFMA wrappers (BF16 in, fp32 accumulate). Lane layouts, checked on the hardware:
//  16x16x32: lane l holds A[l%16][8*(l/16)+j], B[8*(l/16)+j][l%16] (j = 0..7) and
//            C[4*(l/16)+r][l%16] (r = 0..3).
//  32x32x16: lane l holds A[l%32][8*(l/32)+j], B[8*(l/32)+j][l%32] and
//            C[8*(r/4) + 4*(l/32) + r%4][l%32] (r = 0..15).
// Which real k sits in slot (lane group, j) is free as long as A and B agree.
// ---------------------------------------------------------------------------------------
__device__ __forceinline__ f32x4 mfma16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma32(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

// ---------------------------------------------------------------------------------------
// Encoders of the quantizer (bit-exact round to nearest, ties to even).
// ---------------------------------------------------------------------------------------

// r >= 0 and finite -> E4M3FN code, saturating at 448 (0x7E).
__device__ __forceinline__ uint32_t e4m3_rne(float r) {
  if (!(r < 448.0f)) return 0x7Eu;
  if (r < 0.015625f) {  // below 2^-6: subnormal codes, spacing 2^-9; r * 512 is exact
    return (uint32_t)__builtin_rintf(r * 512.0f);  // 0..8; 8 is the code of 2^-6
  }
  uint32_t u = __float_as_uint(r);
  uint32_t e = (u >> 23) - 127u + 7u;  // biased E4M3 exponent, 1..15
  uint32_t mant = u & 0x7FFFFFu;
  uint32_t keep = mant >> 20;
  uint32_t rest = mant & 0xFFFFFu;
  uint32_t code = (e << 3) | keep;
  if (rest > 0x80000u || (rest == 0x80000u && (keep & 1u))) code += 1u;  // carries into e
  return code > 0x7Eu ? 0x7Eu : code;
}

// E4M3FN code (finite) -> f32
__device__ __forceinline__ float e4m3_value(uint32_t code) {
  return __builtin_amdgcn_cvt_f32_fp8(code, 0);
}

// Two finite values -> their E2M1 codes in byte `SEL` of `old` (a in the low nibble):
// v_cvt_scalef32_pk_fp4_f32 with scale 1.0 rounds to nearest with ties to the even code,
// saturates at 6 and keeps the sign bit (-0 -> 0x8). On gfx950 it agrees with that rule,
// written out as threshold counts (|q| > 0.25, >= 0.75, > 1.25, >= 1.75, > 2.5, >= 3.5,
// > 5), for every finite fp32 input (checked exhaustively on the device).
template <int SEL>
__device__ __forceinline__ uint32_t e2m1_rne2(uint32_t old, float a, float b) {
  return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(old, a, b, 1.0f, SEL);
}

__device__ __forceinline__ bool is_finite(float v) {
  return (__float_as_uint(v) & 0x7F800000u) != 0x7F800000u;
}

// One 16-block of a row under tensor scale t, by the quantization rule, each step one
// correctly rounded fp32 operation in the stated order:
//   ratio = (amax_b / 6) / t (0 when t == 0);  s = E4M3_RNE(ratio);
//   q_k = x_k / (e4m3(s) * t) (+-0 when that is 0);  code_k = E2M1_RNE(q_k).
// Returns the scale byte; lo / hi receive codes 0..7 / 8..15, low nibble first. Shared by
// the quantizer and the weight-streaming kernel's in-call activation quantization, so
// the two agree bit for bit.
__device__ __forceinline__ uint32_t quantize16(const float v[16], float t, uint32_t& lo,
                                               uint32_t& hi) {
#pragma clang fp contract(off)
  float amax_b = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; i++) amax_b = fmaxf(amax_b, __builtin_fabsf(v[i]));
  const float ratio = (t == 0.0f) ? 0.0f : (amax_b / 6.0f) / t;
  const uint32_t s = e4m3_rne(ratio);
  const float den = e4m3_value(s) * t;
  float q[16];
#pragma unroll
  for (int i = 0; i < 16; i++) q[i] = (den == 0.0f) ? __builtin_copysignf(0.0f, v[i]) : v[i] / den;
  lo = e2m1_rne2<0>(0u, q[0], q[1]);
  lo = e2m1_rne2<1>(lo, q[2], q[3]);
  lo = e2m1_rne2<2>(lo, q[4], q[5]);
  lo = e2m1_rne2<3>(lo, q[6], q[7]);
  hi = e2m1_rne2<0>(0u, q[8], q[9]);
  hi = e2m1_rne2<1>(hi, q[10], q[11]);
  hi = e2m1_rne2<2>(hi, q[12], q[13]);
  hi = e2m1_rne2<3>(hi, q[14], q[15]);
  return s;
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// f32 -> BF16 bits, round to nearest even (finite inputs)
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float v) {
  uint32_t u = __float_as_uint(v);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// silu(g) = g / (1 + e^-g), from the hardware's base-2 exponential and reciprocal (a few
// fp32 ulp; the BF16 product it feeds rounds as the exact value does almost everywhere,
// and never more than one BF16 ulp away). Large negative g: e^-g overflows to +inf and
// the result is -0; large positive g: the result is g.
__device__ __forceinline__ float silu(float g) {
  const float e = __builtin_amdgcn_exp2f(g * -1.44269504088896341f);
  return g * __builtin_amdgcn_rcpf(1.0f + e);
}

}  // namespace nvfp4
