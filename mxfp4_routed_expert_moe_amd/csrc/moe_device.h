// Device-side helpers shared by the gfx950 kernels of the routed-MoE layer.
//
// Number formats follow the page "Native 1017 DSpark draft on the NVLink pair (N1-NATIVE)", section 2 "Official semantics":
// E2M1 nibbles (low nibble = even input), E8M0 scales 2^(b-127), FP8 E4M3 (OCP "e4m3fn"), bf16 with
// round-to-nearest-even at every rounding point.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short short8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bits_to_f32(uint32_t u) { return __builtin_bit_cast(float, u); }
__device__ __forceinline__ uint32_t f32_to_bits(float f) { return __builtin_bit_cast(uint32_t, f); }

// bf16 bit pattern -> fp32 (exact)
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return bits_to_f32(uint32_t(b) << 16); }

// fp32 -> bf16 bit pattern, round to nearest even (inputs are finite): one v_cvt_pk_bf16_f32
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }

// fp32 -> the bf16 value it rounds to, as an fp32
__device__ __forceinline__ float round_bf16(float f) { return bf16_to_f32(f32_to_bf16_rne(f)); }

// E8M0 byte -> fp32 scale 2^(b-127); bytes 1..254 are exact normal fp32 values
__device__ __forceinline__ float e8m0_to_f32(uint32_t b) { return bits_to_f32((b & 0xFFu) << 23); }

// Activation QDQ scale (section 2, act_quant with a ue8m0 scale): E = ceil(log2(fp32(max(amax, 1e-4)
// * fp32(1/448)))) read from the fp32 bits. Returns E; the stored E8M0 byte is E + 127.
__device__ __forceinline__ int qdq_exponent(float amax) {
  float a = fmaxf(amax, 1e-4f);
  float v = a * (1.0f / 448.0f);
  uint32_t u = f32_to_bits(v);
  int e = int((u >> 23) & 0xFFu) - 127;
  return e + ((u & 0x7FFFFFu) != 0u);
}

// 2^-E as an exact fp32 (E in [-126, 126])
__device__ __forceinline__ float exp2_neg(int E) { return bits_to_f32(uint32_t(127 - E) << 23); }

// fp32 value v with |v| <= 448 -> E4M3fn code, round to nearest even, subnormals kept, sign of zero kept.
__device__ __forceinline__ uint32_t e4m3_encode_rne(float v) {
  uint32_t u = f32_to_bits(v);
  uint32_t sign = (u >> 24) & 0x80u;
  uint32_t a = u & 0x7FFFFFFFu;
  uint32_t code;
  if (a < 0x3C800000u) {                       // |v| < 2^-6: subnormal, quantum 2^-9
    float m = __builtin_rintf(bits_to_f32(a) * 512.0f);
    code = uint32_t(m);                          // 0..8 (8 is the smallest normal, code 0x08)
  } else {                                       // round the fp32 mantissa to 3 bits
    uint32_t r = a + 0x7FFFFu + ((a >> 20) & 1u);
    code = (r >> 20) - (120u << 3);              // rebias exponent 127 -> 7
  }
  return code | sign;
}

// QDQ of one value given the block exponent E: clamp(x / 2^E, +-448) -> E4M3 code
__device__ __forceinline__ uint32_t qdq_code(float x, float inv_scale) {
  float q = x * inv_scale;                       // exact: power-of-two scaling
  q = fminf(fmaxf(q, -448.0f), 448.0f);
  return e4m3_encode_rne(q);
}

// Four QDQ codes packed little-endian into a dword (x0 in the low byte), with the gfx950 FP8 converter
// (v_cvt_pk_fp8_f32: E4M3fn, round to nearest even, subnormals kept) on the clamped quotients; equal
// to qdq_code on every bf16 input (checked exhaustively on the GPU).
__device__ __forceinline__ uint32_t qdq_code4(float x0, float x1, float x2, float x3, float inv_scale) {
  auto q = [&](float x) { return fminf(fmaxf(x * inv_scale, -448.0f), 448.0f); };
  const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(q(x0), q(x1), 0, false);
  return uint32_t(__builtin_amdgcn_cvt_pk_fp8_f32(q(x2), q(x3), lo, true));
}

// Packed FP4 byte -> two bf16 (low nibble first) times the E8M0 scale, via the gfx950 converter
template <int BYTE>
__device__ __forceinline__ uint32_t fp4x2_to_bf16x2(uint32_t packed4, float scale) {
  bf16x2 r = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(packed4, scale, BYTE);
  return __builtin_bit_cast(uint32_t, r);
}

// Two E4M3 codes (word WORD of a dword) -> two bf16 times the scale
template <bool WORD>
__device__ __forceinline__ uint32_t fp8x2_to_bf16x2(uint32_t packed8, float scale) {
  bf16x2 r = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(packed8, scale, WORD);
  return __builtin_bit_cast(uint32_t, r);
}

// e^x in fp32 as 2^(x log2 e) on the hardware base-2 exponential (v_exp_f32, 1 ulp). The product
// x log2 e is carried as hi + lo: hi = fp32(x * L2E_HI), lo = the exact error of that product (an FMA)
// plus x * L2E_LO, where L2E_HI + L2E_LO is log2 e to twice fp32 precision (a Cody-Waite split); then
// e^x = 2^hi (1 + lo ln 2). Overflow (x above ln FLT_MAX) returns +inf.
__device__ __forceinline__ float exp_f32(float x) {
  constexpr float kL2eHi = 1.44269502162933349609375f;   // fp32(log2 e)
  constexpr float kL2eLo = 1.9259629911266175e-8f;       // log2 e - kL2eHi
  constexpr float kLn2 = 0.693147180559945309f;
  const float hi = x * kL2eHi;
  const float lo = fmaf(x, kL2eLo, fmaf(x, kL2eHi, -hi));
  const float p = __builtin_amdgcn_exp2f(hi);
  return x > 88.72f ? __builtin_inff() : fmaf(p, lo * kLn2, p);
}

// g / d for d >= 1 or d = +inf: hardware reciprocal (1 ulp), then one FMA correction of the quotient
// from its exact residual g - d q.
__device__ __forceinline__ float div_by_ge1(float g, float d) {
  const float r = __builtin_amdgcn_rcpf(d);
  const float q = g * r;
  const float q2 = fmaf(fmaf(-d, q, g), r, q);
  return d == __builtin_inff() ? g * 0.0f : q2;
}

// SwiGLU of the routed/shared expert (section 2 "Expert", section 4 math): g and u are the
// bf16-rounded linear outputs; u is clamped to [-10, 10] and g to at most 10; then
// h = (g / (1 + exp(-g))) * u in fp32, times the route weight rw (1 for the shared expert).
__device__ __forceinline__ float swiglu(float g, float u, float rw, bool weighted) {
  g = fminf(g, 10.0f);
  u = fminf(fmaxf(u, -10.0f), 10.0f);
  const float d = 1.0f + exp_f32(-g);
  float h = div_by_ge1(g, d) * u;
  if (weighted) h = rw * h;
  return h;
}

}  // namespace moe
