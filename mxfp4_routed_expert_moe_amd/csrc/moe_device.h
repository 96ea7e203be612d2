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

// Two values rounded to bf16 (round to nearest even) and back to fp32 with one packed conversion
// (v_cvt_pk_bf16_f32): the same bits as round_bf16 on each.
__device__ __forceinline__ void round_bf16x2(float& a, float& b) {
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  const uint32_t pk = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{a, b}, bf16x2_t));
  a = bits_to_f32(pk << 16);
  b = bits_to_f32(pk & 0xFFFF0000u);
}

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

// e^x in fp32 for x <= 80 as 2^(x log2 e) on the hardware base-2 exponential (v_exp_f32, 1 ulp). The
// product x log2 e is carried as hi + lo: hi = fp32(x * L2E_HI), lo = the exact error of that product (an
// FMA) plus x * L2E_LO, where L2E_HI + L2E_LO is log2 e to twice fp32 precision (a Cody-Waite split); then
// e^x = 2^hi (1 + lo ln 2). (No overflow guard: the caller keeps x at most 80, e^80 < 2^116.)
__device__ __forceinline__ float exp_f32(float x) {
  constexpr float kL2eHi = 1.44269502162933349609375f;   // fp32(log2 e)
  constexpr float kL2eLo = 1.9259629911266175e-8f;       // log2 e - kL2eHi
  constexpr float kLn2 = 0.693147180559945309f;
  const float hi = x * kL2eHi;
  const float lo = fmaf(x, kL2eLo, fmaf(x, kL2eHi, -hi));
  const float p = __builtin_amdgcn_exp2f(hi);
  return fmaf(p, lo * kLn2, p);
}

// g / d for finite d >= 1: hardware reciprocal (1 ulp), then one FMA correction of the quotient from its
// exact residual g - d q.
__device__ __forceinline__ float div_by_ge1(float g, float d) {
  const float r = __builtin_amdgcn_rcpf(d);
  const float q = g * r;
  return fmaf(fmaf(-d, q, g), r, q);
}

// SwiGLU of the routed/shared expert (section 2 "Expert", section 4 math): g and u are the
// bf16-rounded linear outputs; u is clamped to [-10, 10] and g to at most 10; then
// h = (g / (1 + exp(-g))) * u in fp32, times the route weight rw (1 for the shared expert).
// g is also held at -80 from below, which keeps e^-g finite (one v_med3 instead of overflow guards): below
// -80 the exact |h| is under 80 e^-80 * 10 * rw < 1.5e-32 * rw and the computed one (silu(-80) * u * rw)
// too, both far under the 2^-32 below which the QDQ that follows makes every value a zero code of h's
// sign (its scale is at least 2^-22), and both have the sign of -u * rw: the codes are the same.
__device__ __forceinline__ float swiglu(float g, float u, float rw, bool weighted) {
  g = fminf(fmaxf(g, -80.0f), 10.0f);
  u = fminf(fmaxf(u, -10.0f), 10.0f);
  const float d = 1.0f + exp_f32(-g);
  float h = div_by_ge1(g, d) * u;
  if (weighted) h = rw * h;
  return h;
}

// The SwiGLU step of an epilogue for four (g, u) accumulator pairs of a lane (any type indexable 0..3): g
// and u rounded to bf16 as pairs, swiglu, h rounded to bf16 two at a time. Writes h[0..3] and returns the
// largest |h| of the four.
template <class V>
__device__ __forceinline__ float swiglu_bf16x4(const V& ga, const V& ua, float rw, bool weighted, float* h) {
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    float gv = ga[v], uv = ua[v];
    round_bf16x2(gv, uv);
    h[v] = swiglu(gv, uv, rw, weighted);
  }
  round_bf16x2(h[0], h[1]);
  round_bf16x2(h[2], h[3]);
  return fmaxf(fmaxf(fabsf(h[0]), fabsf(h[1])), fmaxf(fabsf(h[2]), fabsf(h[3])));
}

}  // namespace moe
