// Per-token router selection and per-32 activation QDQ as device functions, shared by the separate
// router kernels and the fused decode-width select + permute kernel, so that every path makes the same
// decisions in the same fp32 order.
//
// Gate (page "Native 1017 DSpark draft on the NVLink pair (N1-NATIVE)", section 2 "Gate"): scores sqrt(softplus(l)), top-k of
// scores + bias (the bias only selects), the chosen scores normalised by their sum + 1e-20 and scaled
// by the route scale. Activation QDQ (same section, "Quantized linear"): per 32 inputs, E8M0 scale
// 2^ceil(log2(max(amax, 1e-4) / 448)) and E4M3 codes.
#pragma once

#include "moe_device.h"

namespace moe {

// Partial logit planes per token: H / 512 at decode widths (H <= 8192), 4 above.
constexpr int kMaxLogitParts = 16;

// fp32 -> unsigned key with the same order (finite values; -0 and +0 both map to the key of +0, as
// they compare equal). Every finite value maps above 0.
__device__ __forceinline__ uint32_t ordered_key(float f) {
  const uint32_t b = __float_as_uint(f + 0.0f);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// Maximum of a 32-bit value over the 64 lanes of the wave, returned to every lane (wave-uniform).
// Inside each 16-lane row: DPP exchanges with the lane at xor 1 and xor 2 (quad permutes), then with the
// mirrored lane in the 8-lane half and in the row, each step taking the larger value, so every lane
// ends with its row's maximum; then the four row maxima are read as scalars.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, false));    // quad_perm [1, 0, 3, 2]
  v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, false));    // quad_perm [2, 3, 0, 1]
  v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x141, 0xF, 0xF, false));   // row_half_mirror
  v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x140, 0xF, 0xF, false));   // row_mirror
  const uint32_t m01 = max((uint32_t)__builtin_amdgcn_readlane((int)v, 0), (uint32_t)__builtin_amdgcn_readlane((int)v, 16));
  const uint32_t m23 = max((uint32_t)__builtin_amdgcn_readlane((int)v, 32), (uint32_t)__builtin_amdgcn_readlane((int)v, 48));
  return max(m01, m23);
}

// Lane 0's value after an xor butterfly over the 64 lanes (offsets 32, 16, 8, 4, 2, 1 in that order, each step
// a += a[lane ^ offset]), with the same bits. Offsets 32 and 16 are lane permutes; for 8, 4, 2 and 1, every lane
// that lane 0's sum depends on has lane < offset, so its partner lane ^ offset = lane + offset lies in the same
// 16-lane row and a DPP row shift reads it. Only lane 0's result is meaningful.
__device__ __forceinline__ float wave_sum_lane0(float a) {
  a += __shfl_xor(a, 32, 64);
  a += __shfl_xor(a, 16, 64);
  a += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(a), 0x108, 0xF, 0xF, true));   // row_shl:8
  a += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(a), 0x104, 0xF, 0xF, true));   // row_shl:4
  a += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(a), 0x102, 0xF, 0xF, true));   // row_shl:2
  a += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(a), 0x101, 0xF, 0xF, true));   // row_shl:1
  return a;
}

// Inclusive prefix sum of a 32-bit value over the 64 lanes of the wave, on DPP: inside each 16-lane row by
// shifts of 1, 2, 4 and 8 lanes (lanes past the row's start add 0), then across rows by adding lane 15 to rows 1
// and 3 and lane 31 to rows 2 and 3.
__device__ __forceinline__ int wave_incl_scan(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, true);    // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, true);    // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, true);    // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, true);    // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xA, 0xF, false);   // row_bcast:15 into rows 1, 3
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xC, 0xF, false);   // row_bcast:31 into rows 2, 3
  return v;
}

// One wave selects the experts of token t from the partial logit planes [nparts][M][E] (added in
// ascending plane order). Lane r writes ids[t * k + r] and rw[t * k + r] (r = rank, descending
// selection score); when sid is given, the ids to sid[t * k + r] too, and when emask is given (t < 64)
// it sets bit t of emask[id] for each chosen expert. The k ids of a token are distinct. k <= 8; NJ experts
// per lane, E <= 64 * NJ (NJ = 2 for E <= 128 halves the per-lane work; the decisions do not depend on NJ).
template <int NJ>
__device__ __forceinline__ void select_token(int t, int M, int E, int k, float route_scale, int nparts,
                                             const float* __restrict__ logits, const float* __restrict__ gate_b,
                                             int lane, int32_t* __restrict__ ids, float* __restrict__ rw,
                                             int* sid, unsigned long long* emask) {
  // scores and selection values: lane owns experts lane, lane + 64, ... Every partial logit load is
  // issued before the first is used; the planes are then added in ascending order.
  const size_t plane = (size_t)M * E;
  float pv[NJ][kMaxLogitParts], bias[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int e = lane + 64 * j;
    bias[j] = 0.0f;
    if (e < E) {
      const float* lp = logits + (size_t)t * E + e;
#pragma unroll
      for (int c = 0; c < kMaxLogitParts; ++c) pv[j][c] = c < nparts ? lp[c * plane] : 0.0f;
      bias[j] = gate_b[e];
    }
  }
  float sc[NJ];
  uint32_t key[NJ];   // selection order as one unsigned key: ordered fp32 bits of the selection score
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int e = lane + 64 * j;
    sc[j] = 0.0f;
    key[j] = 0u;   // below every real candidate
    if (e < E) {
      float l = pv[j][0];
#pragma unroll
      for (int c = 1; c < kMaxLogitParts; ++c)
        if (c < nparts) l = l + pv[j][c];
      const float sp = l > 20.0f ? l : log1pf(expf(l));
      sc[j] = sqrtf(sp);
      key[j] = ordered_key(sc[j] + bias[j]);
    }
  }
  // k rounds of a wave-wide maximum: the larger selection score wins, equal scores go to the lower
  // expert id; the winner's lane then hands over its unbiased score
  float wsel[8];
  int isel[8];
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    wsel[r] = 0.0f;
    isel[r] = 0;
    if (r >= k) continue;
    // the largest key over the wave, then its lowest expert id (id = lane + 64 j: the smallest j that holds
    // it, then the lowest lane): the same order as a maximum of (key, -id) pairs, in 32-bit steps
    uint32_t best = key[0];
#pragma unroll
    for (int j = 1; j < NJ; ++j) best = max(best, key[j]);
    best = wave_max_u32(best);
    int win = 0;
#pragma unroll
    for (int j = NJ - 1; j >= 0; --j) {
      const unsigned long long hit = __ballot(key[j] == best);
      if (hit != 0ull) win = 64 * j + (__ffsll(hit) - 1);
    }
    const int jw = win >> 6;
    float mine = sc[0];
#pragma unroll
    for (int j = 1; j < NJ; ++j)
      if (jw == j) mine = sc[j];
    wsel[r] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(mine), win & 63));
    isel[r] = win;
#pragma unroll
    for (int j = 0; j < NJ; ++j)
      if (lane + 64 * j == win) key[j] = 0u;   // remove the winner
  }
  // the selected scores are wave-uniform, so every lane forms the same normalising sum (slot order); lane r < k
  // then writes slot r
  float sum = 0.0f;
#pragma unroll
  for (int r = 0; r < 8; ++r)
    if (r < k) sum = sum + wsel[r];
  const float denom = sum + 1e-20f;
  if (lane < k) {
    float wv = wsel[0];
    int iv = isel[0];
#pragma unroll
    for (int r = 1; r < 8; ++r)
      if (lane == r) {
        wv = wsel[r];
        iv = isel[r];
      }
    ids[(size_t)t * k + lane] = iv;
    rw[(size_t)t * k + lane] = (wv / denom) * route_scale;
    if (sid != nullptr) sid[t * k + lane] = iv;
    if (emask != nullptr) atomicOr(&emask[iv], 1ull << t);
  }
}

// QDQ of one 32-wide block of a bf16 row into registers: the 32 E4M3 codes (little-endian, 16 per
// u32x4) and the returned E8M0 byte.
__device__ __forceinline__ uint8_t qdq_block32_regs(const uint16_t* __restrict__ src, u32x4& q0, u32x4& q1) {
  u32x4 raw[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) raw[i] = *reinterpret_cast<const u32x4*>(src + 8 * i);
  float v[32];
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[8 * i + 2 * j] = bits_to_f32(raw[i][j] << 16);
      v[8 * i + 2 * j + 1] = bits_to_f32(raw[i][j] & 0xFFFF0000u);
    }
#pragma unroll
  for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
  const int E8 = qdq_exponent(amax);
  const float inv = exp2_neg(E8);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    q0[i] = qdq_code4(v[4 * i], v[4 * i + 1], v[4 * i + 2], v[4 * i + 3], inv);
    q1[i] = qdq_code4(v[16 + 4 * i], v[17 + 4 * i], v[18 + 4 * i], v[19 + 4 * i], inv);
  }
  return uint8_t(E8 + 127);
}

// QDQ of one 32-wide block of a bf16 row: 32 E4M3 codes to q (16-byte aligned) and the E8M0 byte to *s.
__device__ __forceinline__ void qdq_block32(const uint16_t* __restrict__ src, uint8_t* __restrict__ q,
                                            uint8_t* __restrict__ s) {
  u32x4 q0, q1;
  const uint8_t sc = qdq_block32_regs(src, q0, q1);
  u32x4* dst = reinterpret_cast<u32x4*>(q);
  dst[0] = q0;
  dst[1] = q1;
  *s = sc;
}

}  // namespace moe
