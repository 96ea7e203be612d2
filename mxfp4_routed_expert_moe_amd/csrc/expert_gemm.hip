// Expert GEMMs at decode width (few rows per expert) on gfx950.
//
// Math (DeepSeek-V4.1-Flash native-tensor page, section 4 "Kernel contract", per (t, j) with
// e = ids[t, j]): g = bf16(sum_k x w1), u = bf16(sum_k x w3), u = clamp(u, -10, 10), g = min(g, 10),
// h = (g / (1 + exp(-g))) * u, h = rw * h, h16 = bf16(h), h_q = act_qdq(h16) per 32;
// y = bf16(sum_k h_q w2). The shared expert (section 2 "Expert") is the same without rw.
//
// Design. The weights are the large operand and are streamed exactly once per launch: a block owns
// one expert and one block of weight rows, its four waves split the inner dimension, and each lane
// issues 128-bit loads of packed FP4 (16 bytes = 32 weights of one row). The gfx950 converters
// (v_cvt_scalef32_pk_bf16_fp4 / _fp8) turn codes times their E8M0 scale into bf16 in registers; the
// values are exact in bf16 (section 2: decoded weights and QDQ'd activations are bf16-exact), so
// the bf16 MFMA (v_mfma_f32_16x16x32_bf16) forms exact products summed in fp32: the result differs
// from the official arithmetic only in fp32 summation order. Tokens of the expert fill the MFMA's
// 16 columns (missing ones are zero). The four waves' fp32 partials are added in a fixed order in
// LDS, so results are deterministic.
//
// Operand layout of v_mfma_f32_16x16x32_bf16: lane l supplies row (l % 16) of A (a weight row) and
// column (l % 16) of B (a token), 8 values each; the output element (4 * (l / 16) + v, l % 16) sits in
// accumulator v of lane l. The 8 values of lane group g = l / 16 in MFMA i of a 128-wide step are the
// inputs k0 + 32 g + 8 i .. + 7 for both operands, so each lane's 16-byte FP4 load covers exactly one
// E8M0 scale block.
#include "kernels.h"
#include "moe_device.h"

namespace moe {

constexpr int kWaves = 4;

// Load and convert the A operand (16 weight rows x 128 inputs) for one step: 4 MFMA fragments.
template <int WF>
__device__ __forceinline__ void load_a(const GemmProblem& p, const void* wbase, const uint8_t* sbase, int e,
                                       int row, int k0, int g, bf16x8 (&A)[4]) {
  const int K = p.K;
  if constexpr (WF == W_MXFP4) {
    const uint8_t* w = static_cast<const uint8_t*>(wbase) + (size_t)e * p.w_expert_stride + (size_t)row * (K / 2);
    const u32x4 raw = *reinterpret_cast<const u32x4*>(w + k0 / 2 + 16 * g);
    const float sc = e8m0_to_f32(sbase[(size_t)e * p.s_expert_stride + (size_t)row * (K / 32) + k0 / 32 + g]);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint32_t d[4] = {fp4x2_to_bf16x2<0>(raw[i], sc), fp4x2_to_bf16x2<1>(raw[i], sc),
                       fp4x2_to_bf16x2<2>(raw[i], sc), fp4x2_to_bf16x2<3>(raw[i], sc)};
      A[i] = __builtin_bit_cast(bf16x8, u32x4{d[0], d[1], d[2], d[3]});
    }
  } else if constexpr (WF == W_FP8_BLOCK32) {
    const uint8_t* w = static_cast<const uint8_t*>(wbase) + (size_t)e * p.w_expert_stride + (size_t)row * K;
    const u32x4 r0 = *reinterpret_cast<const u32x4*>(w + k0 + 32 * g);
    const u32x4 r1 = *reinterpret_cast<const u32x4*>(w + k0 + 32 * g + 16);
    const float sc = e8m0_to_f32(sbase[(size_t)e * p.s_expert_stride + (size_t)(row / 32) * (K / 32) + k0 / 32 + g]);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t d0 = (i < 2) ? r0[2 * i] : r1[2 * i - 4];
      const uint32_t d1 = (i < 2) ? r0[2 * i + 1] : r1[2 * i - 3];
      A[i] = __builtin_bit_cast(bf16x8, u32x4{fp8x2_to_bf16x2<false>(d0, sc), fp8x2_to_bf16x2<true>(d0, sc),
                                              fp8x2_to_bf16x2<false>(d1, sc), fp8x2_to_bf16x2<true>(d1, sc)});
    }
  } else {  // W_BF16
    const uint16_t* w = static_cast<const uint16_t*>(wbase) + (size_t)e * p.w_expert_stride + (size_t)row * K;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      A[i] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(w + k0 + 32 * g + 8 * i));
  }
}

// Load and convert the B operand (one token row, 32 E4M3 codes + scale per lane) for one step.
__device__ __forceinline__ void load_b(const GemmProblem& p, int arow, bool valid, int k0, int g, bf16x8 (&B)[4]) {
  u32x4 r0 = {0u, 0u, 0u, 0u}, r1 = {0u, 0u, 0u, 0u};
  float sc = 0.0f;
  if (valid) {
    const uint8_t* a = p.act_q + (size_t)arow * p.K + k0 + 32 * g;
    r0 = *reinterpret_cast<const u32x4*>(a);
    r1 = *reinterpret_cast<const u32x4*>(a + 16);
    sc = e8m0_to_f32(p.act_s[(size_t)arow * (p.K / 32) + k0 / 32 + g]);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t d0 = (i < 2) ? r0[2 * i] : r1[2 * i - 4];
    const uint32_t d1 = (i < 2) ? r0[2 * i + 1] : r1[2 * i - 3];
    B[i] = __builtin_bit_cast(bf16x8, u32x4{fp8x2_to_bf16x2<false>(d0, sc), fp8x2_to_bf16x2<true>(d0, sc),
                                            fp8x2_to_bf16x2<false>(d1, sc), fp8x2_to_bf16x2<true>(d1, sc)});
  }
}

// One block: expert slot blockIdx.y, weight rows [n0, n0 + NB), all rows (tokens) of the expert in
// groups of 16. GEMM1: tiles 0,1 = w1 rows n0..n0+31, tiles 2,3 = w3 rows n0..n0+31 (NB = 32).
// GEMM2: tiles 0..3 = w2 rows n0..n0+63 (NB = 64).
template <int WF, bool GEMM1>
__global__ __launch_bounds__(256) void expert_gemm_small(GemmProblem p) {
  constexpr int NB = GEMM1 ? 32 : 64;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int r16 = lane & 15, g = lane >> 4;
  int e, row0, nrows;
  if (p.dense) {
    if (blockIdx.y > 0) return;
    e = 0; row0 = 0; nrows = p.M;
  } else {
    e = p.active[blockIdx.y];
    if (e < 0) return;
    row0 = p.offsets[e];
    nrows = p.offsets[e + 1] - row0;
  }
  const int n0 = blockIdx.x * NB;
  const int nsteps = p.K / 128;
  const int s_begin = (nsteps * wave) / kWaves, s_end = (nsteps * (wave + 1)) / kWaves;
  __shared__ float red[kWaves][4][4][64];

  for (int tg = 0; tg < nrows; tg += 16) {
    const bool valid = tg + r16 < nrows;
    const int pos = row0 + tg + r16;
    int arow = 0;
    if (valid) arow = (p.act_by_token && !p.dense) ? p.pairs[pos] / p.k : pos;
    f32x4 acc[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int st = s_begin; st < s_end; ++st) {
      const int k0 = st * 128;
      bf16x8 B[4];
      load_b(p, arow, valid, k0, g, B);
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        bf16x8 A[4];
        if constexpr (GEMM1) {
          const int row = n0 + 16 * (t & 1) + r16;
          if (t < 2) load_a<WF>(p, p.wa, p.sa, e, row, k0, g, A);
          else load_a<WF>(p, p.wb, p.sb, e, row, k0, g, A);
        } else {
          load_a<WF>(p, p.wa, p.sa, e, n0 + 16 * t + r16, k0, g, A);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[i], B[i], acc[t], 0, 0, 0);
      }
    }
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int v = 0; v < 4; ++v) red[wave][t][v][lane] = acc[t][v];
    __syncthreads();
    if (wave == 0) {
      float sum[4][4];
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          float s = red[0][t][v][lane];
#pragma unroll
          for (int w = 1; w < kWaves; ++w) s = s + red[w][t][v][lane];
          sum[t][v] = s;
        }
      if constexpr (GEMM1) {
        float rwv = 1.0f;
        if (valid && !p.dense) rwv = p.rw[p.pairs[pos]];
        float h[2][4];
        float amax = 0.0f;
#pragma unroll
        for (int half = 0; half < 2; ++half)
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const float gv = round_bf16(sum[half][v]);
            const float uv = round_bf16(sum[2 + half][v]);
            h[half][v] = round_bf16(swiglu(gv, uv, rwv, !p.dense));
            amax = fmaxf(amax, fabsf(h[half][v]));
          }
        // the 32 rows of this QDQ block for token column r16 live in lanes r16 + 16 g, g = 0..3
        amax = fmaxf(amax, __shfl_xor(amax, 16, 64));
        amax = fmaxf(amax, __shfl_xor(amax, 32, 64));
        const int E8 = qdq_exponent(amax);
        const float inv = exp2_neg(E8);
        if (valid) {
#pragma unroll
          for (int half = 0; half < 2; ++half) {
            uint32_t packed = 0;
#pragma unroll
            for (int v = 0; v < 4; ++v) packed |= qdq_code(h[half][v], inv) << (8 * v);
            *reinterpret_cast<uint32_t*>(p.h_q + (size_t)pos * p.N + n0 + 16 * half + 4 * g) = packed;
          }
          if (g == 0) p.h_s[(size_t)pos * (p.N / 32) + n0 / 32] = uint8_t(E8 + 127);
        }
      } else {
        if (valid) {
          const int orow = p.dense ? pos : p.pairs[pos];
          uint16_t* o = p.out + (size_t)orow * p.N + n0 + 4 * g;
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            const uint32_t lo = uint32_t(f32_to_bf16_rne(sum[t][0])) | (uint32_t(f32_to_bf16_rne(sum[t][1])) << 16);
            const uint32_t hi = uint32_t(f32_to_bf16_rne(sum[t][2])) | (uint32_t(f32_to_bf16_rne(sum[t][3])) << 16);
            *reinterpret_cast<u32x2*>(o + 16 * t) = u32x2{lo, hi};
          }
        }
      }
    }
    __syncthreads();
  }
}

template <bool GEMM1>
static void launch_small(WeightFormat f, const GemmProblem& p, int max_active, hipStream_t s) {
  constexpr int NB = GEMM1 ? 32 : 64;
  dim3 grid(p.N / NB, p.dense ? 1 : max_active);
  switch (f) {
    case W_MXFP4: expert_gemm_small<W_MXFP4, GEMM1><<<grid, dim3(256), 0, s>>>(p); break;
    case W_FP8_BLOCK32: expert_gemm_small<W_FP8_BLOCK32, GEMM1><<<grid, dim3(256), 0, s>>>(p); break;
    case W_BF16: expert_gemm_small<W_BF16, GEMM1><<<grid, dim3(256), 0, s>>>(p); break;
  }
}

void launch_gemm1_small(WeightFormat f, const GemmProblem& p, int max_active, hipStream_t s) {
  launch_small<true>(f, p, max_active, s);
}

void launch_gemm2_small(WeightFormat f, const GemmProblem& p, int max_active, hipStream_t s) {
  launch_small<false>(f, p, max_active, s);
}

}  // namespace moe
