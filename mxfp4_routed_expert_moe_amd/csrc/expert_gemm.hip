// Expert GEMMs at decode width (few rows per expert) on gfx950.
//
// Math (page "Native 1017 DSpark draft on the NVLink pair (N1-NATIVE)", section 4 "Kernel contract", per (t, j) with
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
          amax = fmaxf(amax, swiglu_bf16x4(sum[half], sum[2 + half], rwv, !p.dense, h[half]));
        // the 32 rows of this QDQ block for token column r16 live in lanes r16 + 16 g, g = 0..3
        amax = fmaxf(amax, __shfl_xor(amax, 16, 64));
        amax = fmaxf(amax, __shfl_xor(amax, 32, 64));
        const int E8 = qdq_exponent(amax);
        const float inv = exp2_neg(E8);
        if (valid) {
#pragma unroll
          for (int half = 0; half < 2; ++half) {
            const uint32_t packed = qdq_code4(h[half][0], h[half][1], h[half][2], h[half][3], inv);
            *reinterpret_cast<uint32_t*>(p.h_q + (size_t)pos * p.N + n0 + 16 * half + 4 * g) = packed;
          }
          if (g == 0) p.h_s[(size_t)pos * (p.N / 32) + n0 / 32] = uint8_t(E8 + 127);
        }
      } else {
        if (valid) {
          const int orow = p.dense ? pos : (p.out_rows ? p.out_rows[pos] : p.pairs[pos]);
          if (p.out_f32) {
            float* o = p.out_f32 + (size_t)orow * p.N + n0 + 4 * g;
#pragma unroll
            for (int t = 0; t < 4; ++t)
              *reinterpret_cast<f32x4*>(o + 16 * t) = f32x4{sum[t][0], sum[t][1], sum[t][2], sum[t][3]};
          } else {
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


// =================================================================================================
// Decode-width GEMMs on the block-scaled matrix cores (MXFP4 or FP8 weights, E4M3 activations).
//
// The weights stream from HBM once and feed v_mfma_scale_f32_16x16x128_f8f6f4 as stored: no
// conversion instructions. A block owns one expert and four 16-row weight fragments (GEMM1: w1 and w3
// rows of the same 32 output columns, so the SwiGLU pairs and the 32-column QDQ block meet in one
// block; GEMM2: 64 rows of w2). Wave f streams fragment f over the whole inner dimension (16 rows, each
// a contiguous run of bytes), prefetching kStreamU steps ahead, so the only vector-memory traffic in
// the loop is the wave's own weight rows. The E8M0 scales of the 64 rows and up to 4 activation rows
// of the expert (E4M3 codes and scales) are staged in LDS at the start; experts with more rows are
// processed kRows (4 or 8) rows at a time. GEMM1's w1 and w3 fragments meet in LDS for the SwiGLU/QDQ epilogue, which
// two waves share; GEMM2's waves store their own rows.
//
// Operand layout (measured on gfx950): lane l = (row l % 16, group g = l / 16); an E2M1 operand
// holds K [32g, 32g + 32) of the 128-wide step (one stored 16-byte MX block); an E4M3 operand holds
// K [16g, 16g + 16) and [64 + 16g, 64 + 16g + 16); lane l supplies the E8M0 scale of K block g of its
// row (the low byte of the scale operand).
// =================================================================================================
namespace {

// activation rows staged in LDS per pass (the MFMA's 16 columns hold up to 16): 4 while the experts average
// fewer than three rows, which keeps the staging small enough for four blocks per CU; 8 above, so that experts
// with 5 .. 8 rows stream their weights once instead of twice (full-size layer, 8 against 4 rows: M = 64 494 ->
// 452 us, M = 128 720 -> 569 us, M = 256 1234 -> 881 us; M = 48 401 -> 404 us, hence the threshold)
constexpr int kStreamRowsFew = 4, kStreamRowsMany = 8;
// s_waitcnt immediate (gfx9 encoding: vmcnt bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8) for
// vmcnt(0) lgkmcnt(0), expcnt left at its maximum (not waited for)
constexpr int kWaitVmLgkm0 = 0x7 << 4;

// Direct global -> LDS copy of a run of nbytes (a multiple of UNIT = 16 or 4) by one wave: lane i moves
// UNIT bytes of every 64 * UNIT-byte piece (the copy lands at lds + off + i * UNIT). Every copy of the
// run is issued before any is waited for.
template <int UNIT>
__device__ __forceinline__ void stage_run(uint8_t* lds, const uint8_t* src, int nbytes, int lane) {
  static_assert(UNIT == 16 || UNIT == 4, "direct-to-LDS copies move 16 or 4 bytes per lane");
  for (int off = 0; off < nbytes; off += 64 * UNIT)
    if (off + UNIT * lane < nbytes) {
      const void* g = static_cast<const void*>(src + off + UNIT * lane);
      auto* l = (__attribute__((address_space(3))) void*)(lds + off);
      if constexpr (UNIT == 16) __builtin_amdgcn_global_load_lds(g, l, 16, 0, 0);
      else __builtin_amdgcn_global_load_lds(g, l, 4, 0, 0);
    }
}

template <int WF>
struct StreamA;   // one 16-row x 128-K weight fragment of a lane
// Weight bytes are read once per call, so the loads carry the non-temporal hint (streamed through the
// caches without displacing other lines): decode_m8 GEMM1 83.4 -> 72.8 us, layer 142.8 -> 128.6 us, old
// and new builds in alternating processes on one box.
// `src` is the lane's first 16 bytes and KSTRIDE the bytes between consecutive 128-wide K steps: 64
// along a stored row, 1024 between the fragments of the fragment-order copy. (A compile-time stride
// keeps the prefetch addresses immediate offsets; computed at run time, the compiler waited for every
// load in flight before issuing the next.)
template <>
struct StreamA<W_MXFP4> {
  u32x4 d;
  template <int KSTRIDE>
  __device__ __forceinline__ void load(const uint8_t* src, int ks) {
    d = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src + ks * KSTRIDE));
  }
  __device__ __forceinline__ i32x8 frag() const {
    return i32x8{(int)d[0], (int)d[1], (int)d[2], (int)d[3], 0, 0, 0, 0};
  }
  static constexpr int kFmt = 4;
};
template <>
struct StreamA<W_FP8_BLOCK32> {
  u32x4 d0, d1;
  template <int KSTRIDE>
  __device__ __forceinline__ void load(const uint8_t* src, int ks) {
    d0 = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src + ks * KSTRIDE));
    d1 = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src + ks * KSTRIDE + 64));
  }
  __device__ __forceinline__ i32x8 frag() const {
    return i32x8{(int)d0[0], (int)d0[1], (int)d0[2], (int)d0[3], (int)d1[0], (int)d1[1], (int)d1[2], (int)d1[3]};
  }
  static constexpr int kFmt = 0;
};

}  // namespace

// Dynamic LDS: scales [64][K/32], activation codes [kRows][K], activation scales [kRows][K/32], then the
// [4 waves][64 lanes] fp32x4 exchange of the fragments and the [2][16] amax halves (GEMM1).
// kStreamU: K steps per weight register set (two sets alternate). 4 by default; 3 where the step count is a
// multiple of 6 and not of 8 (w2 at I = 2304: 18 steps), so that no batch of loads re-reads past the last step
// (decode layer: GEMM2 40.8 -> 39.4 us, interleaved A/B on one box).
template <int WF, bool GEMM1, bool TILED, int kStreamU = 4, int kRows = kStreamRowsFew>
__global__ __launch_bounds__(256) void expert_gemm_stream(GemmProblem p) {
  static_assert(!TILED || WF == W_MXFP4, "the fragment-order copy holds MXFP4 codes");
  extern __shared__ __align__(16) uint8_t dyn[];
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
  const int K = p.K, nk = K / 128, KB = K / 32;
  uint8_t* sc = dyn;                                   // [64][KB]
  uint8_t* xb = sc + 64 * KB;                          // [kRows][K]
  uint8_t* xsb = xb + kRows * K;                       // [kRows][KB]
  f32x4* xch = reinterpret_cast<f32x4*>(dyn + ((64 * KB + kRows * (K + KB) + 15) & ~15));   // [4][64]
  float* amx = reinterpret_cast<float*>(xch + 4 * 64);                                            // [2][16]
  // block rows: GEMM1 output columns c0 .. c0 + 31 (LDS rows 0..31 = w1, 32..63 = w3); GEMM2 rows c0 .. c0 + 63
  const int c0 = GEMM1 ? blockIdx.x * 32 : blockIdx.x * 64;
  auto grow_of = [&](int r) { return GEMM1 ? c0 + (r & 31) : c0 + r; };
  const size_t wrow_bytes = (WF == W_MXFP4) ? (size_t)K / 2 : (size_t)K;
  const int lrow = (GEMM1 ? 32 * (wave >> 1) + 16 * (wave & 1) : 16 * wave) + r16;   // this wave's fragment
  // the lane's weight bytes of K step 0 and the stride between steps: along its stored row (16 bytes of
  // K block g), or, in the fragment-order copy, lane's 16 bytes of fragment (row / 16, step)
  const uint8_t* wmat = static_cast<const uint8_t*>((GEMM1 && wave >= 2) ? p.wb : p.wa) + (size_t)e * p.w_expert_stride;
  constexpr int kKStride = TILED ? 1024 : (WF == W_MXFP4 ? 64 : 128);
  const uint8_t* wsrc = TILED ? wmat + ((size_t)(grow_of(lrow) >> 4) * nk) * 1024 + 16 * lane
                              : wmat + (size_t)grow_of(lrow) * wrow_bytes + 16 * g;

  for (int tg = 0; tg < nrows; tg += kRows) {
    const int n = min(kRows, nrows - tg);
    // staging: runs of contiguous bytes copied straight into LDS, one run per wave in turn, all in
    // flight together. Run 0/1: the weight scales (MXFP4: the 64 rows' E8M0 bytes, two K-byte runs for
    // GEMM1 (w1, w3 rows) or one 2K-byte run for GEMM2; FP8: the two 32-row blocks' scale rows). Then
    // the n activation rows and their scales. Staged rows past n are not written: the lanes that read
    // them produce output columns that the epilogue discards.
    {
      int run = 0;
      auto mine = [&]() { return (run++ & 3) == wave; };
      if (tg == 0) {
        if constexpr (WF == W_MXFP4) {
          const uint8_t* s1 = p.sa + (size_t)e * p.s_expert_stride + (size_t)c0 * KB;
          if (GEMM1) {
            if (mine()) stage_run<16>(sc, s1, 32 * KB, lane);
            if (mine()) stage_run<16>(sc + 32 * KB, p.sb + (size_t)e * p.s_expert_stride + (size_t)c0 * KB, 32 * KB, lane);
          } else {
            if (mine()) stage_run<16>(sc, s1, 64 * KB, lane);
          }
        } else {   // 32 x 32 blocks: one scale row per 32 weight rows
          if (mine()) stage_run<4>(sc, p.sa + (size_t)(c0 / 32) * KB, KB, lane);
          if (mine()) stage_run<4>(sc + KB, (GEMM1 ? p.sb + (size_t)(c0 / 32) * KB : p.sa + (size_t)(c0 / 32 + 1) * KB), KB, lane);
        }
      }
      for (int t = 0; t < n; ++t) {
        const int pos = row0 + tg + t;
        const int arow = (p.act_by_token && !p.dense) ? p.pairs[pos] / p.k : pos;
        if (mine()) stage_run<16>(xb + t * K, p.act_q + (size_t)arow * K, K, lane);
        if (mine()) stage_run<4>(xsb + t * KB, p.act_s + (size_t)arow * KB, KB, lane);
      }
    }
    // the first weight batch (in bounds for any nk: short K repeats the last step)
    // two register sets in turn (no copies between them): while the MFMAs run on one set's kStreamU steps,
    // the other set's loads are in flight.
    StreamA<WF> A[kStreamU], Bs[kStreamU];
#pragma unroll
    for (int u = 0; u < kStreamU; ++u) A[u].template load<kKStride>(wsrc, min(u, nk - 1));
    // every copy of this wave has landed in LDS (vmcnt counts the LDS-bound loads too); then meet. The
    // wait is the builtin, not inline asm, so that the compiler knows the copies are done: otherwise it
    // counts them as outstanding, and with loads of two kinds in flight it waits for all of them (vmcnt(0))
    // before every use of a weight register, leaving only one batch of steps in flight.
    __builtin_amdgcn_s_waitcnt(kWaitVmLgkm0);
    __builtin_amdgcn_s_barrier();
    const int bt = r16 & (kRows - 1);   // lanes past the staged rows compute a staged row (discarded)
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    auto run = [&](const StreamA<WF> (&R)[kStreamU], int ks0) {
#pragma unroll
      for (int u = 0; u < kStreamU; ++u) {
        const int ks = ks0 + u;
        if (ks < nk) {
          const u32x4 b0 = *reinterpret_cast<const u32x4*>(xb + bt * K + ks * 128 + 16 * g);
          const u32x4 b1 = *reinterpret_cast<const u32x4*>(xb + bt * K + ks * 128 + 64 + 16 * g);
          const i32x8 B = i32x8{(int)b0[0], (int)b0[1], (int)b0[2], (int)b0[3], (int)b1[0], (int)b1[1], (int)b1[2],
                                (int)b1[3]};
          acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(R[u].frag(), B, acc, StreamA<WF>::kFmt, 0, 0,
                                                                 (int)sc[(WF == W_MXFP4 ? lrow : lrow >> 5) * KB + 4 * ks + g], 0,
                                                                 (int)xsb[bt * KB + 4 * ks + g]);
        }
      }
    };
    // The loads are never conditional: with a guarded load the compiler no longer knows how many loads
    // are in flight and waits for all of them before each MFMA. Steps past the last re-read it (in
    // bounds, unused). Measured choice: on the fragment-order copy every batch is issued, also the one
    // after the last step; on the stored layout (GEMM2: 18 steps) the loop leaves before a batch that
    // has no step.
    for (int ks0 = 0; ks0 < nk; ks0 += 2 * kStreamU) {
      if constexpr (!TILED) {
        if (ks0 + kStreamU >= nk) {
          run(A, ks0);
          break;
        }
      }
#pragma unroll
      for (int u = 0; u < kStreamU; ++u) Bs[u].template load<kKStride>(wsrc, min(ks0 + kStreamU + u, nk - 1));
      run(A, ks0);
      if constexpr (!TILED) {
        if (ks0 + 2 * kStreamU >= nk) {
          run(Bs, ks0 + kStreamU);
          break;
        }
      }
#pragma unroll
      for (int u = 0; u < kStreamU; ++u) A[u].template load<kKStride>(wsrc, min(ks0 + 2 * kStreamU + u, nk - 1));
      run(Bs, ks0 + kStreamU);
    }
    // epilogue (lane: weight rows 4g..4g+3 of its fragment, activation row r16)
    const bool valid = r16 < n;
    const int pos = row0 + tg + r16;
    if constexpr (GEMM1) {
      // waves 0 and 1 each finish 16 of the block's 32 output columns: g from their own w1 fragment, u from
      // the w3 fragment of wave + 2 (through LDS); the amax of the 32-column QDQ block meets in LDS
      xch[wave * 64 + lane] = acc;
      __syncthreads();
      float h[4];
      if (wave < 2) {
        const f32x4 gf = xch[wave * 64 + lane], uf = xch[(wave + 2) * 64 + lane];
        float rwv = 1.0f;
        if (valid && !p.dense) rwv = p.rw[p.pairs[pos]];
        float amax = swiglu_bf16x4(gf, uf, rwv, !p.dense, h);
        // this wave's 16 columns of row r16 live in lanes r16 + 16 g, g = 0..3
        amax = fmaxf(amax, __shfl_xor(amax, 16, 64));
        amax = fmaxf(amax, __shfl_xor(amax, 32, 64));
        if (g == 0) amx[wave * 16 + r16] = amax;
      }
      __syncthreads();
      if (wave < 2) {
        const int E8 = qdq_exponent(fmaxf(amx[r16], amx[16 + r16]));
        const float inv = exp2_neg(E8);
        if (valid) {
          *reinterpret_cast<uint32_t*>(p.h_q + (size_t)pos * p.N + c0 + 16 * wave + 4 * g) =
              qdq_code4(h[0], h[1], h[2], h[3], inv);
          if (wave == 0 && g == 0) p.h_s[(size_t)pos * (p.N / 32) + c0 / 32] = uint8_t(E8 + 127);
        }
      }
    } else {
      // each wave holds the whole inner dimension of its 16 rows: it stores them itself
      if (valid) {
        const int orow = p.dense ? pos : (p.out_rows ? p.out_rows[pos] : p.pairs[pos]);
        if (p.out_f32) {
          *reinterpret_cast<f32x4*>(p.out_f32 + (size_t)orow * p.N + c0 + 16 * wave + 4 * g) = acc;
        } else {
          const uint32_t lo = uint32_t(f32_to_bf16_rne(acc[0])) | (uint32_t(f32_to_bf16_rne(acc[1])) << 16);
          const uint32_t hi = uint32_t(f32_to_bf16_rne(acc[2])) | (uint32_t(f32_to_bf16_rne(acc[3])) << 16);
          *reinterpret_cast<u32x2*>(p.out + (size_t)orow * p.N + c0 + 16 * wave + 4 * g) = u32x2{lo, hi};
        }
      }
    }
    __syncthreads();   // staging and exchange buffers are reused by the next row group
  }
}

size_t stream_lds_bytes(int K, int rows) {
  const int KB = K / 32;
  return (size_t)((64 * KB + rows * (K + KB) + 15) & ~15) + 4 * 64 * sizeof(f32x4) + 32 * sizeof(float);
}

// Rows per pass: a function of (M, k, E) only, so launch geometry never depends on routed data. The per-row
// arithmetic (the same MFMAs over the same K steps) does not depend on it, so outputs are identical either way.
// The 8-row staging is used only while it fits 64 KB of LDS (K up to about 6,000; the contract's H = 5120 takes
// 56.7 KB); larger K keeps 4 rows.
static int stream_rows(const GemmProblem& p) {
  if (stream_lds_bytes(p.K, kStreamRowsMany) > 65536) return kStreamRowsFew;
  if (p.dense) return p.M > kStreamRowsFew ? kStreamRowsMany : kStreamRowsFew;
  return (long long)p.M * p.k >= 3LL * p.num_experts ? kStreamRowsMany : kStreamRowsFew;
}

template <int WF, bool GEMM1, bool TILED, int U>
static void launch_stream_rows(const GemmProblem& p, dim3 grid, hipStream_t s) {
  const int rows = stream_rows(p);
  const size_t lds = stream_lds_bytes(p.K, rows);
  if (rows == kStreamRowsMany)
    expert_gemm_stream<WF, GEMM1, TILED, U, kStreamRowsMany><<<grid, dim3(256), lds, s>>>(p);
  else
    expert_gemm_stream<WF, GEMM1, TILED, U, kStreamRowsFew><<<grid, dim3(256), lds, s>>>(p);
}

template <bool GEMM1>
static void launch_stream(WeightFormat f, const GemmProblem& p, int max_active, hipStream_t s) {
  dim3 grid(GEMM1 ? p.N / 32 : p.N / 64, p.dense ? 1 : max_active);
  switch (f) {
    case W_MXFP4:
      if (p.w_tiled && (p.K / 128) % 6 == 0 && (p.K / 128) % 8 != 0)
        launch_stream_rows<W_MXFP4, GEMM1, true, 3>(p, grid, s);
      else if (p.w_tiled) launch_stream_rows<W_MXFP4, GEMM1, true, 4>(p, grid, s);
      else launch_stream_rows<W_MXFP4, GEMM1, false, 4>(p, grid, s);
      break;
    case W_FP8_BLOCK32: launch_stream_rows<W_FP8_BLOCK32, GEMM1, false, 4>(p, grid, s); break;
    default: break;   // the bf16 arm uses launch_small
  }
}

void launch_gemm1_stream(WeightFormat f, const GemmProblem& p, int max_active, hipStream_t s) {
  launch_stream<true>(f, p, max_active, s);
}

void launch_gemm2_stream(WeightFormat f, const GemmProblem& p, int max_active, hipStream_t s) {
  launch_stream<false>(f, p, max_active, s);
}

}  // namespace moe
