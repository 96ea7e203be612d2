// Grouped expert GEMMs of the decoded-BF16 arm at prefill widths, on gfx950's bf16 matrix cores.
//
// Math (page "Native 1017 DSpark draft on the NVLink pair (N1-NATIVE)", section 4 "Kernel contract", the
// expanded-weight form): the weights hold exactly code * 2^(b-127) in bf16, and a QDQ'd activation
// code * 2^(s-127) is exact in bf16 as well, so every product is exact in fp32 and the arm sums the same
// terms as the packed arm; only the order of the fp32 additions differs. g, u -> bf16 -> clamped SwiGLU
// times rw -> bf16 -> QDQ per 32 along I -> h; y = bf16(h_hat w2^T).
//
// v_mfma_f32_16x16x32_bf16 (operand layout measured on gfx950): lane l supplies row l % 16 of A and of B
// with the inputs 8 (l / 16) .. + 7 of the 32-wide step; result (row 4 (l / 16) + v of A, row l % 16 of B)
// is accumulator v of lane l.
//
// Tiling: the work list, tile list and XCD-aware block order of the block-scaled kernels; a block is four
// waves over 128 activation rows of one expert. GEMM1: wave w holds w1 rows n0 + 32 w .. + 31 (A fragments
// 0, 1) and the same rows of w3 (fragments 2, 3), so a SwiGLU pair and a 32-column QDQ block meet in one
// lane (128 output columns per block); GEMM2: wave w holds w2 rows n0 + 64 w .. + 63 (256 per block).
// Each weight row is used by one wave only, so the weights go straight from memory into registers, kAhead
// 64-wide K steps ahead of the step computed (bf16 rows: 128 contiguous bytes per row and step). The
// activation tile (E4M3 codes and E8M0 scales, gathered by token for GEMM1) is loaded into registers the
// same number of steps ahead, widened to bf16 with the hardware converter (exact) and written to a
// two-slot LDS ring that the four waves read; 16-byte chunks are XOR-swizzled so the 16 rows of a
// fragment read distinct banks.
#include "kernels.h"
#include "moe_device.h"

namespace moe {

namespace {

constexpr int kBfRows = 128;   // activation rows per block: the row tiles of the work list
constexpr int kBfK = 64;       // K per step: one 128-byte bf16 row segment
constexpr int kAhead = 1;      // steps of weight and activation loads in flight beyond the one computed (1, 2 and
                               // 3 measured within 3 % of each other at 8192 tokens; 1 the fastest)
constexpr int kSets = kAhead + 1;

struct BfStage {
  uint16_t a[kBfRows * kBfK];   // bf16 activations, 128-byte rows of 8 swizzled 16-byte chunks
};

// physical chunk = logical chunk ^ key(row): rows of one parity fill one half of the 64 banks and the 8
// rows of a parity take 8 distinct chunks, so 16 consecutive rows read distinct banks
__device__ __forceinline__ int bf_key(int r) { return ((r >> 1) ^ (4 * (r & 1))) & 7; }

struct ActRegs {
  u32x4 c0, c1;   // 32 E4M3 codes of one row (one 32-wide K block of the step)
  uint32_t sc;    // its E8M0 byte
};

// This wave's LDS accesses are done, then meet the other waves. (__syncthreads() would also wait for every
// outstanding global load, the steps loaded ahead included.)
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

template <bool B>
struct Tag { static constexpr bool value = B; };

template <int N>
struct Slot { static constexpr int value = N; };

}  // namespace

template <bool GEMM1>
__global__ __launch_bounds__(256, 1) void expert_gemm_bf16(GemmProblem p, const int32_t* __restrict__ tile_e,
                                                           const int32_t* __restrict__ tile_r0,
                                                           const int32_t* __restrict__ info) {
  __shared__ __align__(16) BfStage ring[2];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int r16 = lane & 15, g = lane >> 4;
  const int C = GEMM1 ? p.N / 128 : (p.N + 255) / 256;   // column tiles
  const int RT = info[0];                                  // row tiles
  const int W = RT * C;
  const int L = blockIdx.x;
  if (L >= W) return;
  int w = L / 8;
  for (int i = 0; i < L % 8; ++i) w += (W - i + 7) / 8;   // blocks of the XCDs before this one
  const int ew = tile_e[w / C];
  const int first = info[1 + ew], nt = info[1 + p.num_experts + ew];
  const int local = w - first * C;
  const int cx = local / nt, ty = first + local % nt;
  const int e = tile_e[ty];
  const int row0 = tile_r0[ty];
  const int nrows = min(kBfRows, p.offsets[e + 1] - row0);
  const int K = p.K, nk = K / kBfK;
  const int n0 = cx * (GEMM1 ? 128 : 256);

  // ---- weight sources: fragment a, lane (r16, g): row grow(a), inputs 64 s + 32 j + 8 g .. + 7 ----------
  auto grow = [&](int a) {
    if constexpr (GEMM1) return n0 + 32 * wave + 16 * (a & 1) + r16;
    else return min(n0 + 64 * wave + 16 * a + r16, p.N - 1);   // rows past N repeat row N - 1, never stored
  };
  const uint16_t* wbase_a = static_cast<const uint16_t*>(p.wa) + (size_t)e * p.w_expert_stride;
  const uint16_t* wbase_b = GEMM1 ? static_cast<const uint16_t*>(p.wb) + (size_t)e * p.w_expert_stride : wbase_a;
  uint32_t woff[4];   // element offsets within the expert matrix (N * K <= 2^31)
#pragma unroll
  for (int a = 0; a < 4; ++a) woff[a] = (uint32_t)grow(a) * (uint32_t)K + 8u * g;
  auto load_w = [&](u32x4 (&A)[4][2], int s) {
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int j = 0; j < 2; ++j)
        A[a][j] = *reinterpret_cast<const u32x4*>(((GEMM1 && a >= 2) ? wbase_b : wbase_a) + woff[a] + kBfK * s + 32 * j);
  };

  // ---- activation sources: thread -> tile row tid / 2, K block tid % 2 of each step -----------------
  const int at = tid >> 1, ah = tid & 1;
  const uint8_t* acode;
  const uint8_t* ascale;
  {
    const int pos = row0 + (at < nrows ? at : 0);   // rows past the tile repeat row 0 (never stored)
    const int arow = p.act_by_token ? p.pairs[pos] / p.k : pos;
    acode = p.act_q + (size_t)arow * K + 32 * ah;
    ascale = p.act_s + (size_t)arow * (K / 32) + ah;
  }
  auto load_act = [&](ActRegs& R, int s) {
    R.c0 = *reinterpret_cast<const u32x4*>(acode + kBfK * s);
    R.c1 = *reinterpret_cast<const u32x4*>(acode + kBfK * s + 16);
    R.sc = ascale[2 * s];
  };
  // widen the 32 codes to bf16 (code * scale, exact) into logical chunks 4 ah .. 4 ah + 3 of row `at`
  auto act_to_lds = [&](const ActRegs& R, BfStage& st) {
    const float scale = e8m0_to_f32(R.sc);
    const int key = bf_key(at);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t d0 = i < 2 ? R.c0[2 * i] : R.c1[2 * i - 4];
      const uint32_t d1 = i < 2 ? R.c0[2 * i + 1] : R.c1[2 * i - 3];
      const u32x4 v = u32x4{fp8x2_to_bf16x2<false>(d0, scale), fp8x2_to_bf16x2<true>(d0, scale),
                            fp8x2_to_bf16x2<false>(d1, scale), fp8x2_to_bf16x2<true>(d1, scale)};
      *reinterpret_cast<u32x4*>(&st.a[at * kBfK + 8 * ((4 * ah + i) ^ key)]) = v;
    }
  };

  const int nbv = min(8, (nrows + 15) / 16);   // B fragments that hold a row of the tile
  f32x4 acc[4][8];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 8; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](const u32x4 (&A)[4][2], const BfStage& st, auto part) {
    constexpr bool PART = decltype(part)::value;
#pragma unroll
    for (int b = 0; b < 8; ++b) {
      if (!PART || b < nbv) {
        const int t = 16 * b + r16, key = bf_key(t);
        const u32x4 b0 = *reinterpret_cast<const u32x4*>(&st.a[t * kBfK + 8 * (g ^ key)]);
        const u32x4 b1 = *reinterpret_cast<const u32x4*>(&st.a[t * kBfK + 8 * ((4 + g) ^ key)]);
#pragma unroll
        for (int a = 0; a < 4; ++a)
          acc[a][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, A[a][0]),
                                                             __builtin_bit_cast(bf16x8, b0), acc[a][b], 0, 0, 0);
#pragma unroll
        for (int a = 0; a < 4; ++a)
          acc[a][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, A[a][1]),
                                                             __builtin_bit_cast(bf16x8, b1), acc[a][b], 0, 0, 0);
      }
    }
    // schedule: the two LDS reads of fragment b, then its eight MFMAs
#pragma unroll
    for (int b = 0; b < 8; ++b) {
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
    }
  };

  // Register sets rotate over kSets steps: step s computes with set s % kSets, converts the activations of
  // step s + 1 into LDS slot (s + 1) % 2, then loads step s + kSets into set s % kSets. The compiler's wait
  // counts follow the loads into each register, so only the loads of step s + 1 are waited for.
  u32x4 Wr[kSets][4][2];
  ActRegs Ar[kSets];
  load_w(Wr[0], 0);
  load_act(Ar[0], 0);
#pragma unroll
  for (int j = 1; j < kSets; ++j)
    if (j < nk) {
      load_w(Wr[j], j);
      load_act(Ar[j], j);
    }
  act_to_lds(Ar[0], ring[0]);
  lds_barrier();

  auto step = [&](auto slot, int s, auto part) {
    constexpr int J = decltype(slot)::value;
    if (s >= nk) return;
    compute(Wr[J], ring[s & 1], part);
    if (s + 1 < nk) act_to_lds(Ar[(J + 1) % kSets], ring[(s + 1) & 1]);
    if (s + kSets < nk) {
      load_w(Wr[J], s + kSets);
      load_act(Ar[J], s + kSets);
    }
    // slot (s + 1) % 2 is written; every wave is past its reads of slot s % 2 before the next write to it
    lds_barrier();
  };
  auto kloop = [&](auto part) {
    for (int s0 = 0; s0 < nk; s0 += kSets) {
      step(Slot<0>{}, s0, part);
      step(Slot<1>{}, s0 + 1, part);
      if constexpr (kSets > 2) step(Slot<2>{}, s0 + 2, part);
      if constexpr (kSets > 3) step(Slot<3>{}, s0 + 3, part);
    }
  };
  static_assert(kSets >= 2 && kSets <= 4, "the loop body names up to four register sets");
  if (nbv == 8) kloop(Tag<false>{});
  else kloop(Tag<true>{});

  // ---- epilogue: lane holds weight rows 4g..4g+3 of each A fragment for activation row r16 of each B
  // fragment ------------------------------------------------------------------------------------------
#pragma unroll
  for (int b = 0; b < 8; ++b) {
    const int tt = 16 * b + r16;
    const bool valid = tt < nrows;
    const int pos = row0 + tt;
    if constexpr (GEMM1) {
      float rwv = 1.0f;
      if (valid) rwv = p.rw[p.pairs[pos]];
      float h[2][4];
      float amax = 0.0f;
#pragma unroll
      for (int half = 0; half < 2; ++half)
        amax = fmaxf(amax, swiglu_bf16x4(acc[half][b], acc[2 + half][b], rwv, true, h[half]));
      // the 32 columns of this QDQ block for row r16 live in lanes r16 + 16 g, g = 0..3
      amax = fmaxf(amax, __shfl_xor(amax, 16, 64));
      amax = fmaxf(amax, __shfl_xor(amax, 32, 64));
      const int E8 = qdq_exponent(amax);
      const float inv = exp2_neg(E8);
      if (valid) {
        const int col0 = n0 + 32 * wave;
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          const uint32_t packed = qdq_code4(h[half][0], h[half][1], h[half][2], h[half][3], inv);
          *reinterpret_cast<uint32_t*>(p.h_q + (size_t)pos * p.N + col0 + 16 * half + 4 * g) = packed;
        }
        if (g == 0) p.h_s[(size_t)pos * (p.N / 32) + col0 / 32] = uint8_t(E8 + 127);
      }
    } else {
      if (valid && n0 + 64 * wave < p.N) {
        const int orow = p.pairs[pos];
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          const int col = n0 + 64 * wave + 16 * a + 4 * g;
          if (p.out_f32) {
            *reinterpret_cast<f32x4*>(p.out_f32 + (size_t)orow * p.N + col) = acc[a][b];
          } else {
            const uint32_t lo = uint32_t(f32_to_bf16_rne(acc[a][b][0])) | (uint32_t(f32_to_bf16_rne(acc[a][b][1])) << 16);
            const uint32_t hi = uint32_t(f32_to_bf16_rne(acc[a][b][2])) | (uint32_t(f32_to_bf16_rne(acc[a][b][3])) << 16);
            *reinterpret_cast<u32x2*>(p.out + (size_t)orow * p.N + col) = u32x2{lo, hi};
          }
        }
      }
    }
  }
}

void launch_gemm1_bf16(const GemmProblem& p, int max_tiles, const int32_t* tile_e, const int32_t* tile_r0,
                       const int32_t* info, hipStream_t s) {
  expert_gemm_bf16<true><<<dim3((p.N / 128) * max_tiles), dim3(256), 0, s>>>(p, tile_e, tile_r0, info);
}

void launch_gemm2_bf16(const GemmProblem& p, int max_tiles, const int32_t* tile_e, const int32_t* tile_r0,
                       const int32_t* info, hipStream_t s) {
  expert_gemm_bf16<false><<<dim3(((p.N + 255) / 256) * max_tiles), dim3(256), 0, s>>>(p, tile_e, tile_r0, info);
}

}  // namespace moe
