// Dense FP8 linear of the method's projection family (page "Native 1017 DSpark draft on the NVLink pair (N1-NATIVE)", section 4
// "Dense"): y = bf16(sum_k act_qdq(x) W) with W FP8 E4M3 [N, K] and one E8M0 scale per 32x32 block,
// the same numerics as the shared expert's w2 (section 2 "Quantized linear").
//
// Decode widths (M <= 64): the weights stream from HBM once through the block-scaled matrix cores, with
// the inner dimension split across blocks so that even N = 512 fills the chip. Block (c, z) owns 64
// weight rows (one 16-row fragment per wave) and the z-th run of 128-wide K steps; the M activation
// rows of that run (E4M3 codes and scales) and the two 32-row weight-scale rows are copied into LDS
// once (or, given the bf16 rows, QDQ'd straight into LDS by the block). The partial sums of the runs are added in ascending run order by a second kernel (fp32, then
// bf16 or fp32 out). Wider batches use the prefill-width grouped GEMM as a single expert.
//
// Operand layout (measured on gfx950): lane l = (row l % 16, group g = l / 16); an E4M3 operand holds K
// [16g, 16g + 16) and [64 + 16g, 64 + 16g + 16) of the step; lane l supplies the E8M0 scale of K block g
// of its row; the result (4g + v, l % 16) is accumulator v of lane l.
#include <algorithm>

#include "kernels.h"
#include "moe_device.h"
#include "route_device.h"

namespace moe {

// Per-32 E4M3 QDQ of every row of x [M, K] (K a multiple of 32): thread per 32-wide block.
__global__ __launch_bounds__(256) void qdq_rows_kernel(long long nblk, const uint16_t* __restrict__ x,
                                                       uint8_t* __restrict__ xq, uint8_t* __restrict__ xs) {
  for (long long b = (long long)blockIdx.x * 256 + threadIdx.x; b < nblk; b += (long long)gridDim.x * 256)
    qdq_block32(x + b * 32, xq + b * 32, xs + b);
}

void launch_qdq_rows(int M, int K, const uint16_t* x, uint8_t* xq, uint8_t* xs, hipStream_t s) {
  const long long nblk = (long long)M * (K / 32);
  const int grid = (int)std::min<long long>((nblk + 255) / 256, 4096);
  qdq_rows_kernel<<<dim3(grid), dim3(256), 0, s>>>(nblk, x, xq, xs);
}

namespace {

constexpr int kDenseInFlight = 1;       // K steps per weight register set (two sets take turns; 1 beat 2 and 4)
constexpr int kDenseWaitVmLgkm0 = 0x7 << 4;   // s_waitcnt vmcnt(0) expcnt(7) lgkmcnt(0)

// copy of a run of nbytes (a multiple of UNIT) straight into LDS by one wave
template <int UNIT>
__device__ __forceinline__ void dense_run(uint8_t* lds, const uint8_t* src, int nbytes, int lane) {
  for (int off = 0; off < nbytes; off += 64 * UNIT)
    if (off + UNIT * lane < nbytes) {
      const void* g = static_cast<const void*>(src + off + UNIT * lane);
      auto* l = (__attribute__((address_space(3))) void*)(lds + off);
      if constexpr (UNIT == 16) __builtin_amdgcn_global_load_lds(g, l, 16, 0, 0);
      else __builtin_amdgcn_global_load_lds(g, l, 4, 0, 0);
    }
}

}  // namespace

// Dynamic LDS: activation codes [M][S * 128], activation scales [M][S * 4], weight scales [2][S * 4]
// (S = steps of this run).
// TILED: w is the fragment-order copy ([N / 16][K / 64][64 lanes][16 bytes]: lane l of chunk q holds bytes
// 64 q + 16 (l / 16) .. + 15 of row 16 f + l % 16), so each weight load of a wave reads 1 KB of consecutive
// bytes instead of 64-byte pieces of 16 rows.
template <bool TILED>
__global__ __launch_bounds__(256) void fp8_linear_stream(int M, int N, int K, int steps_per_run,
                                                         const uint16_t* __restrict__ x,
                                                         const uint8_t* __restrict__ xq, const uint8_t* __restrict__ xs,
                                                         const uint8_t* __restrict__ w, const uint8_t* __restrict__ s,
                                                         float* __restrict__ part, uint16_t* __restrict__ y,
                                                         float* __restrict__ y32) {
  extern __shared__ __align__(16) uint8_t dyn[];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, r16 = lane & 15, g = lane >> 4;
  const int nk = K / 128, KB = K / 32;
  const int lo = blockIdx.y * steps_per_run, hi = min(nk, lo + steps_per_run), ns = hi - lo;
  if (ns <= 0) return;
  const int n0 = blockIdx.x * 64;
  uint8_t* xb = dyn;                                   // [M][steps_per_run * 128]
  uint8_t* xsb = xb + M * steps_per_run * 128;         // [M][steps_per_run * 4]
  uint8_t* wsb = xsb + M * steps_per_run * 4;          // [2][steps_per_run * 4]
  const int RL = steps_per_run * 128, SL = steps_per_run * 4;
  {
    int run = 0;
    auto mine = [&]() { return (run++ & 3) == wave; };
    if (x == nullptr) {   // QDQ'd rows given: copy this run's codes and scales
      for (int t = 0; t < M; ++t) {
        if (mine()) dense_run<16>(xb + t * RL, xq + (size_t)t * K + lo * 128, ns * 128, lane);
        if (mine()) dense_run<4>(xsb + t * SL, xs + (size_t)t * KB + lo * 4, ns * 4, lane);
      }
    }
    if (mine()) dense_run<4>(wsb, s + (size_t)(n0 / 32) * KB + lo * 4, ns * 4, lane);
    if (mine()) dense_run<4>(wsb + SL, s + (size_t)(n0 / 32 + 1) * KB + lo * 4, ns * 4, lane);
  }
  // the first weight steps are in flight while the activations are staged
  // lane's bytes of a step: wsrc + ks * kStepBytes (first 16) and + kHalf (second 16)
  constexpr int kStepBytes = TILED ? 2048 : 128, kHalf = TILED ? 1024 : 64;
  const uint8_t* wsrc = TILED ? w + (size_t)((n0 + 16 * wave) / 16) * (size_t)(K / 64) * 1024 + 16 * lane
                              : w + (size_t)(n0 + 16 * wave + r16) * K + 16 * g;
  const int nt = (M + 15) / 16;   // 16-token groups (the MFMA's B columns)
  f32x4 acc[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) acc[q] = f32x4{0.f, 0.f, 0.f, 0.f};
  // Weight loads: two register sets of U K steps take turns, so one set's loads are in flight while the
  // other's MFMAs run. Loads are never guarded by a condition (past the run's last step they re-read it),
  // and the sets are never copied into each other: either would make the compiler wait for every load in
  // flight before the first MFMA of a set, not just for that set's own.
  constexpr int U = kDenseInFlight;
  u32x4 PA[U], PB[U], QA[U], QB[U];
  auto load = [&](u32x4 (&RA)[U], u32x4 (&RB)[U], int j) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int ks = lo + min(j + u, ns - 1);
      // weight bytes are read once per call: non-temporal loads
      RA[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(wsrc + (size_t)ks * kStepBytes));
      RB[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(wsrc + (size_t)ks * kStepBytes + kHalf));
    }
  };
  load(PA, PB, 0);
  if (x != nullptr) {   // bf16 rows given: QDQ this run's 32-wide blocks straight into LDS (thread per block)
    const int nb = ns * 4;
    for (int i = threadIdx.x; i < M * nb; i += 256) {
      const int t = i / nb, j = i % nb;
      u32x4 q0, q1;
      const uint8_t sc = qdq_block32_regs(x + (size_t)t * K + lo * 128 + j * 32, q0, q1);
      *reinterpret_cast<u32x4*>(xb + t * RL + j * 32) = q0;
      *reinterpret_cast<u32x4*>(xb + t * RL + j * 32 + 16) = q1;
      xsb[t * SL + j] = sc;
    }
  }
  // staging done (the builtin wait, unlike one in asm, is seen by the compiler's wait placement), then meet
  __builtin_amdgcn_s_waitcnt(kDenseWaitVmLgkm0);
  __syncthreads();
  auto run = [&](const u32x4 (&RA)[U], const u32x4 (&RB)[U], int j0) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int j = j0 + u;
      if (j < ns) {
        const i32x8 Af = i32x8{(int)RA[u][0], (int)RA[u][1], (int)RA[u][2], (int)RA[u][3],
                               (int)RB[u][0], (int)RB[u][1], (int)RB[u][2], (int)RB[u][3]};
        const int sa = wsb[(wave >> 1) * SL + 4 * j + g];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          if (q < nt) {
            const int t = min(16 * q + r16, M - 1);   // columns past M repeat the last row (discarded)
            const u32x4 b0 = *reinterpret_cast<const u32x4*>(xb + t * RL + j * 128 + 16 * g);
            const u32x4 b1 = *reinterpret_cast<const u32x4*>(xb + t * RL + j * 128 + 64 + 16 * g);
            const i32x8 Bf = i32x8{(int)b0[0], (int)b0[1], (int)b0[2], (int)b0[3],
                                   (int)b1[0], (int)b1[1], (int)b1[2], (int)b1[3]};
            acc[q] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(Af, Bf, acc[q], 0, 0, 0, sa, 0,
                                                                     (int)xsb[t * SL + 4 * j + g]);
          }
        }
      }
    }
  };
  for (int j0 = 0; j0 < ns; j0 += 2 * U) {
    load(QA, QB, j0 + U);
    run(PA, PB, j0);
    load(PA, PB, j0 + 2 * U);
    run(QA, QB, j0 + U);
  }
  // lane: weight rows n0 + 16 wave + 4g .. + 3 of token 16 q + r16
  const int n = n0 + 16 * wave + 4 * g;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int t = 16 * q + r16;
    if (q < nt && t < M) {
      if (part != nullptr) {
        *reinterpret_cast<f32x4*>(part + ((size_t)blockIdx.y * M + t) * N + n) = acc[q];
      } else if (y32 != nullptr) {
        *reinterpret_cast<f32x4*>(y32 + (size_t)t * N + n) = acc[q];
      } else {
        const uint32_t a = uint32_t(f32_to_bf16_rne(acc[q][0])) | (uint32_t(f32_to_bf16_rne(acc[q][1])) << 16);
        const uint32_t b = uint32_t(f32_to_bf16_rne(acc[q][2])) | (uint32_t(f32_to_bf16_rne(acc[q][3])) << 16);
        *reinterpret_cast<u32x2*>(y + (size_t)t * N + n) = u32x2{a, b};
      }
    }
  }
}

// y = the runs' fp32 partial sums added in ascending run order, then bf16 (or fp32): 4 outputs per thread.
__global__ __launch_bounds__(256) void dense_reduce_kernel(long long n4, int runs, long long stride,
                                                           const float* __restrict__ part, uint16_t* __restrict__ y,
                                                           float* __restrict__ y32) {
  for (long long i = (long long)blockIdx.x * 256 + threadIdx.x; i < n4; i += (long long)gridDim.x * 256) {
    // eight runs' loads in flight at a time, added in ascending run order
    f32x4 a = *reinterpret_cast<const f32x4*>(part + 4 * i);
    for (int z0 = 1; z0 < runs; z0 += 8) {
      f32x4 b[8];
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (z0 + u < runs) b[u] = *reinterpret_cast<const f32x4*>(part + (z0 + u) * stride + 4 * i);
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (z0 + u < runs) a = f32x4{a[0] + b[u][0], a[1] + b[u][1], a[2] + b[u][2], a[3] + b[u][3]};
    }
    if (y32 != nullptr) {
      *reinterpret_cast<f32x4*>(y32 + 4 * i) = a;
    } else {
      const uint32_t lo = uint32_t(f32_to_bf16_rne(a[0])) | (uint32_t(f32_to_bf16_rne(a[1])) << 16);
      const uint32_t hi = uint32_t(f32_to_bf16_rne(a[2])) | (uint32_t(f32_to_bf16_rne(a[3])) << 16);
      *reinterpret_cast<u32x2*>(y + 4 * i) = u32x2{lo, hi};
    }
  }
}

void launch_fp8_linear_stream(int M, int N, int K, const uint16_t* x, const uint8_t* xq, const uint8_t* xs,
                              const uint8_t* w, bool w_tiled, const uint8_t* s, float* part, uint16_t* y, float* y32,
                              hipStream_t st) {
  const DensePlan pl = dense_plan(M, N, K);
  dim3 grid(N / 64, pl.runs);
  auto stream = [&](float* pp, uint16_t* yy, float* yy32) {
    if (w_tiled)
      fp8_linear_stream<true><<<grid, dim3(256), pl.lds, st>>>(M, N, K, pl.steps_per_run, x, xq, xs, w, s, pp, yy, yy32);
    else
      fp8_linear_stream<false><<<grid, dim3(256), pl.lds, st>>>(M, N, K, pl.steps_per_run, x, xq, xs, w, s, pp, yy,
                                                                yy32);
  };
  if (pl.runs > 1) {
    stream(part, nullptr, nullptr);
    const long long n4 = (long long)M * N / 4;
    const int rg = (int)std::min<long long>((n4 + 255) / 256, 4096);
    dense_reduce_kernel<<<dim3(rg), dim3(256), 0, st>>>(n4, pl.runs, (long long)M * N, part, y, y32);
  } else {
    stream(nullptr, y, y32);
  }
}

}  // namespace moe
