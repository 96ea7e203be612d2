// Grouped expert GEMMs for many rows per expert (prefill) on gfx950's block-scaled matrix cores.
//
// Math (DeepSeek-V4.1-Flash native-tensor page, section 2 "Quantized linear" and section 4 "Kernel
// contract"): per 32-wide K block the exact products of E4M3 activation codes and E2M1 (or E4M3) weight
// codes are summed, multiplied by the two E8M0 scales and accumulated in fp32; g and u are rounded to
// bf16, clamped, h = rw * silu(g) * u in fp32, bf16, QDQ per 32 along I; y = bf16(h_hat w2^T).
//
// v_mfma_scale_f32_16x16x128_f8f6f4 computes exactly that per instruction, and the stored MX bytes
// and scale bytes feed it as they are (no decode, no conversion instructions). Operand layout of the
// instruction on gfx950 (measured with one-hot probes): lane l supplies operand row l % 16; with
// g = l / 16, an E2M1 operand holds the 32 consecutive K values [32g, 32g + 32) (16 bytes), an E4M3
// operand holds K [16g, 16g + 16) in its first 16 bytes and K [64 + 16g, 64 + 16g + 16) in its last
// 16; in both cases lane l supplies the E8M0 scale of K block g ([32g, 32g + 32)) of its row. The
// result element (row 4g + v of A, row l % 16 of B) is accumulator v of lane l.
//
// Tiling. A block computes 128 weight rows x 128 rows of one expert (GEMM1: the same 64 output columns
// of w1 and w3, so the SwiGLU pairs sit in one lane). Four waves in a 2 x 2 layout each own 64 weight
// rows x 64 rows (16 MFMAs per 128-wide K step, 64 fp32 accumulators per lane). K steps of 128 are
// staged through double-buffered LDS with padded row strides (conflict-free 128-bit reads). The rows of
// an expert are its sorted positions offsets[e] .. offsets[e+1]; GEMM1 gathers the activation row of
// each position's token, GEMM2 reads the QDQ'd h rows in sorted order and scatters y to the pair's slot
// row. The (expert, row tile) of a block comes from a tile list built on the device from the expert
// counts (tile_map_kernel): launch geometry depends only on (dims, M); blocks past the list exit.
#include "kernels.h"
#include "moe_device.h"

namespace moe {

namespace {

constexpr int kTileN = 128;   // weight rows per block
constexpr int kTileM = 128;   // activation rows per block
constexpr int kStepK = 128;   // K per stage (one MFMA K)
constexpr int kActStride = kStepK + 16;              // E4M3 activation row in LDS (bytes)
constexpr int kFmtFp8 = 0, kFmtFp4 = 4;              // operand formats of the scaled MFMA

template <int WF>
struct WTraits;
template <>
struct WTraits<W_MXFP4> {
  static constexpr int kRowBytes = kStepK / 2;       // packed bytes of one weight row per stage
  static constexpr int kStride = kRowBytes + 16;
  static constexpr int kFmt = kFmtFp4;
};
template <>
struct WTraits<W_FP8_BLOCK32> {
  static constexpr int kRowBytes = kStepK;
  static constexpr int kStride = kRowBytes + 16;
  static constexpr int kFmt = kFmtFp8;
};

template <int WF>
struct Smem {
  uint8_t w[2][kTileN][WTraits<WF>::kStride];
  uint8_t a[2][kTileM][kActStride];
  uint8_t ws[2][kTileN][4];   // E8M0 of the 4 K blocks of a stage, per weight row
  uint8_t as[2][kTileM][4];   // per activation row
};

}  // namespace

// Row-tile list of the grouped GEMMs: for every expert with rows, ceil(count / kTileM) tiles in
// ascending expert order. tile_e[y] = expert (-1 past the end), tile_r0[y] = first sorted position.
__global__ __launch_bounds__(256) void tile_map_kernel(int E, int max_tiles, const int32_t* __restrict__ offsets,
                                                       int32_t* __restrict__ tile_e, int32_t* __restrict__ tile_r0) {
  __shared__ int scan[256];
  const int e = threadIdx.x;
  int nt = 0, r0 = 0;
  if (e < E) {
    r0 = offsets[e];
    nt = (offsets[e + 1] - r0 + kTileM - 1) / kTileM;
  }
  scan[e] = nt;
  __syncthreads();
  for (int d = 1; d < 256; d <<= 1) {   // inclusive Hillis-Steele scan
    const int v = (e >= d) ? scan[e - d] : 0;
    __syncthreads();
    scan[e] += v;
    __syncthreads();
  }
  const int first = scan[e] - nt, total = scan[255];
  for (int i = 0; i < nt; ++i) {
    tile_e[first + i] = e;
    tile_r0[first + i] = r0 + i * kTileM;
  }
  for (int y = total + e; y < max_tiles; y += 256) tile_e[y] = -1;
}

template <int WF, bool GEMM1>
__global__ __launch_bounds__(256, 2) void expert_gemm_mfma(GemmProblem p, const int32_t* __restrict__ tile_e,
                                                           const int32_t* __restrict__ tile_r0) {
  using T = WTraits<WF>;
  __shared__ Smem<WF> sm;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int r16 = lane & 15, g = lane >> 4;
  const int wn = wave & 1, wm = wave >> 1;

  int e, row0, nrows;
  if (p.dense) {
    e = 0;
    row0 = blockIdx.y * kTileM;
    nrows = min(kTileM, p.M - row0);
    if (nrows <= 0) return;
  } else {
    e = tile_e[blockIdx.y];
    if (e < 0) return;
    row0 = tile_r0[blockIdx.y];
    nrows = min(kTileM, p.offsets[e + 1] - row0);
  }
  const int K = p.K;
  const int nk = K / kStepK;
  // weight rows of this block: GEMM1 rows 0..63 = w1 rows n0h..n0h+63, rows 64..127 = w3 rows n0h..;
  // GEMM2 rows 0..127 = w2 rows n0..n0+127
  const int n0 = blockIdx.x * (GEMM1 ? kTileN / 2 : kTileN);

  // ---- per-thread global load assignments ----------------------------------------------------
  // weights: kTileN rows x kRowBytes per stage in 16-byte chunks
  constexpr int kWChunks = T::kRowBytes / 16;                      // 4 (FP4) or 8 (FP8) per row
  constexpr int kWLoads = kTileN * kWChunks / 256;                 // 2 or 4 per thread
  const uint8_t* wsrc[kWLoads];
  int wdst_row[kWLoads], wdst_col[kWLoads];
#pragma unroll
  for (int i = 0; i < kWLoads; ++i) {
    const int c = tid + 256 * i;
    const int r = c / kWChunks, ch = c % kWChunks;
    int grow;
    const uint8_t* base;
    if (GEMM1) {
      grow = n0 + (r & 63);
      base = static_cast<const uint8_t*>(r < 64 ? p.wa : p.wb);
    } else {
      grow = n0 + r;
      base = static_cast<const uint8_t*>(p.wa);
    }
    const size_t row_bytes = (WF == W_MXFP4) ? (size_t)K / 2 : (size_t)K;
    wsrc[i] = base + (size_t)e * p.w_expert_stride + (size_t)grow * row_bytes + ch * 16;
    wdst_row[i] = r;
    wdst_col[i] = ch * 16;
  }
  // weight scales: one dword (4 K blocks) per weight row, threads 0..127
  const uint8_t* wssrc = nullptr;
  if (tid < kTileN) {
    const int r = tid;
    int grow;
    const uint8_t* base;
    if (GEMM1) {
      grow = n0 + (r & 63);
      base = r < 64 ? p.sa : p.sb;
    } else {
      grow = n0 + r;
      base = p.sa;
    }
    if (WF == W_MXFP4) wssrc = base + (size_t)e * p.s_expert_stride + (size_t)grow * (K / 32);
    else wssrc = base + (size_t)(grow / 32) * (K / 32);
  }
  // activations: kTileM rows x 128 bytes per stage = 8 chunks per row, 4 per thread
  const uint8_t* asrc[4];
  bool aval[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = (tid >> 3) + 32 * i, ch = tid & 7;
    aval[i] = r < nrows;
    int arow = 0;
    if (aval[i]) {
      const int pos = row0 + r;
      arow = (p.act_by_token && !p.dense) ? p.pairs[pos] / p.k : pos;
    }
    asrc[i] = p.act_q + (size_t)arow * K + ch * 16;
  }
  const uint8_t* assrc = nullptr;   // activation scales: threads 128..255, one dword per row
  bool asval = false;
  if (tid >= 128) {
    const int r = tid - 128;
    asval = r < nrows;
    int arow = 0;
    if (asval) {
      const int pos = row0 + r;
      arow = (p.act_by_token && !p.dense) ? p.pairs[pos] / p.k : pos;
    }
    assrc = p.act_s + (size_t)arow * (K / 32);
  }

  u32x4 wreg[kWLoads], areg[4];
  uint32_t sreg = 0;
  auto gload = [&](int ks) {
    const int kb = ks * kStepK;
#pragma unroll
    for (int i = 0; i < kWLoads; ++i)
      wreg[i] = *reinterpret_cast<const u32x4*>(wsrc[i] + (WF == W_MXFP4 ? kb / 2 : kb));
#pragma unroll
    for (int i = 0; i < 4; ++i)
      areg[i] = aval[i] ? *reinterpret_cast<const u32x4*>(asrc[i] + kb) : u32x4{0u, 0u, 0u, 0u};
    if (tid < kTileN) sreg = *reinterpret_cast<const uint32_t*>(wssrc + kb / 32);
    else sreg = asval ? *reinterpret_cast<const uint32_t*>(assrc + kb / 32) : 0x7F7F7F7Fu;
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < kWLoads; ++i)
      *reinterpret_cast<u32x4*>(&sm.w[buf][wdst_row[i]][wdst_col[i]]) = wreg[i];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      *reinterpret_cast<u32x4*>(&sm.a[buf][(tid >> 3) + 32 * i][(tid & 7) * 16]) = areg[i];
    if (tid < kTileN) *reinterpret_cast<uint32_t*>(&sm.ws[buf][tid][0]) = sreg;
    else *reinterpret_cast<uint32_t*>(&sm.as[buf][tid - 128][0]) = sreg;
  };

  // ---- main loop -------------------------------------------------------------------------------
  f32x4 acc[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};

  // LDS rows of this wave's four A fragments
  int arow_l[4];
#pragma unroll
  for (int a = 0; a < 4; ++a) arow_l[a] = GEMM1 ? (64 * (a >> 1) + 32 * wn + 16 * (a & 1)) : (64 * wn + 16 * a);

  gload(0);
  lstore(0);
  __syncthreads();
  for (int ks = 0; ks < nk; ++ks) {
    const int buf = ks & 1;
    if (ks + 1 < nk) gload(ks + 1);
    i32x8 Af[4], Bf[4];
    int asc[4], bsc[4];
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const uint8_t* src = &sm.w[buf][arow_l[a] + r16][0];
      if constexpr (WF == W_MXFP4) {
        const u32x4 v = *reinterpret_cast<const u32x4*>(src + 16 * g);
        Af[a] = i32x8{(int)v[0], (int)v[1], (int)v[2], (int)v[3], 0, 0, 0, 0};
      } else {
        const u32x4 v0 = *reinterpret_cast<const u32x4*>(src + 16 * g);
        const u32x4 v1 = *reinterpret_cast<const u32x4*>(src + 64 + 16 * g);
        Af[a] = i32x8{(int)v0[0], (int)v0[1], (int)v0[2], (int)v0[3], (int)v1[0], (int)v1[1], (int)v1[2], (int)v1[3]};
      }
      asc[a] = sm.ws[buf][arow_l[a] + r16][g];
    }
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const uint8_t* src = &sm.a[buf][64 * wm + 16 * b + r16][0];
      const u32x4 v0 = *reinterpret_cast<const u32x4*>(src + 16 * g);
      const u32x4 v1 = *reinterpret_cast<const u32x4*>(src + 64 + 16 * g);
      Bf[b] = i32x8{(int)v0[0], (int)v0[1], (int)v0[2], (int)v0[3], (int)v1[0], (int)v1[1], (int)v1[2], (int)v1[3]};
      bsc[b] = sm.as[buf][64 * wm + 16 * b + r16][g];
    }
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int b = 0; b < 4; ++b)
        acc[a][b] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(Af[a], Bf[b], acc[a][b], T::kFmt, kFmtFp8, 0,
                                                                     asc[a], 0, bsc[b]);
    if (ks + 1 < nk) lstore(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue: lane holds weight rows 4g..4g+3 of each A fragment for row (token) r16 of each B
  // fragment ----------------------------------------------------------------------------------------
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    const int tt = 64 * wm + 16 * b + r16;
    const bool valid = tt < nrows;
    const int pos = row0 + tt;
    if constexpr (GEMM1) {
      float rwv = 1.0f;
      if (valid && !p.dense) rwv = p.rw[p.pairs[pos]];
      float h[2][4];
      float amax = 0.0f;
#pragma unroll
      for (int half = 0; half < 2; ++half)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const float gv = round_bf16(acc[half][b][v]);
          const float uv = round_bf16(acc[2 + half][b][v]);
          h[half][v] = round_bf16(swiglu(gv, uv, rwv, !p.dense));
          amax = fmaxf(amax, fabsf(h[half][v]));
        }
      // the 32 columns of this QDQ block for row r16 live in lanes r16 + 16 g, g = 0..3
      amax = fmaxf(amax, __shfl_xor(amax, 16, 64));
      amax = fmaxf(amax, __shfl_xor(amax, 32, 64));
      const int E8 = qdq_exponent(amax);
      const float inv = exp2_neg(E8);
      if (valid) {
        const int col0 = n0 + 32 * wn;
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          uint32_t packed = 0;
#pragma unroll
          for (int v = 0; v < 4; ++v) packed |= qdq_code(h[half][v], inv) << (8 * v);
          *reinterpret_cast<uint32_t*>(p.h_q + (size_t)pos * p.N + col0 + 16 * half + 4 * g) = packed;
        }
        if (g == 0) p.h_s[(size_t)pos * (p.N / 32) + col0 / 32] = uint8_t(E8 + 127);
      }
    } else {
      if (valid) {
        const int orow = p.dense ? pos : p.pairs[pos];
        uint16_t* o = p.out + (size_t)orow * p.N + n0 + 64 * wn + 4 * g;
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          const uint32_t lo = uint32_t(f32_to_bf16_rne(acc[a][b][0])) | (uint32_t(f32_to_bf16_rne(acc[a][b][1])) << 16);
          const uint32_t hi = uint32_t(f32_to_bf16_rne(acc[a][b][2])) | (uint32_t(f32_to_bf16_rne(acc[a][b][3])) << 16);
          *reinterpret_cast<u32x2*>(o + 16 * a) = u32x2{lo, hi};
        }
      }
    }
  }
}

int mfma_max_tiles(int P, int E) { return (P + kTileM - 1) / kTileM + (P < E ? P : E); }

void launch_tile_map(int E, int max_tiles, const int32_t* offsets, int32_t* tile_e, int32_t* tile_r0, hipStream_t s) {
  tile_map_kernel<<<dim3(1), dim3(256), 0, s>>>(E, max_tiles, offsets, tile_e, tile_r0);
}

template <bool GEMM1>
static void launch_mfma(WeightFormat f, const GemmProblem& p, int max_tiles, const int32_t* tile_e,
                        const int32_t* tile_r0, hipStream_t s) {
  const int cols = GEMM1 ? p.N / (kTileN / 2) : p.N / kTileN;
  const int rows = p.dense ? (p.M + kTileM - 1) / kTileM : max_tiles;
  dim3 grid(cols, rows);
  switch (f) {
    case W_MXFP4: expert_gemm_mfma<W_MXFP4, GEMM1><<<grid, dim3(256), 0, s>>>(p, tile_e, tile_r0); break;
    case W_FP8_BLOCK32: expert_gemm_mfma<W_FP8_BLOCK32, GEMM1><<<grid, dim3(256), 0, s>>>(p, tile_e, tile_r0); break;
    default: break;   // the bf16 arm has no block-scaled form; the caller never asks for it here
  }
}

void launch_gemm1_mfma(WeightFormat f, const GemmProblem& p, int max_tiles, const int32_t* tile_e,
                       const int32_t* tile_r0, hipStream_t s) {
  launch_mfma<true>(f, p, max_tiles, tile_e, tile_r0, s);
}

void launch_gemm2_mfma(WeightFormat f, const GemmProblem& p, int max_tiles, const int32_t* tile_e,
                       const int32_t* tile_r0, hipStream_t s) {
  launch_mfma<false>(f, p, max_tiles, tile_e, tile_r0, s);
}

}  // namespace moe
