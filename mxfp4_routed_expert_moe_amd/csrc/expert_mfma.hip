// Grouped expert GEMMs for many rows per expert (prefill) on gfx950's block-scaled matrix cores.
//
// Math (page "Native 1017 DSpark draft on the NVLink pair (N1-NATIVE)", section 2 "Quantized linear" and section 4 "Kernel
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
// Tiling. A block computes 256 weight rows x 128 rows of one expert (GEMM1: the same 128 output columns
// of w1 and w3, so the SwiGLU pairs sit in one lane). Four waves in a 2 x 2 layout each own 128 weight
// rows x 64 rows (32 MFMAs per 128-wide K step, 128 fp32 accumulators per lane: the larger wave tile
// cuts LDS bytes per MFMA). K steps of 128 stream into an LDS ring by direct global-to-LDS copies, with
// XOR-swizzled 16-byte chunks (conflict-free fragment reads): for MXFP4 weights a two-stage ring and two
// blocks per CU, whose waves share the SIMDs and overlap each other's copies, fragment reads and MFMAs;
// for FP8 weights a three-stage ring issued two stages ahead, one block per CU. (MXFP4 weights in the
// fragment-order copy go to the second kernel below, which loads them straight into registers.) The rows of
// an expert are its sorted positions offsets[e] .. offsets[e+1]; GEMM1 gathers the activation row of
// each position's token, GEMM2 reads the QDQ'd h rows in sorted order and scatters y to the pair's slot
// row. The (expert, row tile) of a block comes from a tile list built on the device from the expert
// counts (tile_map_kernel): launch geometry depends only on (dims, M); blocks past the list exit.
#include "kernels.h"
#include "moe_device.h"

namespace moe {

namespace {

constexpr int kTileM = 128;   // activation rows per block (weight rows per block: the TN template argument)
constexpr int kStepK = 128;   // K per stage (one MFMA K)
constexpr int kFmtFp8 = 0, kFmtFp4 = 4;   // operand formats of the scaled MFMA

template <int WF>
struct WTraits;
template <>
struct WTraits<W_MXFP4> {
  static constexpr int kRowBytes = kStepK / 2;   // packed bytes of one weight row per stage
  static constexpr int kFmt = kFmtFp4;
};
template <>
struct WTraits<W_FP8_BLOCK32> {
  static constexpr int kRowBytes = kStepK;
  static constexpr int kFmt = kFmtFp8;
};

// XOR swizzle of the 16-byte chunks of an LDS row: physical chunk = logical chunk ^ key(row). The keys
// make the 16 rows of an MFMA fragment read distinct banks whether ds_read_b128 serves 8 or 16 lanes
// per cycle (checked exhaustively for both).
template <int RowBytes>
__device__ __forceinline__ int chunk_key(int r) {
  if constexpr (RowBytes == 64) return (r ^ (r >> 2)) & 3;
  else return ((r >> 1) ^ (4 * (r & 1))) & 7;
}

// One ring stage: weight rows, activation rows, and the E8M0 bytes of the stage's 4 K blocks per row.
template <int WF, int TN>
struct Stage {
  uint8_t w[TN * WTraits<WF>::kRowBytes];
  uint8_t a[kTileM * kStepK];
  uint8_t ws[TN * 4];
  uint8_t as[kTileM * 4];
};

// Asynchronous global -> LDS copy of 16 (or 4) bytes per lane: lane i of the wave writes at lds + i * bytes.
__device__ __forceinline__ void dma16(const uint8_t* g, uint8_t* lds_wave) {
  __builtin_amdgcn_global_load_lds(static_cast<const void*>(g), (__attribute__((address_space(3))) void*)lds_wave, 16,
                                   0, 0);
}
__device__ __forceinline__ void dma4(const uint8_t* g, uint8_t* lds_wave) {
  __builtin_amdgcn_global_load_lds(static_cast<const void*>(g), (__attribute__((address_space(3))) void*)lds_wave, 4,
                                   0, 0);
}

// Wait until at most N vector-memory loads of this wave are outstanding (older ones have landed, LDS
// DMA included), finish this wave's LDS reads, then meet the other waves. __syncthreads() would wait
// for every outstanding load and drain the ring.
template <int N>
__device__ __forceinline__ void ring_barrier() {
  if constexpr (N == 0) asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
  else if constexpr (N == 8) asm volatile("s_waitcnt vmcnt(8) lgkmcnt(0)\n\ts_barrier" ::: "memory");
  else if constexpr (N == 16) asm volatile("s_waitcnt vmcnt(16) lgkmcnt(0)\n\ts_barrier" ::: "memory");
  else if constexpr (N == 10) asm volatile("s_waitcnt vmcnt(10) lgkmcnt(0)\n\ts_barrier" ::: "memory");
  else if constexpr (N == 14) asm volatile("s_waitcnt vmcnt(14) lgkmcnt(0)\n\ts_barrier" ::: "memory");
  else if constexpr (N == 20) asm volatile("s_waitcnt vmcnt(20) lgkmcnt(0)\n\ts_barrier" ::: "memory");
  else if constexpr (N == 28) asm volatile("s_waitcnt vmcnt(28) lgkmcnt(0)\n\ts_barrier" ::: "memory");
  else static_assert(N == 0 || N == 8 || N == 16 || N == 10 || N == 14 || N == 20 || N == 28, "vmcnt immediate");
}

// Compile-time tags: every B fragment of the wave holds tile rows (kFull) or the tile may be partial.
struct FullTag { static constexpr bool value = false; };
struct PartialTag { static constexpr bool value = true; };
constexpr FullTag kFull{};
constexpr PartialTag kPartial{};

// Fragments of one stage held in registers (double-buffered across stages).
template <int WF>
struct Frags {
  u32x4 a0[8], a1[8];   // A fragment bytes (a1: second 16 bytes, E4M3 weights only)
  u32x4 b0[4], b1[4];
  int as[8], bs[4];
};

}  // namespace

// Row-tile list of the grouped GEMMs: for every expert with rows, ceil(count / kTileM) tiles in
// ascending expert order. tile_e[y] = expert (-1 past the end), tile_r0[y] = first sorted position;
// info[0] = number of tiles, info[1 + e] = first tile of expert e, info[1 + E + e] = its tile count.
__global__ __launch_bounds__(256) void tile_map_kernel(int E, int max_tiles, const int32_t* __restrict__ offsets,
                                                       int32_t* __restrict__ tile_e, int32_t* __restrict__ tile_r0,
                                                       int32_t* __restrict__ info) {
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
  if (e < E) {
    info[1 + e] = first;
    info[1 + E + e] = nt;
  }
  if (e == 0) info[0] = total;
}

// DMA instructions per wave per stage (TN / 64 waves): weights, 64 rows per wave (MXFP4: 4 of 16 rows x
// 64 B; FP8: 8 of 8 rows x 128 B), activations (128 rows over the waves, 8 rows x 128 B per instruction),
// weight scales (1 of 64 rows x 4 B), activation scales (1 of 128 / waves rows x 4 B).
template <int WF, int TN>
constexpr int loads_per_stage() { return (WF == W_MXFP4 ? 4 : 8) + 16 / (TN / 64) + 1 + 1; }

// Work order. The grid is one-dimensional: cols x (row tiles) blocks. Workgroups are dealt to the 8 XCDs
// round-robin (block L runs on XCD L % 8), and each XCD has its own L2. Block L is remapped to work item
// w so that every XCD gets one contiguous range of the work list, and the list runs expert by expert,
// column tile by column tile, row tile by row tile: the blocks an XCD runs together share a weight tile
// and the expert's activation rows stay in that XCD's L2.
// PAIR: 4 waves and a two-stage ring (67 KB of LDS), two blocks per CU; their waves share the SIMDs, and
// because the two blocks meet at their own barriers, one block's fragment reads and copies overlap the
// other's MFMAs. Otherwise one block per CU with a three-stage ring.
template <int WF, bool GEMM1, int TN, bool TILED, bool PAIR = false>
__global__ __launch_bounds__(TN, PAIR ? 2 : 1) void expert_gemm_mfma(GemmProblem p, const int32_t* __restrict__ tile_e,
                                                           const int32_t* __restrict__ tile_r0,
                                                           const int32_t* __restrict__ info) {
  static_assert(!TILED || WF == W_MXFP4, "the fragment-order copy holds MXFP4 codes");
  using T = WTraits<WF>;
  constexpr int kRB = T::kRowBytes, kCh = kRB / 16;
  constexpr int NW = TN / 64;                          // waves (each 128 weight rows x 64 activation rows)
  constexpr int kWInstr = 64 * kRB / 1024;             // weight DMA per wave per stage (4 or 8)
  constexpr int kWRows = 1024 / kRB;                   // rows per instruction (16 or 8)
  constexpr int kAInstr = 16 / NW;                     // activation DMA per wave per stage
  constexpr int kARows = kTileM / NW;                  // activation rows per wave
  constexpr int LPS = loads_per_stage<WF, TN>();
  constexpr int kStages = PAIR ? 2 : 3;   // LDS ring depth
  static_assert(!PAIR || TN == 256, "two blocks per CU: 4 waves");
  __shared__ __align__(16) Stage<WF, TN> ring[kStages];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int r16 = lane & 15, g = lane >> 4;
  const int wn = wave % (NW / 2), wm = wave / (NW / 2);

  const int C = GEMM1 ? p.N / (TN / 2) : (p.N + TN - 1) / TN;               // column tiles
  const int RT = p.dense ? (p.M + kTileM - 1) / kTileM : info[0];           // row tiles
  const int W = RT * C;
  const int L = blockIdx.x;
  if (L >= W) return;
  int w = L / 8;
  for (int i = 0; i < L % 8; ++i) w += (W - i + 7) / 8;   // blocks of the XCDs before this one
  int first, nt;
  if (p.dense) {
    first = 0;
    nt = RT;
  } else {
    const int ew = tile_e[w / C];
    first = info[1 + ew];
    nt = info[1 + p.num_experts + ew];
  }
  const int local = w - first * C;
  const int cx = local / nt, ty = first + local % nt;
  int e, row0, nrows;
  if (p.dense) {
    e = 0;
    row0 = ty * kTileM;
    nrows = min(kTileM, p.M - row0);
  } else {
    e = tile_e[ty];
    row0 = tile_r0[ty];
    nrows = min(kTileM, p.offsets[e + 1] - row0);
  }
  const int K = p.K, KB = K / 32;
  const int nk = K / kStepK;
  // weight rows of this block: GEMM1 LDS rows [0, TN/2) = w1 rows n0.., [TN/2, TN) = the same rows of w3;
  // GEMM2 LDS rows [0, TN) = w2 rows n0.. (rows past N repeat row N-1 and are never stored)
  const int n0 = cx * (GEMM1 ? TN / 2 : TN);
  const size_t wrow_bytes = (WF == W_MXFP4) ? (size_t)K / 2 : (size_t)K;
  auto grow_of = [&](int r) { return GEMM1 ? n0 + (r % (TN / 2)) : min(n0 + r, p.N - 1); };

  // ---- per-lane DMA sources (the stage offset is added per stage) ------------------------------
  // An MXFP4 instruction moves one 16-row fragment (16 rows x 64 B). In the fragment-order copy those
  // 1024 bytes are contiguous (lane l' = 16 c + row % 16 holds logical chunk c of the row), so the lanes
  // of one copy read one contiguous kilobyte, in the permuted order the LDS swizzle asks for.
  constexpr int wstage = TILED ? 1024 : (WF == W_MXFP4 ? kStepK / 2 : kStepK);   // bytes between stages
  const uint8_t* wsrc[kWInstr];
#pragma unroll
  for (int i = 0; i < kWInstr; ++i) {
    const int r = wave * 64 + i * kWRows + lane / kCh;             // LDS weight row
    const int gc = (lane % kCh) ^ chunk_key<kRB>(r);               // physical chunk lane%kCh holds logical gc
    const uint8_t* base = static_cast<const uint8_t*>((GEMM1 && r >= TN / 2) ? p.wb : p.wa) + (size_t)e * p.w_expert_stride;
    const int gr = grow_of(r);
    wsrc[i] = TILED ? base + ((size_t)(gr >> 4) * nk) * 1024 + (16 * gc + (gr & 15)) * 16
                    : base + (size_t)gr * wrow_bytes + gc * 16;
  }
  auto act_row = [&](int t) {   // activation row of LDS row t (rows past the tile repeat row 0)
    const int pos = row0 + (t < nrows ? t : 0);
    return (p.act_by_token && !p.dense) ? p.pairs[pos] / p.k : pos;
  };
  const uint8_t* asrc[kAInstr];
#pragma unroll
  for (int i = 0; i < kAInstr; ++i) {
    const int t = wave * kARows + i * 8 + lane / 8;
    const int gc = (lane % 8) ^ chunk_key<kStepK>(t);
    asrc[i] = p.act_q + (size_t)act_row(t) * K + gc * 16;
  }
  // weight scales: 4 bytes per row per stage; stage-major MXFP4 scales put a stage's rows side by side
  const uint8_t* wssrc;
  const size_t ws_step = (WF == W_MXFP4 && p.s_stage_major) ? (size_t)p.N * 4 : 4;
  {
    const int r = wave * 64 + lane;
    const uint8_t* sb = (GEMM1 && r >= TN / 2) ? p.sb : p.sa;
    if (WF == W_MXFP4)
      wssrc = sb + (size_t)e * p.s_expert_stride + (size_t)grow_of(r) * (p.s_stage_major ? 4 : KB);
    else
      wssrc = sb + (size_t)(grow_of(r) / 32) * KB;
  }
  // activation scales of the wave's kARows rows: 4 bytes per row per stage (stage-major: side by side)
  const uint8_t* assrc;
  size_t as_step = 4;
  if (p.a_stage_major) {
    const int t = wave * kARows + (lane % kARows);
    assrc = p.act_s + (size_t)(row0 + (t < nrows ? t : 0)) * 4;
    as_step = (size_t)p.M * p.k * 4;
  } else {
    assrc = p.act_s + (size_t)act_row(wave * kARows + (lane % kARows)) * KB;
  }
  auto issue = [&](int s) {
    Stage<WF, TN>& st = ring[s % kStages];
    const int k0 = s * kStepK;
#pragma unroll
    for (int i = 0; i < kWInstr; ++i)
      dma16(wsrc[i] + s * wstage, &st.w[(wave * 64 + i * kWRows) * kRB]);
#pragma unroll
    for (int i = 0; i < kAInstr; ++i) dma16(asrc[i] + k0, &st.a[(wave * kARows + i * 8) * kStepK]);
    dma4(wssrc + (size_t)s * ws_step, &st.ws[wave * 64 * 4]);
    if (lane < kARows) dma4(assrc + (size_t)s * as_step, &st.as[wave * kARows * 4]);
  };

  f32x4 acc[8][4];
#pragma unroll
  for (int a = 0; a < 8; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};
  // LDS rows of this wave's eight A fragments (weight rows) and four B fragments (activation rows)
  int arow_l[8], brow_l[4];
#pragma unroll
  for (int a = 0; a < 8; ++a)
    arow_l[a] = (GEMM1 ? ((TN / 2) * (a >> 2) + 64 * wn + 16 * (a & 3)) : (128 * wn + 16 * a)) + r16;
#pragma unroll
  for (int b = 0; b < 4; ++b) brow_l[b] = 64 * wm + 16 * b + r16;

  // B fragments of this wave that hold a row of the tile (the last tile of an expert is partial):
  // the others are neither read nor multiplied (wave-uniform)
  const int nbv = min(4, max(0, (nrows - 64 * wm + 15) / 16));
  // PART: the tile may be partial (checked per fragment); otherwise all four B fragments hold rows
  auto read_frags = [&](Frags<WF>& F, int s, auto part) {
    constexpr bool PART = decltype(part)::value;
    const Stage<WF, TN>& st = ring[s % kStages];
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      if (PART && b >= nbv) continue;
      const int t = brow_l[b];
      const int key = chunk_key<kStepK>(t);
      F.b0[b] = *reinterpret_cast<const u32x4*>(&st.a[t * kStepK + 16 * (g ^ key)]);
      F.b1[b] = *reinterpret_cast<const u32x4*>(&st.a[t * kStepK + 16 * ((4 + g) ^ key)]);
      F.bs[b] = st.as[t * 4 + g];
    }
    if (PART && nbv == 0) return;
#pragma unroll
    for (int a = 0; a < 8; ++a) {
      const int r = arow_l[a];
      const int key = chunk_key<kRB>(r);
      F.a0[a] = *reinterpret_cast<const u32x4*>(&st.w[r * kRB + 16 * (g ^ key)]);
      if constexpr (WF == W_FP8_BLOCK32) F.a1[a] = *reinterpret_cast<const u32x4*>(&st.w[r * kRB + 16 * ((4 + g) ^ key)]);
      F.as[a] = st.ws[r * 4 + g];
    }
  };
  auto mfmas = [&](const Frags<WF>& F, auto part) {
    constexpr bool PART = decltype(part)::value;
#pragma unroll
    for (int a = 0; a < 8; ++a) {
      i32x8 Af;
      if constexpr (WF == W_MXFP4)
        Af = i32x8{(int)F.a0[a][0], (int)F.a0[a][1], (int)F.a0[a][2], (int)F.a0[a][3], 0, 0, 0, 0};
      else
        Af = i32x8{(int)F.a0[a][0], (int)F.a0[a][1], (int)F.a0[a][2], (int)F.a0[a][3],
                   (int)F.a1[a][0], (int)F.a1[a][1], (int)F.a1[a][2], (int)F.a1[a][3]};
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        if (PART && b >= nbv) continue;
        const i32x8 Bf = i32x8{(int)F.b0[b][0], (int)F.b0[b][1], (int)F.b0[b][2], (int)F.b0[b][3],
                               (int)F.b1[b][0], (int)F.b1[b][1], (int)F.b1[b][2], (int)F.b1[b][3]};
        acc[a][b] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(Af, Bf, acc[a][b], T::kFmt, kFmtFp8, 0, F.as[a],
                                                                     0, F.bs[b]);
      }
    }
  };
  // one pipelined step: stage s + 1 has landed; refill the slot of stage s; MFMAs of stage s (registers
  // `cur`) interleaved with the LDS reads of stage s + 1 (registers `nxt`)
  auto step = [&](Frags<WF>& cur, Frags<WF>& nxt, int s) {
    if (s + 2 < nk) ring_barrier<LPS>();
    else ring_barrier<0>();
    if (s + 3 < nk) issue(s + 3);
    mfmas(cur, kFull);
    read_frags(nxt, s + 1, kFull);
    // scheduling: one LDS read after each MFMA (the reads do not depend on the MFMAs)
#pragma unroll
    for (int i = 0; i < (WF == W_MXFP4 ? 28 : 32); ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
  };

  if constexpr (NW == 4 && !PAIR) {
    // one wave per SIMD: fragments double-buffered in registers, LDS reads of stage s + 1 interleaved
    // with the MFMAs of stage s
    Frags<WF> F0, F1;
    issue(0);
    if (nk > 1) issue(1);
    if (nk > 2) issue(2);
    if (nk > 2) ring_barrier<2 * LPS>();   // stage 0 landed (stages 1, 2 in flight)
    else if (nk > 1) ring_barrier<LPS>();
    else ring_barrier<0>();
    read_frags(F0, 0, kFull);
    int s = 0;
    for (; s + 2 < nk; s += 2) {   // pairs of steps keep the two register sets static
      step(F0, F1, s);
      step(F1, F0, s + 1);
    }
    if (s + 1 < nk) {
      step(F0, F1, s);
      mfmas(F1, kFull);
    } else {
      mfmas(F0, kFull);
    }
  } else {
    // two waves per SIMD cover each other's LDS latency: one fragment set (fits 256 registers)
    // (a partial tile, the last one of an expert, runs its own copy of the loop that skips the empty
    // B fragments; full tiles run a copy without the checks)
    // (two-stage ring: stage s + 1 is issued at step s, so each wait is for everything in flight)
    Frags<WF> F;
    constexpr int D = kStages - 1;   // stages in flight ahead of the one computed
    issue(0);
    if (D > 1 && nk > 1) issue(1);
    auto kloop = [&](auto part) {
      for (int s = 0; s < nk; ++s) {
        if (D > 1 && s + 1 < nk) ring_barrier<LPS>();   // stage s landed (stage s + 1 may still be in flight)
        else ring_barrier<0>();
        if (s + D < nk) issue(s + D);           // into the slot computed at s - 1: every wave is past it
        read_frags(F, s, part);
        mfmas(F, part);
      }
    };
    if (nbv == 4) kloop(kFull);
    else kloop(kPartial);
  }

  // ---- epilogue: lane holds weight rows 4g..4g+3 of each A fragment for activation row r16 of each B
  // fragment -------------------------------------------------------------------------------------------
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    const int tt = 64 * wm + 16 * b + r16;
    const bool valid = tt < nrows;
    const int pos = row0 + tt;
    if constexpr (GEMM1) {
      float rwv = 1.0f;
      if (valid && !p.dense) rwv = p.rw[p.pairs[pos]];
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {   // two 32-column QDQ blocks: fragments (2qb, 2qb+1) of w1 with those of w3
        float h[2][4];
        float amax = 0.0f;
#pragma unroll
        for (int half = 0; half < 2; ++half)
          amax = fmaxf(amax, swiglu_bf16x4(acc[2 * qb + half][b], acc[4 + 2 * qb + half][b], rwv, !p.dense, h[half]));
        // the 32 columns of this QDQ block for row r16 live in lanes r16 + 16 g, g = 0..3
        amax = fmaxf(amax, __shfl_xor(amax, 16, 64));
        amax = fmaxf(amax, __shfl_xor(amax, 32, 64));
        const int E8 = qdq_exponent(amax);
        const float inv = exp2_neg(E8);
        if (valid) {
          const int col0 = n0 + 64 * wn + 32 * qb;
#pragma unroll
          for (int half = 0; half < 2; ++half) {
            const uint32_t packed = qdq_code4(h[half][0], h[half][1], h[half][2], h[half][3], inv);
            *reinterpret_cast<uint32_t*>(p.h_q + (size_t)pos * p.N + col0 + 16 * half + 4 * g) = packed;
          }
          if (g == 0) {
            const size_t at = p.h_s_stage_major
                                  ? ((size_t)(col0 / 128) * p.M * p.k + pos) * 4 + (col0 / 32) % 4
                                  : (size_t)pos * (p.N / 32) + col0 / 32;
            p.h_s[at] = uint8_t(E8 + 127);
          }
        }
      }
    } else {
      if (valid && n0 + 128 * wn < p.N) {
        const int orow = p.dense ? pos : p.pairs[pos];
        if (p.out_f32) {
          float* o = p.out_f32 + (size_t)orow * p.N + n0 + 128 * wn + 4 * g;
#pragma unroll
          for (int a = 0; a < 8; ++a) *reinterpret_cast<f32x4*>(o + 16 * a) = acc[a][b];
        } else {
          uint16_t* o = p.out + (size_t)orow * p.N + n0 + 128 * wn + 4 * g;
#pragma unroll
          for (int a = 0; a < 8; ++a) {
            const uint32_t lo = uint32_t(f32_to_bf16_rne(acc[a][b][0])) | (uint32_t(f32_to_bf16_rne(acc[a][b][1])) << 16);
            const uint32_t hi = uint32_t(f32_to_bf16_rne(acc[a][b][2])) | (uint32_t(f32_to_bf16_rne(acc[a][b][3])) << 16);
            *reinterpret_cast<u32x2*>(o + 16 * a) = u32x2{lo, hi};
          }
        }
      }
    }
  }
}

// =================================================================================================
// MXFP4 variant with the weights streamed straight into registers. Each weight row is used by exactly
// one wave (wave tile: 64 weight rows x the block's 128 activation rows), so the weights need no LDS:
// every lane loads its own 16-byte MX blocks (one per 16-row fragment per 128-wide K step), as the
// MFMA's A operand wants them. Only the activation tile (128 rows x 128 E4M3 bytes per step, shared by
// the four waves) and the E8M0 bytes of the step go through a three-slot LDS ring of direct copies,
// 17.5 KB per slot, so two blocks fit on a CU: one block's epilogue overlaps the other's matrix work.
// GEMM1: wave w holds w1 rows n0 + 32 w .. + 31 (fragments 0, 1) and the same rows of w3 (fragments 2, 3),
// so a SwiGLU pair and a 32-column QDQ block meet in one lane; the block covers 128 output columns.
// GEMM2: wave w holds w2 rows n0 + 64 w .. + 63; the block covers 256 output columns.
// =================================================================================================
namespace {

constexpr int kDaStages = 3;
struct DaStage {
  uint8_t a[kTileM * kStepK];   // activation codes, 128-byte rows, chunks swizzled
  uint8_t ws[256 * 4];          // weight scales, row 64 w + 16 a + r16 of fragment a of wave w
  uint8_t as[kTileM * 4];       // activation scales
};

}  // namespace

template <bool GEMM1, bool TILED>
__global__ __launch_bounds__(256, 2) void expert_gemm_mfma_da(GemmProblem p, const int32_t* __restrict__ tile_e,
                                                              const int32_t* __restrict__ tile_r0,
                                                              const int32_t* __restrict__ info) {
  __shared__ __align__(16) DaStage ring[kDaStages];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int r16 = lane & 15, g = lane >> 4;
  const int C = GEMM1 ? p.N / 128 : (p.N + 255) / 256;                     // column tiles
  const int RT = info[0];                                                   // row tiles
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
  const int nrows = min(kTileM, p.offsets[e + 1] - row0);
  const int K = p.K, KB = K / 32, nk = K / kStepK;
  const int n0 = cx * (GEMM1 ? 128 : 256);
  // global row of fragment a (0..3), row r of this wave
  auto grow = [&](int a, int r) {
    if constexpr (GEMM1) return n0 + 32 * wave + 16 * (a & 1) + r;
    else return min(n0 + 64 * wave + 16 * a + r, p.N - 1);
  };
  // weight rows: a wave-uniform base per matrix plus a 32-bit lane offset per fragment (an expert
  // matrix is N * K / 2 < 2^31 bytes)
  const uint8_t* wbase_a = static_cast<const uint8_t*>(p.wa) + (size_t)e * p.w_expert_stride;
  const uint8_t* wbase_b = GEMM1 ? static_cast<const uint8_t*>(p.wb) + (size_t)e * p.w_expert_stride : wbase_a;
  // (fragment-order copy: lane's 16 bytes of fragment (row / 16, step), 1024 bytes between steps;
  // rows past N repeat the last fragment, whose outputs are never stored)
  uint32_t aoff[4];
  constexpr int astage = TILED ? 1024 : kStepK / 2;
#pragma unroll
  for (int a = 0; a < 4; ++a)
    aoff[a] = TILED ? (uint32_t)(min(grow(a, 0), p.N - 16) >> 4) * (uint32_t)nk * 1024u + 16u * lane
                    : (uint32_t)grow(a, r16) * (uint32_t)(K / 2) + 16u * g;
  // per-stage copies: activation rows (4 of 8 rows x 128 B per wave), weight scales (the wave's 64 rows,
  // 4 bytes each), activation scales (32 rows per wave, 4 bytes each)
  auto act_row = [&](int t) {
    const int pos = row0 + (t < nrows ? t : 0);
    return (p.act_by_token && !p.dense) ? p.pairs[pos] / p.k : pos;
  };
  const uint8_t* asrc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int t = wave * 32 + i * 8 + lane / 8;
    const int gc = (lane % 8) ^ chunk_key<kStepK>(t);
    asrc[i] = p.act_q + (size_t)act_row(t) * K + gc * 16;
  }
  const size_t ws_step = p.s_stage_major ? (size_t)p.N * 4 : 4;
  const uint8_t* wssrc;
  {
    const int a = lane >> 4;
    const uint8_t* sb = (GEMM1 && a >= 2) ? p.sb : p.sa;
    wssrc = sb + (size_t)e * p.s_expert_stride + (size_t)grow(a, r16) * (p.s_stage_major ? 4 : KB);
  }
  const uint8_t* assrc;
  size_t as_step = 4;
  {
    const int t = wave * 32 + (lane & 31);
    if (p.a_stage_major) {
      assrc = p.act_s + (size_t)(row0 + (t < nrows ? t : 0)) * 4;
      as_step = (size_t)p.M * p.k * 4;
    } else {
      assrc = p.act_s + (size_t)act_row(t) * KB;
    }
  }
  auto issue_lds = [&](int s) {
    DaStage& st = ring[s % kDaStages];
    const int k0 = s * kStepK;
#pragma unroll
    for (int i = 0; i < 4; ++i) dma16(asrc[i] + k0, &st.a[(wave * 32 + i * 8) * kStepK]);
    dma4(wssrc + (size_t)s * ws_step, &st.ws[wave * 64 * 4]);
    if (lane < 32) dma4(assrc + (size_t)s * as_step, &st.as[wave * 32 * 4]);
  };
  auto load_a = [&](u32x4 (&A)[4], int s) {
#pragma unroll
    for (int a = 0; a < 4; ++a)
      A[a] = *reinterpret_cast<const u32x4*>(((GEMM1 && a >= 2) ? wbase_b : wbase_a) + aoff[a] + s * astage);
  };

  // B fragments of this wave's 128 rows that hold a row of the tile (the last tile of an expert is partial)
  const int nbv = min(8, (nrows + 15) / 16);
  f32x4 acc[4][8];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 8; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](const u32x4 (&A)[4], int s, auto part) {
    constexpr bool PART = decltype(part)::value;
    const DaStage& st = ring[s % kDaStages];
    int sa[4];
#pragma unroll
    for (int a = 0; a < 4; ++a) sa[a] = st.ws[(wave * 64 + 16 * a + r16) * 4 + g];
    i32x8 Af[4];
#pragma unroll
    for (int a = 0; a < 4; ++a) Af[a] = i32x8{(int)A[a][0], (int)A[a][1], (int)A[a][2], (int)A[a][3], 0, 0, 0, 0};
#pragma unroll
    for (int b = 0; b < 8; ++b) {
      if (!PART || b < nbv) {
        const int t = 16 * b + r16;
        const int key = chunk_key<kStepK>(t);
        const u32x4 b0 = *reinterpret_cast<const u32x4*>(&st.a[t * kStepK + 16 * (g ^ key)]);
        const u32x4 b1 = *reinterpret_cast<const u32x4*>(&st.a[t * kStepK + 16 * ((4 + g) ^ key)]);
        const int sb = st.as[t * 4 + g];
        const i32x8 Bf = i32x8{(int)b0[0], (int)b0[1], (int)b0[2], (int)b0[3], (int)b1[0], (int)b1[1], (int)b1[2],
                               (int)b1[3]};
#pragma unroll
        for (int a = 0; a < 4; ++a)
          acc[a][b] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(Af[a], Bf, acc[a][b], kFmtFp4, kFmtFp8, 0,
                                                                       sa[a], 0, sb);
      }
    }
    // schedule: the three LDS reads of fragment b, then its four MFMAs (keeps one B fragment live)
#pragma unroll
    for (int b = 0; b < 8; ++b) {
      __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
    }
  };
  // Issue order: at step s the weight blocks of step s + 1 (4 loads into registers), then the LDS copies
  // of step s + 2 (6: 4 activation, 1 weight-scale, 1 activation-scale), then the MFMAs of step s. So
  // before step s only the copies of step s + 1 may still be in flight: vmcnt(6) (0 near the end).
  auto wait_stage = [&](int s) {
    if (s + 1 < nk) asm volatile("s_waitcnt vmcnt(6) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    else asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
  };
  u32x4 A0[4], A1[4];
  issue_lds(0);
  load_a(A0, 0);
  if (nk > 1) issue_lds(1);
  // (the last, partial row tile of an expert runs a copy of the loop that skips its empty 16-row
  // activation fragments; full tiles run a copy without the checks)
  auto kloop = [&](auto part) {
    for (int s = 0; s < nk; ++s) {
      wait_stage(s);
      if (s + 1 < nk) load_a(A1, s + 1);
      if (s + 2 < nk) issue_lds(s + 2);
      compute(A0, s, part);
#pragma unroll
      for (int a = 0; a < 4; ++a) A0[a] = A1[a];
    }
  };  if (nbv == 8) kloop(kFull);
  else kloop(kPartial);

  // ---- epilogue: lane holds weight rows 4g..4g+3 of each A fragment for activation row r16 of each B
  // fragment
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
        if (g == 0) {
          const size_t at = p.h_s_stage_major ? ((size_t)(col0 / 128) * p.M * p.k + pos) * 4 + (col0 / 32) % 4
                                              : (size_t)pos * (p.N / 32) + col0 / 32;
          p.h_s[at] = uint8_t(E8 + 127);
        }
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

// One block per 64 rows of one matrix: the rows' scale bytes go through LDS (coalesced dword reads
// along the rows, coalesced dword writes along the stage-major rows).
__global__ __launch_bounds__(256) void scales_stage_major_kernel(int N, int KB, const uint8_t* __restrict__ s,
                                                                 uint8_t* __restrict__ S) {
  __shared__ uint32_t t[64][65];
  const int q4 = KB / 4;   // stages (dwords per row), at most 64
  const int n0 = blockIdx.x * 64;
  const size_t m = blockIdx.y;
  const uint32_t* src = reinterpret_cast<const uint32_t*>(s + (m * N + n0) * (size_t)KB);
  for (int i = threadIdx.x; i < 64 * q4; i += 256) t[i / q4][i % q4] = src[i];
  __syncthreads();
  uint32_t* dst = reinterpret_cast<uint32_t*>(S + m * N * (size_t)KB);
  for (int i = threadIdx.x; i < 64 * q4; i += 256) {
    const int q = i / 64, r = i % 64;
    dst[(size_t)q * N + n0 + r] = t[r][q];
  }
}

void launch_scales_stage_major(int mats, int N, int K, const uint8_t* s, uint8_t* S, hipStream_t st) {
  scales_stage_major_kernel<<<dim3(N / 64, mats), dim3(256), 0, st>>>(N, K / 32, s, S);
}

// Thread per (sorted position, group of four stages): the four dwords of stages 4G .. 4G + 3 of the token's scale
// row (one 16-byte load when the rows are whole 16-byte units, VEC) go to four stage planes; along a wave the
// positions are consecutive, so each store is one contiguous 256-byte run.
template <bool VEC>
__global__ __launch_bounds__(256) void gather_act_scales_kernel(int P, int k, int q4, const int32_t* __restrict__ pairs,
                                                                const uint8_t* __restrict__ x_s, uint8_t* __restrict__ out) {
  const int pos = blockIdx.x * 256 + threadIdx.x, q0 = 4 * blockIdx.y;
  if (pos >= P) return;
  const int t = pairs ? pairs[pos] / k : pos;
  const uint32_t* row = reinterpret_cast<const uint32_t*>(x_s + (size_t)t * q4 * 4);
  uint32_t* dst = reinterpret_cast<uint32_t*>(out) + (size_t)q0 * P + pos;
  if (VEC) {
    const u32x4 v = *reinterpret_cast<const u32x4*>(row + q0);
#pragma unroll
    for (int i = 0; i < 4; ++i) dst[(size_t)i * P] = v[i];
  } else {
    for (int i = 0; i < 4 && q0 + i < q4; ++i) dst[(size_t)i * P] = row[q0 + i];
  }
}

void launch_gather_act_scales(int P, int k, int K, const int32_t* pairs, const uint8_t* x_s, uint8_t* out,
                              hipStream_t st) {
  const int q4 = K / 128;   // stages; a scale row is 4 * q4 bytes
  const dim3 grid((P + 255) / 256, (q4 + 3) / 4);
  if (q4 % 4 == 0 && (reinterpret_cast<uintptr_t>(x_s) & 15u) == 0)
    gather_act_scales_kernel<true><<<grid, dim3(256), 0, st>>>(P, k, q4, pairs, x_s, out);
  else
    gather_act_scales_kernel<false><<<grid, dim3(256), 0, st>>>(P, k, q4, pairs, x_s, out);
}

int mfma_max_tiles(int P, int E) { return (P + kTileM - 1) / kTileM + (P < E ? P : E); }

void launch_tile_map(int E, int max_tiles, const int32_t* offsets, int32_t* tile_e, int32_t* tile_r0, int32_t* info,
                     hipStream_t s) {
  tile_map_kernel<<<dim3(1), dim3(256), 0, s>>>(E, max_tiles, offsets, tile_e, tile_r0, info);
}

template <int WF, bool GEMM1, int TN, bool PAIR = false>
static void launch_mfma_tn(const GemmProblem& p, int max_tiles, const int32_t* tile_e, const int32_t* tile_r0,
                           const int32_t* info, hipStream_t s) {
  const int cols = GEMM1 ? p.N / (TN / 2) : (p.N + TN - 1) / TN;
  const int rows = p.dense ? (p.M + kTileM - 1) / kTileM : max_tiles;
  if constexpr (WF == W_MXFP4) {
    if (p.w_tiled) {
      expert_gemm_mfma<WF, GEMM1, TN, true, PAIR><<<dim3(cols * rows), dim3(TN), 0, s>>>(p, tile_e, tile_r0, info);
      return;
    }
  }
  expert_gemm_mfma<WF, GEMM1, TN, false, PAIR><<<dim3(cols * rows), dim3(TN), 0, s>>>(p, tile_e, tile_r0, info);
}

// MXFP4 weights on the fragment-order copy: both GEMMs load the weights straight into registers (measured at
// M = 8192, interleaved with the ring kernel: GEMM1 1.17-1.19 ms against 1.22-1.23 ms; GEMM2 625 against
// 662 us). On the stored layout the paired ring serves both: GEMM1 256 weight rows per block, two blocks per
// CU (1.20 ms, against 1.29 ms for 512-row blocks of 8 waves with a three-stage ring, one block per CU).
// FP8 weights (twice the bytes per row): 256 rows, one block per CU.
template <bool GEMM1>
static void launch_mfma(WeightFormat f, const GemmProblem& p, int max_tiles, const int32_t* tile_e,
                        const int32_t* tile_r0, const int32_t* info, hipStream_t s) {
  switch (f) {
    case W_MXFP4:
      if constexpr (GEMM1) {
        if (p.w_tiled)
          expert_gemm_mfma_da<true, true><<<dim3((p.N / 128) * max_tiles), dim3(256), 0, s>>>(p, tile_e, tile_r0, info);
        else   // long K on the stored layout: the LDS ring of copies
          launch_mfma_tn<W_MXFP4, GEMM1, 256, true>(p, max_tiles, tile_e, tile_r0, info, s);
      } else if (p.w_tiled) {   // fragment-order weights: straight into registers, two blocks per CU
        expert_gemm_mfma_da<false, true><<<dim3(((p.N + 255) / 256) * max_tiles), dim3(256), 0, s>>>(p, tile_e,
                                                                                                    tile_r0, info);
      } else {   // stored layout: the paired ring (measured at M = 8192: 644 us, against 728 us in registers; on
                 // the fragment-order copy the register kernel wins, 625 against 662 us)
        launch_mfma_tn<W_MXFP4, GEMM1, 256, true>(p, max_tiles, tile_e, tile_r0, info, s);
      }
      break;
    case W_FP8_BLOCK32: launch_mfma_tn<W_FP8_BLOCK32, GEMM1, 256>(p, max_tiles, tile_e, tile_r0, info, s); break;
    default: break;   // the bf16 arm has no block-scaled form; the caller never asks for it here
  }
}

void launch_gemm1_mfma(WeightFormat f, const GemmProblem& p, int max_tiles, const int32_t* tile_e,
                       const int32_t* tile_r0, const int32_t* info, hipStream_t s) {
  launch_mfma<true>(f, p, max_tiles, tile_e, tile_r0, info, s);
}

void launch_gemm2_mfma(WeightFormat f, const GemmProblem& p, int max_tiles, const int32_t* tile_e,
                       const int32_t* tile_r0, const int32_t* info, hipStream_t s) {
  launch_mfma<false>(f, p, max_tiles, tile_e, tile_r0, info, s);
}

}  // namespace moe
