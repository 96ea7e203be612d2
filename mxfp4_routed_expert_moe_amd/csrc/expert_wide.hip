// Grouped expert GEMMs at prefill width (many rows per expert) on gfx950's block-scaled matrix cores, MXFP4
// weights in the fragment-order copy: a 512 x 128 block tile with one wave per SIMD.
//
// Math (page "Native 1017 DSpark draft on the NVLink pair (N1-NATIVE)", section 2 "Quantized linear" and section 4 "Kernel
// contract"): per 32-wide K block the exact products of E4M3 activation codes and E2M1 weight codes are
// summed, multiplied by the two E8M0 scales and accumulated in fp32; g and u are rounded to bf16, clamped,
// h = rw * silu(g) * u in fp32, bf16, QDQ per 32 along I; y = bf16(h_hat w2^T). One
// v_mfma_scale_f32_16x16x128_f8f6f4 computes exactly that for a 16 x 16 x 128 piece (operand layout, measured
// on gfx950: lane l supplies operand row l % 16; with g = l / 16 an E2M1 operand holds K [32g, 32g + 32), an
// E4M3 operand K [16g, 16g + 16) then K [64 + 16g, 64 + 16g + 16); lane l supplies the E8M0 scale of K block g
// of its row; result element (row 4g + v of A, row l % 16 of B) is accumulator v of lane l).
//
// Tile. A block computes 512 weight rows x 128 rows of one expert (sorted positions offsets[e] + ...), four
// waves of 128 weight rows x all 128 expert rows: 64 MFMAs and 256 fp32 accumulators per wave per 128-wide K
// step. GEMM1 gives wave w the w1 rows n0 + 64w .. + 63 and the same rows of w3 (a SwiGLU pair and a 32-column
// QDQ block meet in one lane; the block covers 256 output columns); GEMM2 gives wave w the w2 rows
// n0 + 128w .. + 127 (512 output columns). Against a 256 x 128 tile this moves a quarter fewer bytes from L2
// per flop.
//
// Data flow. Each weight row is used by one wave only, so the weights go straight from the fragment-order
// copy into registers (one 1 KB contiguous load per 16-row fragment and step), two steps ahead of their use
// in three rotating register sets; in a full tile the eight loads of a step go out one between each group of
// eight MFMAs. The activation rows (shared by the four waves) and the E8M0 bytes of both
// operands go into a three-slot LDS ring by direct global-to-LDS copies, two steps ahead. The activation
// copies place each 16-row fragment in the order its MFMA lanes read it, so every fragment read is one
// conflict-free 16-byte read per lane and half. Every wave issues the same five copies and eight loads per
// step, always (steps past the last re-read the last one), so one exact wait count covers the ring: at the
// top of step s each wave waits until the copies of step s + 1 have landed and meets the others (the slot of
// step s - 1 is then free). The first B fragment and the weight scales of step s + 1 are read during the last
// MFMAs of step s. Addresses are buffer-resource offsets: one lane offset per stream instead of a 64-bit
// address per lane.
//
// The (expert, row tile) of a block comes from the device-built tile list (tile_map_kernel); launch geometry
// depends only on (dims, M); blocks past the list exit. Work order is XCD-aware (every XCD runs one contiguous
// range of the list, ordered expert -> column tile -> row tile), so the row tiles of an expert that share a
// weight tile run together on one XCD and its L2 serves the repeats.
#include <type_traits>

#include "kernels.h"
#include "moe_device.h"

namespace moe {

namespace {

constexpr int kTN = 512;          // weight rows per block
constexpr int kTM = 128;          // expert rows per block (the tile map's row tile)
constexpr int kStep = 128;        // K per step
constexpr int kBAhead = 2;        // activation / scale copies issued this many steps ahead of their use
constexpr int kSlots = 3;         // LDS ring slots (six slots, three steps ahead, measured slower: past 64 KB
                                  // the LDS reads need more address registers and the loop spilled)
constexpr int kAAhead = 2;        // weight loads issued this many steps ahead of their use
constexpr int kASets = 3;         // weight register sets
constexpr int kGroup = 3;         // steps per unrolled loop group: lcm(kSlots, kASets)
constexpr int kCopies = 5, kLoads = 8;   // per wave and step: 4 activation + 1 scale copies, 8 weight loads
// at the top of step s the copies of step s + 1 must have landed; issued after them: the weight loads of
// their own step and (kBAhead - 2) whole steps
constexpr int kWaitB = kLoads + (kBAhead - 2) * (kCopies + kLoads);
static_assert(kASets == kAAhead + 1 && kBAhead + 1 <= kSlots && kGroup % kSlots == 0 && kGroup % kASets == 0,
              "ring and register-set rotation");
static_assert(kWaitB < 64, "vmcnt range");

// LDS layout (bytes). The activation fragments of the slots come first; the ring fits below 64 KB, so every
// fragment and scale read is one lane address plus an immediate offset.
//   B  [slot][expert row][8 chunks of 16 bytes, XOR-swizzled by row]   kSlots x 16 KB
//   WS [slot][weight row][4]                                           kSlots x 2 KB
//   AS [slot][expert row][4]                                           kSlots x 512 B
// After the K loop the ring is reused to stage the block's outputs (GEMM2: 128 rows x 1 KB of bf16; GEMM1:
// 128 rows x 256 codes and their scales), so every global store is a contiguous run of a row. The output
// row ids and route weights of the tile sit past the staging area.
constexpr int kBSlot = kTM * 128;
constexpr int kWsSlot = kTN * 4, kAsSlot = kTM * 4;
constexpr int kOffWs = kSlots * kBSlot, kOffAs = kOffWs + kSlots * kWsSlot;
constexpr int kRingBytes = kOffAs + kSlots * kAsSlot;
constexpr int kStageBytes = kTM * kTN * 2;   // GEMM2 bf16 outputs of the block
constexpr int kOffRow = kRingBytes > kStageBytes ? kRingBytes : kStageBytes, kOffRw = kOffRow + kTM * 4;
constexpr int kLdsBytes = kOffRw + kTM * 4;
static_assert(kLdsBytes <= 160 * 1024, "LDS of one workgroup");

// XOR key of the 16-byte chunks of an activation row in LDS: the rows of an MFMA fragment read distinct banks
// whether ds_read_b128 serves 8 or 16 lanes per cycle.
__device__ __forceinline__ int act_key(int r) { return ((r >> 1) ^ (4 * (r & 1))) & 7; }

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
// Asynchronous copy of 16 (or 4) bytes per lane into LDS: lane i writes at lds_wave + i * bytes.
__device__ __forceinline__ void copy16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff, uint8_t* lds_wave) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds_wave, 16, voff, soff, 0, 0);
}
__device__ __forceinline__ void copy4(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff, uint8_t* lds_wave) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds_wave, 4, voff, soff, 0, 0);
}
__device__ __forceinline__ u32x4 load16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}

// s_waitcnt with vmcnt = N and the other counters left free (gfx9 encoding: vmcnt[3:0] | expcnt[6:4] |
// lgkmcnt[11:8] | vmcnt[5:4] << 14).
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

template <int I>
using Int = std::integral_constant<int, I>;

}  // namespace

template <bool GEMM1>
__global__ __launch_bounds__(256, 1) void expert_gemm_wide(GemmProblem p, const int32_t* __restrict__ tile_e,
                                                           const int32_t* __restrict__ tile_r0,
                                                           const int32_t* __restrict__ info) {
  __shared__ __align__(16) uint8_t lds[kLdsBytes];
  // wave-uniform values are kept scalar: every address below is a scalar base plus a 32-bit lane offset
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int r16 = lane & 15, g = lane >> 4;
  const int N = p.N, K = p.K, nk = K / kStep;
  const int P = p.M * p.k;
  const int C = GEMM1 ? (N + 255) / 256 : (N + kTN - 1) / kTN;   // column tiles
  const int W = info[0] * C;
  const int L = blockIdx.x;
  if (L >= W) return;
  int w = L / 8;
  for (int i = 0; i < L % 8; ++i) w += (W - i + 7) / 8;   // blocks of the XCDs before this one
  const int e = tile_e[w / C];
  const int first = info[1 + e], nt = info[1 + p.num_experts + e];
  const int local = w - first * C;
  const int cx = local / nt, ty = first + local % nt;
  const int row0 = tile_r0[ty];
  const int nrows = min(kTM, p.offsets[e + 1] - row0);
  const int n0 = cx * (GEMM1 ? 256 : kTN);

  // ---- weights: fragment (16-row group rg, step s) of a matrix is 1 KB at ((rg * nk + s) * 1024); lane l's
  // 16 bytes at 16 l. Row groups past N re-read the last one (their outputs are never stored).
  const uint32_t wbytes = (uint32_t)(p.w_expert_stride);   // one expert matrix: N * K / 2 bytes
  const __amdgpu_buffer_rsrc_t wra = make_rsrc(static_cast<const uint8_t*>(p.wa) + (size_t)e * p.w_expert_stride, wbytes);
  const __amdgpu_buffer_rsrc_t wrb =
      GEMM1 ? make_rsrc(static_cast<const uint8_t*>(p.wb) + (size_t)e * p.w_expert_stride, wbytes) : wra;
  uint32_t afrag[8];   // byte offset of the fragment row group (wave-uniform)
#pragma unroll
  for (int a = 0; a < 8; ++a) {
    const int rg0 = GEMM1 ? (n0 + 64 * wave) / 16 + (a & 3) : (n0 + 128 * wave) / 16 + a;
    afrag[a] = (uint32_t)min(rg0, N / 16 - 1) * (uint32_t)nk * 1024u;
  }
  const uint32_t aoff = 16u * lane;
  // ---- activation rows: wave w copies rows 32w .. 32w + 31 of the tile, 8 rows (whole 128-byte lines of the
  // step) per copy: lane i takes row 8j + i / 8 and the chunk that lands at its LDS position i % 8, i.e.
  // logical chunk (i % 8) ^ key(row). Rows past the tile repeat its first row.
  const int arows = p.act_by_token ? p.M : P;   // rows of the activation matrix
  const __amdgpu_buffer_rsrc_t brs = make_rsrc(p.act_q, (uint32_t)arows * (uint32_t)K);
  uint32_t boff[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int t = 32 * wave + 8 * j + (lane >> 3);
    const int pos = row0 + (t < nrows ? t : 0);
    const int arow = p.act_by_token ? p.pairs[pos] / p.k : pos;
    boff[j] = (uint32_t)arow * (uint32_t)K + 16u * (uint32_t)((lane & 7) ^ act_key(t));
  }
  // ---- scales (both stage-major: 4 bytes per row and 128-wide step, rows of a step side by side).
  // Waves 0, 1: the weight scales of 256 rows each (GEMM1: w1 rows, then the same w3 rows); waves 2, 3: the
  // activation scales of 64 rows each. Rows past the end re-read the last ones.
  __amdgpu_buffer_rsrc_t srs;
  uint32_t soff, sstep;
  if (wave < 2) {
    const uint8_t* sm = (GEMM1 && wave == 1) ? p.sb : p.sa;
    srs = make_rsrc(sm + (size_t)e * p.s_expert_stride, (uint32_t)p.s_expert_stride);
    soff = 4u * (uint32_t)min(n0 + (GEMM1 ? 0 : 256 * wave) + 4 * lane, N - 4);
    sstep = (uint32_t)N * 4u;
  } else {
    srs = make_rsrc(p.act_s, (uint32_t)P * (uint32_t)(K / 32));
    soff = 4u * (uint32_t)min(row0 + 64 * (wave - 2) + lane, P - 1);
    sstep = (uint32_t)P * 4u;
  }

  u32x4 A[kASets][8];
  // the copies of step j into slot S (steps past the last re-read it)
  auto copies = [&](int j, auto slot) {
    constexpr int S = decltype(slot)::value;
    const uint32_t jj = (uint32_t)min(j, nk - 1);
#pragma unroll
    for (int j = 0; j < 4; ++j) copy16(brs, boff[j], jj * kStep, &lds[S * kBSlot + (32 * wave + 8 * j) * 128]);
    if (wave < 2) copy16(srs, soff, jj * sstep, &lds[kOffWs + S * kWsSlot + wave * 1024]);
    else copy4(srs, soff, jj * sstep, &lds[kOffAs + S * kAsSlot + (wave - 2) * 256]);
  };
  // the weight loads of step j into register set R
  auto loads = [&](int j, auto set) {
    constexpr int R = decltype(set)::value;
    const uint32_t jj = (uint32_t)min(j, nk - 1);
#pragma unroll
    for (int a = 0; a < 8; ++a) A[R][a] = load16((GEMM1 && a >= 4) ? wrb : wra, aoff, afrag[a] + jj * 1024u);
  };

  // per-lane LDS addresses: B fragment data (+ slot, fragment, half as immediates), weight scales (+ slot and
  // fragment), activation scales (+ slot and fragment)
  // (B fragment b, lane l: row 16 b + l % 16, logical chunks g and 4 + g; the key depends on l % 16 only)
  const uint32_t lb0 = 128u * r16 + 16u * (uint32_t)(g ^ act_key(r16));
  const uint32_t lb1 = 128u * r16 + 16u * (uint32_t)((4 + g) ^ act_key(r16));
  const uint32_t lws = kOffWs + 4u * (uint32_t)((GEMM1 ? 64 : 128) * wave + r16) + g;
  const uint32_t las = kOffAs + 4u * r16 + g;
  // weight-scale offset of fragment a (GEMM1: w1 rows in the first 1 KB, the same w3 rows in the second)
  auto ws_off = [&](int a) { return GEMM1 ? (a >= 4 ? 1024 : 0) + 64 * (a & 3) : 64 * a; };
  f32x4 acc[8][8];
#pragma unroll
  for (int a = 0; a < 8; ++a)
#pragma unroll
    for (int b = 0; b < 8; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nbv = min(8, (nrows + 15) / 16);   // 16-row groups holding a row of the tile
  int sa[8], sb;
  u32x4 b0, b1;
  auto read_head = [&](auto set) {   // weight scales and the first B fragment of a step
    constexpr int S = decltype(set)::value;
#pragma unroll
    for (int a = 0; a < 8; ++a) sa[a] = lds[lws + S * kWsSlot + ws_off(a)];
    b0 = *reinterpret_cast<const u32x4*>(&lds[lb0 + S * kBSlot]);
    b1 = *reinterpret_cast<const u32x4*>(&lds[lb1 + S * kBSlot]);
    sb = lds[las + S * kAsSlot];
  };
  // the 64 MFMAs of one step; the B fragments are read one ahead, and after the last one the head of the
  // next step (whose copies have landed: the wait at the top of this step covered them)
  auto compute = [&](int s, auto slot, auto set, auto part) {
    constexpr int S = decltype(slot)::value, R = decltype(set)::value;
    constexpr bool PART = decltype(part)::value;
    constexpr int RN = (S + kAAhead) % kASets;   // register set of step s + 2 (a full tile loads it here)
    const uint32_t jn = (uint32_t)min(s + kAAhead, nk - 1);
    i32x8 Af[8];
#pragma unroll
    for (int a = 0; a < 8; ++a)
      Af[a] = i32x8{(int)A[R][a][0], (int)A[R][a][1], (int)A[R][a][2], (int)A[R][a][3], 0, 0, 0, 0};
    int sac[8];
#pragma unroll
    for (int a = 0; a < 8; ++a) sac[a] = sa[a];
#pragma unroll
    for (int b = 0; b < 8; ++b) {
      if (PART && b >= nbv) continue;
      const i32x8 Bf = i32x8{(int)b0[0], (int)b0[1], (int)b0[2], (int)b0[3], (int)b1[0], (int)b1[1], (int)b1[2],
                             (int)b1[3]};
      const int sbc = sb;
      if (b < 7 && !(PART && b + 1 >= nbv)) {
        b0 = *reinterpret_cast<const u32x4*>(&lds[lb0 + S * kBSlot + (b + 1) * 2048]);
        b1 = *reinterpret_cast<const u32x4*>(&lds[lb1 + S * kBSlot + (b + 1) * 2048]);
        sb = lds[las + S * kAsSlot + 64 * (b + 1)];
      } else if (!PART) {
        read_head(Int<(S + 1) % kSlots>{});
      }
      if constexpr (!PART) A[RN][b] = load16((GEMM1 && b >= 4) ? wrb : wra, aoff, afrag[b] + jn * 1024u);
#pragma unroll
      for (int a = 0; a < 8; ++a)
        acc[a][b] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(Af[a], Bf, acc[a][b], 4, 0, 0, sac[a], 0, sbc);
    }
    if (PART) {
      read_head(Int<(S + 1) % kSlots>{});
    } else {
      // schedule: the reads of B fragment b + 1 (three LDS reads; after the last fragment the eleven reads of
      // the next step's head), weight load b of step s + 2, then the eight MFMAs of fragment b, which hide
      // their latency. (The eight weight loads issued together stall the wave's issue, MFMAs included,
      // while the memory pipeline takes them in.)
#pragma unroll
      for (int b = 0; b < 7; ++b) {
        __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);
        __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x100, 11, 0);
      __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
    }
  };
  // one step s with its ring slot S = s % kSlots and weight set R = s % kASets (compile time in the unrolled
  // loop). The loop runs whole groups of kGroup steps; steps past the last still wait, meet and issue (their
  // copies and loads re-read the last step) but skip the MFMAs. (Leaving the unrolled group early instead
  // makes the register allocator shuffle the 256 accumulators at every exit.)
  auto step = [&](int s, auto slot, auto part) {
    constexpr int S = decltype(slot)::value;
    asm volatile("" ::: "memory");     // (compiler fence: no memory access moves across the wait and barrier)
    wait_vm<kWaitB>();                 // the copies of step s + 1 landed
    __builtin_amdgcn_s_barrier();      // every wave's copies for s + 1 are visible; slot s - 1 is free
    asm volatile("" ::: "memory");
    copies(s + kBAhead, Int<(S + kBAhead) % kSlots>{});
    asm volatile("" ::: "memory");     // (the weight loads stay behind the copies: the waits count on that order)
    // the weight loads of step s + 2: a full tile's between the MFMAs of step s, a partial tile's (whose
    // fragment loop branches) and those of a step past the end here
    constexpr bool PART = decltype(part)::value;
    if constexpr (PART) loads(s + kAAhead, Int<(S + kAAhead) % kASets>{});
    if (s < nk) compute(s, slot, Int<S % kASets>{}, part);
    else if constexpr (!PART) loads(s + kAAhead, Int<(S + kAAhead) % kASets>{});
  };

  // the epilogue's per-row data (pair id, route weight) is fetched now, under the prologue's wait, and kept
  // in LDS: fetched per 16-row group in the epilogue it costs a dependent round trip per group
  int my_row = -1;
  float my_rw = 0.0f;
  const int tr = wave * 64 + lane;   // threads 0 .. 127 take one row of the tile each
  if (tr < kTM && tr < nrows) my_row = p.pairs[row0 + tr];
  copies(0, Int<0>{});
  loads(0, Int<0>{});
  copies(1, Int<1>{});
  loads(1, Int<1>{});
  static_assert(kBAhead == 2 && kAAhead == 2, "prologue");
  if (GEMM1 && my_row >= 0) my_rw = p.rw[my_row];
  asm volatile("" ::: "memory");
  wait_vm<0>();
  if (tr < kTM) {
    *reinterpret_cast<int*>(&lds[kOffRow + 4 * tr]) = my_row;
    *reinterpret_cast<float*>(&lds[kOffRw + 4 * tr]) = my_rw;
  }
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  read_head(Int<0>{});
  auto kloop = [&](auto part) {
    for (int s = 0; s < nk; s += kGroup) {
      step(s, Int<0>{}, part);
      step(s + 1, Int<1>{}, part);
      step(s + 2, Int<2>{}, part);
    }
  };
  static_assert(kGroup == 3, "loop group");
  if (nbv == 8) kloop(std::false_type{});
  else kloop(std::true_type{});
  wait_vm<0>();                        // the re-read steps past the end land before the ring is reused
  __syncthreads();                     // every wave is done with the ring: it stages the outputs now

  // ---- epilogue: lane holds weight rows 4g .. 4g + 3 of each A fragment for expert row r16 of each B fragment
  if constexpr (GEMM1) {
    // h codes staged as [row][256 bytes] (16-byte chunks XOR-swizzled by row), their E8M0 bytes as
    // [row][8] (the block's eight 32-column blocks)
    uint8_t* hst = lds;
    uint8_t* sst = lds + kTM * 256;
#pragma unroll
    for (int b = 0; b < 8; ++b) {
      if (b >= nbv) continue;   // (wave-uniform) 16-row groups past the tile's rows: nothing to compute or store
      const int t = 16 * b + r16;
      const float rwv = t < nrows ? *reinterpret_cast<const float*>(&lds[kOffRw + 4 * t]) : 1.0f;
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {   // the wave's two 32-column QDQ blocks: fragments 2qb, 2qb + 1 (+4: w3)
        float h[2][4];
        float amax = 0.0f;
#pragma unroll
        for (int half = 0; half < 2; ++half)
          amax = fmaxf(amax, swiglu_bf16x4(acc[2 * qb + half][b], acc[4 + 2 * qb + half][b], rwv, true, h[half]));
        // the 32 columns of the block for row r16 live in lanes r16 + 16 g, g = 0..3
        amax = fmaxf(amax, __shfl_xor(amax, 16, 64));
        amax = fmaxf(amax, __shfl_xor(amax, 32, 64));
        const int E8 = qdq_exponent(amax);
        const float inv = exp2_neg(E8);
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          const int chunk = 4 * wave + 2 * qb + half;   // 16 columns of the block's 256
          *reinterpret_cast<uint32_t*>(&hst[256 * t + 16 * (chunk ^ (t & 15)) + 4 * g]) =
              qdq_code4(h[half][0], h[half][1], h[half][2], h[half][3], inv);
        }
        if (g == 0) sst[8 * t + 2 * wave + qb] = uint8_t(E8 + 127);
      }
    }
    __syncthreads();
    // stores: one 16-byte chunk per lane, 16 lanes per row (256 contiguous bytes), 32 rows per wave
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int t = 32 * wave + 4 * j + (lane >> 4), c = lane & 15;
      if (t < nrows && n0 + 16 * c < N)
        *reinterpret_cast<u32x4*>(p.h_q + (size_t)(row0 + t) * N + n0 + 16 * c) =
            *reinterpret_cast<const u32x4*>(&hst[256 * t + 16 * (c ^ (t & 15))]);
    }
    // scales: one dword (four 32-column blocks = one 128-column stage group) per (row, group)
    {
      const int t = threadIdx.x & (kTM - 1), G = threadIdx.x >> 7;   // 256 threads: 128 rows x 2 groups
      const int col = n0 + 128 * G;
      if (t < nrows && col < N) {
        const uint32_t v = *reinterpret_cast<const uint32_t*>(&sst[8 * t + 4 * G]);
        const size_t pos = (size_t)row0 + t;
        uint8_t* dst = p.h_s_stage_major ? p.h_s + ((size_t)(col / 128) * P + pos) * 4
                                         : p.h_s + pos * (N / 32) + col / 32;
        *reinterpret_cast<uint32_t*>(dst) = v;
      }
    }
  } else if (p.out_f32) {   // fp32 partial sums (tensor-parallel mode): 16 bytes per lane and fragment
#pragma unroll
    for (int b = 0; b < 8; ++b) {
      const int t = 16 * b + r16;
      if (t < nrows) {
        const int orow = *reinterpret_cast<const int*>(&lds[kOffRow + 4 * t]);
#pragma unroll
        for (int a = 0; a < 8; ++a) {
          const int col = n0 + 128 * wave + 16 * a + 4 * g;
          if (col < N) *reinterpret_cast<f32x4*>(p.out_f32 + (size_t)orow * N + col) = acc[a][b];
        }
      }
    }
  } else {
    // bf16 outputs staged as [row][1 KB] (16-byte chunks XOR-swizzled by row), then stored a whole row segment
    // (512 columns) per wave instruction
#pragma unroll
    for (int b = 0; b < 8; ++b) {
      if (b >= nbv) continue;   // (wave-uniform) 16-row groups past the tile's rows are never stored
      const int t = 16 * b + r16;
#pragma unroll
      for (int a = 0; a < 8; ++a) {
        const int c = 128 * wave + 16 * a + 4 * g;   // column within the block
        const uint32_t lo = uint32_t(f32_to_bf16_rne(acc[a][b][0])) | (uint32_t(f32_to_bf16_rne(acc[a][b][1])) << 16);
        const uint32_t hi = uint32_t(f32_to_bf16_rne(acc[a][b][2])) | (uint32_t(f32_to_bf16_rne(acc[a][b][3])) << 16);
        *reinterpret_cast<u32x2*>(&lds[1024 * t + 16 * ((c >> 3) ^ (t & 63)) + 2 * (c & 7)]) = u32x2{lo, hi};
      }
    }
    __syncthreads();
#pragma unroll 4
    for (int j = 0; j < 32; ++j) {
      const int t = 32 * wave + j;
      if (t < nrows && n0 + 8 * lane < N) {
        const int orow = *reinterpret_cast<const int*>(&lds[kOffRow + 4 * t]);
        *reinterpret_cast<u32x4*>(p.out + (size_t)orow * N + n0 + 8 * lane) =
            *reinterpret_cast<const u32x4*>(&lds[1024 * t + 16 * (lane ^ (t & 63))]);
      }
    }
  }
}

// Requirements (checked by the caller): MXFP4 weights in the fragment-order copy, scales of both operands
// stage-major, routed rows (act_by_token for GEMM1), N and K multiples of 128, and every operand's bytes below
// 2^31 (32-bit buffer offsets): wide_fits().
void launch_gemm1_wide(const GemmProblem& p, int max_tiles, const int32_t* tile_e, const int32_t* tile_r0,
                       const int32_t* info, hipStream_t s) {
  const int cols = (p.N + 255) / 256;
  expert_gemm_wide<true><<<dim3(cols * max_tiles), dim3(256), 0, s>>>(p, tile_e, tile_r0, info);
}

void launch_gemm2_wide(const GemmProblem& p, int max_tiles, const int32_t* tile_e, const int32_t* tile_r0,
                       const int32_t* info, hipStream_t s) {
  const int cols = (p.N + kTN - 1) / kTN;
  expert_gemm_wide<false><<<dim3(cols * max_tiles), dim3(256), 0, s>>>(p, tile_e, tile_r0, info);
}

}  // namespace moe
