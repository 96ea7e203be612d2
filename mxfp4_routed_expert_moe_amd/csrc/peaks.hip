// Peak-rate microbenchmarks of the two rooflines the layer is measured against, on this GPU (a bench-only
// library, libpeaks.so; not part of libmoe.so):
//   moe_peak_stream_read - every byte of a device buffer read once with 16-byte loads per lane (optionally
//                          non-temporal), the access the decode-width GEMMs make of the packed weights; the
//                          caller sweeps the block count and loads in flight and keeps the best;
//   moe_peak_l2_read     - the same loads from a buffer small enough to stay in every XCD's L2 (the rate at
//                          which the L2s feed the CUs when they hit);
//   moe_peak_mfma        - a dependency-free stream of v_mfma_scale_f32_16x16x128_f8f6f4 on every SIMD, for a
//                          pair of operand formats (E2M1 x E4M3 is the pair of the routed experts).
// Both write one value per wave or block so that no load or MFMA is removed.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kMaxReadBlocks = 8192;

// Each wave reads a contiguous run of the buffer, 1 KB per load instruction (16 bytes per lane), UNROLL loads
// in flight, as a decode GEMM wave streams its weight fragments (NT: with the non-temporal hint);
// XOR-folded into one dword per block.
template <int UNROLL, bool NT>
__global__ __launch_bounds__(256) void stream_read_kernel(const u32x4* __restrict__ buf, size_t n16,
                                                          unsigned* __restrict__ sink) {
  const size_t waves = (size_t)gridDim.x * 4;
  const size_t wave = (size_t)blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  const size_t per = (n16 / 64 + waves - 1) / waves;   // 1 KB pieces per wave
  const size_t p0 = min(wave * per, n16 / 64), p1 = min(p0 + per, n16 / 64);
  auto ld = [&](size_t i) {
    if constexpr (NT) return __builtin_nontemporal_load(buf + i);
    else return buf[i];
  };
  unsigned x = 0;
  size_t q = p0;
  for (; q + UNROLL <= p1; q += UNROLL) {
    u32x4 v[UNROLL];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) v[u] = ld((q + u) * 64 + lane);
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) x ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  for (; q < p1; ++q) {
    const u32x4 v = ld(q * 64 + lane);
    x ^= v[0] ^ v[1] ^ v[2] ^ v[3];
  }
  __shared__ unsigned red[256];
  red[threadIdx.x] = x;
  __syncthreads();
  if (threadIdx.x == 0) {
    unsigned r = 0;
    for (int t = 0; t < 256; ++t) r ^= red[t];
    sink[blockIdx.x] = r;
  }
}

// L2-resident reads: wave w reads the 64 KB window (w mod windows) of a small buffer (all windows fit every XCD's
// L2 after the first pass) reps times, 1 KB per load instruction (16 bytes per lane), 16 loads in flight.
__global__ __launch_bounds__(256) void l2_read_kernel(const u32x4* __restrict__ buf, int windows, int reps,
                                                      unsigned* __restrict__ sink) {
  const int wave = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  const u32x4* base = buf + (size_t)(wave % windows) * 4096;   // 64 KB = 4096 x 16 B
  unsigned x = 0;
  for (int r = 0; r < reps; ++r) {
#pragma unroll 1
    for (int q = 0; q < 64; q += 16) {
      u32x4 v[16];
#pragma unroll
      for (int u = 0; u < 16; ++u) v[u] = base[(size_t)(q + u) * 64 + lane];
#pragma unroll
      for (int u = 0; u < 16; ++u) x ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
    }
    x = (x << 1) | (x >> 31);
  }
  __shared__ unsigned red[256];
  red[threadIdx.x] = x;
  __syncthreads();
  if (threadIdx.x == 0) {
    unsigned t = 0;
    for (int i = 0; i < 256; ++i) t ^= red[i];
    sink[blockIdx.x] = t;
  }
}

// iters x 8 MFMAs per wave on 8 independent accumulators. Operands are finite codes of each format (E4M3 and
// E2M1 bytes 0x38 / 0x22 with small lane-dependent variation), scales 127 (1.0).
template <int FA, int FB>
__global__ __launch_bounds__(256) void mfma_peak_kernel(int iters, float* __restrict__ sink) {
  const int lane = threadIdx.x & 63;
  const int a8 = 0x38383838 ^ (lane & 3), a4 = 0x22222222 ^ ((lane & 1) << 1);
  const int av = FA == 4 ? a4 : a8, bv = FB == 4 ? a4 : a8;
  const i32x8 A = i32x8{av, av ^ 1, av, av ^ 1, av, av, av, av};
  const i32x8 B = i32x8{bv, bv, bv ^ 1, bv, bv, bv ^ 1, bv, bv};
  f32x4 acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, (float)j};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 8; ++j)
      acc[j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A, B, acc[j], FA, FB, 0, 127, 0, 127);
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) s += acc[j][0] + acc[j][1] + acc[j][2] + acc[j][3];
  if (lane == 0) sink[blockIdx.x * 4 + (threadIdx.x >> 6)] = s;
}

}  // namespace

extern "C" {

// Number of dwords the sink of moe_peak_stream_read must hold (the largest block count it takes).
int moe_peak_stream_blocks(void) { return kMaxReadBlocks; }

// Reads `bytes` (a multiple of 1024) of the device buffer `buf` once with `blocks` blocks of 4 waves (1 ..
// moe_peak_stream_blocks()), `unroll` loads in flight per wave (8 or 16), with the non-temporal hint if nt;
// sink: device, moe_peak_stream_blocks() dwords. Returns 0, -1 for a bad argument, -4 if the launch failed.
int moe_peak_stream_read(const void* buf, size_t bytes, int blocks, int unroll, int nt, unsigned* sink, void* stream) {
  if (!buf || !sink || bytes % 1024 != 0 || blocks < 1 || blocks > kMaxReadBlocks) return -1;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const auto* b = static_cast<const u32x4*>(buf);
  const size_t n16 = bytes / 16;
  const dim3 g(blocks), t(256);
  if (unroll == 8 && nt) stream_read_kernel<8, true><<<g, t, 0, s>>>(b, n16, sink);
  else if (unroll == 8) stream_read_kernel<8, false><<<g, t, 0, s>>>(b, n16, sink);
  else if (unroll == 16 && nt) stream_read_kernel<16, true><<<g, t, 0, s>>>(b, n16, sink);
  else if (unroll == 16) stream_read_kernel<16, false><<<g, t, 0, s>>>(b, n16, sink);
  else return -1;
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

// L2-resident read rate: `blocks` blocks (1 .. moe_peak_stream_blocks()) of 4 waves, each wave reading one of
// `windows` 64 KB windows of `buf` (windows * 64 KB bytes, device) reps times. Bytes read = blocks * 4 * reps *
// 65536. sink: device, moe_peak_stream_blocks() dwords. Returns 0, -1 for a bad argument, -4 if the launch failed.
int moe_peak_l2_read(const void* buf, int windows, int blocks, int reps, unsigned* sink, void* stream) {
  if (!buf || !sink || windows < 1 || blocks < 1 || blocks > kMaxReadBlocks || reps < 1) return -1;
  l2_read_kernel<<<dim3(blocks), dim3(256), 0, static_cast<hipStream_t>(stream)>>>(static_cast<const u32x4*>(buf),
                                                                                   windows, reps, sink);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

// `blocks` blocks of 4 waves, each wave issuing iters x 8 scaled 16x16x128 MFMAs of formats (fmt_a, fmt_b):
// (4, 0) E2M1 x E4M3, (0, 0) E4M3 x E4M3 or (4, 4) E2M1 x E2M1. sink: device, 4 * blocks floats.
// flop = blocks * 4 * iters * 8 * 65536. Returns 0, -1 for a bad argument, -4 if the launch failed.
int moe_peak_mfma(int fmt_a, int fmt_b, int blocks, int iters, float* sink, void* stream) {
  if (!sink || blocks <= 0 || iters <= 0) return -1;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (fmt_a == 4 && fmt_b == 0) mfma_peak_kernel<4, 0><<<dim3(blocks), dim3(256), 0, s>>>(iters, sink);
  else if (fmt_a == 0 && fmt_b == 0) mfma_peak_kernel<0, 0><<<dim3(blocks), dim3(256), 0, s>>>(iters, sink);
  else if (fmt_a == 4 && fmt_b == 4) mfma_peak_kernel<4, 4><<<dim3(blocks), dim3(256), 0, s>>>(iters, sink);
  else return -1;
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

}  // extern "C"
