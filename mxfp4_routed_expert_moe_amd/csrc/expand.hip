// Expansion of packed MXFP4 matrices to bf16 (the decoded-BF16 arm's weights), and the fragment-order
// copy of packed E2M1 codes that the routed GEMMs can stream from.
//
// Each value code * 2^(b-127) is exact in bf16 (page "Native 1017 DSpark draft on the NVLink pair (N1-NATIVE)", section 2,
// and section 4 "expanded weights ... values exactly code * 2^(b-127)"). A thread converts one
// 32-value scale block: one 16-byte load of packed nibbles, 16 gfx950 conversions, four 16-byte stores.
#include "kernels.h"
#include "moe_device.h"

namespace moe {

__global__ __launch_bounds__(256) void expand_mxfp4_kernel(long long nblocks, int cols, const uint8_t* __restrict__ w,
                                                           const uint8_t* __restrict__ sc,
                                                           uint16_t* __restrict__ out) {
  const int bpr = cols / 32;
  for (long long i = blockIdx.x * (long long)blockDim.x + threadIdx.x; i < nblocks;
       i += (long long)gridDim.x * blockDim.x) {
    const long long r = i / bpr;
    const int b = int(i - r * bpr);
    const u32x4 raw = *reinterpret_cast<const u32x4*>(w + r * (cols / 2) + b * 16);
    const float s = e8m0_to_f32(sc[i]);
    u32x4* dst = reinterpret_cast<u32x4*>(out + r * cols + b * 32);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      dst[j] = u32x4{fp4x2_to_bf16x2<0>(raw[j], s), fp4x2_to_bf16x2<1>(raw[j], s), fp4x2_to_bf16x2<2>(raw[j], s),
                     fp4x2_to_bf16x2<3>(raw[j], s)};
  }
}

// Fragment order: thread i writes the 16 bytes of lane l = i % 64 of fragment (m, f, q): row 16 f + l % 16,
// bytes 64 q + 16 (l / 16) .. + 15 of that row. Stores are contiguous across the threads; each load is
// one 16-byte piece of a row (a one-time copy).
__global__ __launch_bounds__(256) void tile_mxfp4_kernel(long long nunits, int N, int K, const uint8_t* __restrict__ w,
                                                         uint8_t* __restrict__ out) {
  const int nq = K / 128;
  const long long per_mat = (long long)(N / 16) * nq * 64;
  for (long long i = blockIdx.x * (long long)blockDim.x + threadIdx.x; i < nunits;
       i += (long long)gridDim.x * blockDim.x) {
    const long long m = i / per_mat;
    const long long j = i - m * per_mat;
    const int l = int(j % 64);
    const long long fq = j / 64;
    const int q = int(fq % nq);
    const long long f = fq / nq;
    const long long row = 16 * f + (l % 16);
    const u32x4 v = *reinterpret_cast<const u32x4*>(w + (m * N + row) * (long long)(K / 2) + 64 * q + 16 * (l / 16));
    *reinterpret_cast<u32x4*>(out + i * 16) = v;
  }
}

void launch_tile_mxfp4(int mats, int N, int K, const uint8_t* w, uint8_t* out, hipStream_t s) {
  const long long nunits = (long long)mats * (N / 16) * (K / 128) * 64;
  long long grid = (nunits + 255) / 256;
  if (grid > 256 * 64) grid = 256 * 64;
  if (grid < 1) grid = 1;
  tile_mxfp4_kernel<<<dim3((unsigned)grid), dim3(256), 0, s>>>(nunits, N, K, w, out);
}

void launch_expand_mxfp4(long long rows, int cols, const uint8_t* w, const uint8_t* sc, uint16_t* out,
                         hipStream_t s) {
  const long long nblocks = rows * (cols / 32);
  long long grid = (nblocks + 255) / 256;
  if (grid > 256 * 64) grid = 256 * 64;
  if (grid < 1) grid = 1;
  expand_mxfp4_kernel<<<dim3((unsigned)grid), dim3(256), 0, s>>>(nblocks, cols, w, sc, out);
}

}  // namespace moe
