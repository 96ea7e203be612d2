// Expansion of packed MXFP4 matrices to bf16 (the decoded-BF16 arm's weights).
//
// Each value code * 2^(b-127) is exact in bf16 (DeepSeek-V4.1-Flash native-tensor page, section 2,
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

void launch_expand_mxfp4(long long rows, int cols, const uint8_t* w, const uint8_t* sc, uint16_t* out,
                         hipStream_t s) {
  const long long nblocks = rows * (cols / 32);
  long long grid = (nblocks + 255) / 256;
  if (grid > 256 * 64) grid = 256 * 64;
  if (grid < 1) grid = 1;
  expand_mxfp4_kernel<<<dim3((unsigned)grid), dim3(256), 0, s>>>(nblocks, cols, w, sc, out);
}

}  // namespace moe
