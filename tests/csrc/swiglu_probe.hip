// Test-only probe of the library's device SwiGLU (mxfp4_routed_expert_moe_amd/csrc/moe_device.h): runs
// moe::swiglu elementwise so a test can compare the device fp32 chain (hardware base-2 exponential with a
// two-part log2 e, reciprocal plus one FMA correction) with the oracle's correctly rounded fp32 chain.
// Built into tests/libswiglu_probe.so; never part of libmoe.so.
#include <hip/hip_runtime.h>

#include "../../mxfp4_routed_expert_moe_amd/csrc/moe_device.h"

namespace {

__global__ __launch_bounds__(256) void swiglu_probe_kernel(int n, const float* __restrict__ g,
                                                           const float* __restrict__ u,
                                                           const float* __restrict__ rw, float* __restrict__ h) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) h[i] = moe::swiglu(g[i], u[i], rw[i], true);
}

}  // namespace

// h[i] = the device SwiGLU of bf16-valued g[i], u[i] times the route weight rw[i] (fp32, unrounded).
// All pointers are device pointers of n floats; returns 0, or -1 for a bad argument, -4 if the launch failed.
extern "C" int swiglu_probe(int n, const float* g, const float* u, const float* rw, float* h, void* stream) {
  if (n < 0 || (n > 0 && (!g || !u || !rw || !h))) return -1;
  if (n == 0) return 0;
  swiglu_probe_kernel<<<dim3((n + 255) / 256), dim3(256), 0, static_cast<hipStream_t>(stream)>>>(n, g, u, rw, h);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}
