// Router of the routed-MoE layer on gfx950, and the per-32 E4M3 QDQ of its input rows.
//
// Gate (DeepSeek-V4.1-Flash native-tensor page, section 2 "Gate"): fp32 logits of the raw bf16 x
// against the fp32 gate weight, scores sqrt(softplus(l)), top-k of scores + bias (the bias only
// selects), gathered scores normalised by their sum + 1e-20 and scaled by the route scale.
// Activation QDQ (same section, "Quantized linear"): per 32 inputs, E8M0 scale
// 2^ceil(log2(max(amax, 1e-4) / 448)) and E4M3 codes; done once per row and shared by every expert.
//
// Fixed fp32 orders (recorded so routing is reproducible): each logit is accumulated in fp32 as
// strided partial sums (small M: per 512-wide chunk of H, 64 lanes x an 8-FMA chain, then a
// butterfly, then the chunks added in ascending order; large M: 32-wide chunks summed into a running
// total); the normalising sum adds the k weights in slot order.
#include "kernels.h"
#include "moe_device.h"

namespace moe {

constexpr int kSmallM = 64;
constexpr int kChunkH = 512;   // H columns per partial logit at small M

// Small M: one wave per (expert, 512-wide chunk of H); lane l covers 8 consecutive columns. Every
// wave handles all M <= 64 tokens, so each gate element is read once. The wave's fp32 partial sum
// (8 FMA chain per lane, then a butterfly over the 64 lanes) goes to part[chunk][t][e]; the select
// kernel adds the chunks in ascending order.
__global__ __launch_bounds__(256) void router_logits_small(int M, int H, int E, const uint16_t* __restrict__ x,
                                                           const float* __restrict__ gate_w,
                                                           float* __restrict__ part) {
  const int lane = threadIdx.x & 63;
  const int e = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int chunk = blockIdx.y;
  if (e >= E) return;
  const int h = chunk * kChunkH + lane * 8;
  const bool ok = h < H;
  float4 w0 = make_float4(0.f, 0.f, 0.f, 0.f), w1 = w0;
  if (ok) {
    w0 = *reinterpret_cast<const float4*>(gate_w + (size_t)e * H + h);
    w1 = *reinterpret_cast<const float4*>(gate_w + (size_t)e * H + h + 4);
  }
  const size_t plane = (size_t)M * E;
  for (int t = 0; t < M; ++t) {
    float a = 0.0f;
    if (ok) {
      const u32x4 xv = *reinterpret_cast<const u32x4*>(x + (size_t)t * H + h);
      a = __builtin_fmaf(bits_to_f32(xv[0] << 16), w0.x, a);
      a = __builtin_fmaf(bits_to_f32(xv[0] & 0xFFFF0000u), w0.y, a);
      a = __builtin_fmaf(bits_to_f32(xv[1] << 16), w0.z, a);
      a = __builtin_fmaf(bits_to_f32(xv[1] & 0xFFFF0000u), w0.w, a);
      a = __builtin_fmaf(bits_to_f32(xv[2] << 16), w1.x, a);
      a = __builtin_fmaf(bits_to_f32(xv[2] & 0xFFFF0000u), w1.y, a);
      a = __builtin_fmaf(bits_to_f32(xv[3] << 16), w1.z, a);
      a = __builtin_fmaf(bits_to_f32(xv[3] & 0xFFFF0000u), w1.w, a);
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) a += __shfl_xor(a, off, 64);
    if (lane == 0) part[(size_t)chunk * plane + (size_t)t * E + e] = a;
  }
}

// Tiled fp32 logits for larger M: a block computes 32 tokens x 128 experts, H in chunks of 32.
__global__ __launch_bounds__(256) void router_logits_tiled(int M, int H, int E, const uint16_t* __restrict__ x,
                                                           const float* __restrict__ gate_w,
                                                           float* __restrict__ logits) {
  __shared__ float xs[32][33];
  __shared__ float ws[128][33];
  const int tid = threadIdx.x;
  const int t0 = blockIdx.x * 32, e0 = blockIdx.y * 128;
  const int tt = tid >> 5, te = tid & 31;
  float acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = 0.0f;
  for (int h0 = 0; h0 < H; h0 += 32) {
    {  // x tile: 32 tokens x 32 columns, 4 bf16 per thread
      const int r = tid >> 3, c = (tid & 7) * 4;
      float v0 = 0.f, v1 = 0.f, v2 = 0.f, v3 = 0.f;
      if (t0 + r < M) {
        const uint2 xv = *reinterpret_cast<const uint2*>(x + (size_t)(t0 + r) * H + h0 + c);
        v0 = bits_to_f32(xv.x << 16); v1 = bits_to_f32(xv.x & 0xFFFF0000u);
        v2 = bits_to_f32(xv.y << 16); v3 = bits_to_f32(xv.y & 0xFFFF0000u);
      }
      xs[r][c] = v0; xs[r][c + 1] = v1; xs[r][c + 2] = v2; xs[r][c + 3] = v3;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {  // gate tile: 128 experts x 32 columns, 16 floats per thread
      const int r = (tid >> 3) + 32 * i, c = (tid & 7) * 4;
      float4 w = make_float4(0.f, 0.f, 0.f, 0.f);
      if (e0 + r < E) w = *reinterpret_cast<const float4*>(gate_w + (size_t)(e0 + r) * H + h0 + c);
      ws[r][c] = w.x; ws[r][c + 1] = w.y; ws[r][c + 2] = w.z; ws[r][c + 3] = w.w;
    }
    __syncthreads();
    float part[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) part[i][j] = 0.0f;
#pragma unroll 8
    for (int kk = 0; kk < 32; ++kk) {
      float xv[4], wv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) xv[i] = xs[tt * 4 + i][kk];
#pragma unroll
      for (int j = 0; j < 4; ++j) wv[j] = ws[te + 32 * j][kk];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) part[i][j] = __builtin_fmaf(xv[i], wv[j], part[i][j]);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] += part[i][j];
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int t = t0 + tt * 4 + i;
    if (t >= M) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = e0 + te + 32 * j;
      if (e < E) logits[(size_t)t * E + e] = acc[i][j];
    }
  }
}

struct Cand { float v; float s; int i; };

__device__ __forceinline__ Cand better(Cand a, Cand b) {
  // larger selection score wins; equal scores go to the lower expert id
  return (a.v > b.v || (a.v == b.v && a.i < b.i)) ? a : b;
}

// One block per token. Wave 0: scores, biased top-k, normalisation; all four waves: the QDQ of the
// token's row (one 32-wide block per thread).
__global__ __launch_bounds__(256) void router_select_qdq(int M, int H, int E, int k, float route_scale,
                                                         int nparts, const float* __restrict__ logits,
                                                         const float* __restrict__ gate_b,
                                                         const uint16_t* __restrict__ x,
                                                         int32_t* __restrict__ ids, float* __restrict__ rw,
                                                         uint8_t* __restrict__ x_q, uint8_t* __restrict__ x_s) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x;
  if (threadIdx.x < 64) {
  // ---- scores and selection values: lane owns experts lane, lane + 64, ... (E <= 256)
  float sc[4], sel[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int e = lane + 64 * j;
    sc[j] = 0.0f; sel[j] = -INFINITY;
    if (e < E) {
      // partial logits added in ascending chunk order; four loads in flight at a time
      const float* lp = logits + (size_t)t * E + e;
      const size_t plane = (size_t)M * E;
      float l = lp[0];
      int c = 1;
      for (; c + 3 < nparts; c += 4) {
        const float a0 = lp[c * plane], a1 = lp[(c + 1) * plane], a2 = lp[(c + 2) * plane], a3 = lp[(c + 3) * plane];
        l = l + a0;
        l = l + a1;
        l = l + a2;
        l = l + a3;
      }
      for (; c < nparts; ++c) l = l + lp[c * plane];
      const float sp = l > 20.0f ? l : log1pf(expf(l));
      sc[j] = sqrtf(sp);
      sel[j] = sc[j] + gate_b[e];
    }
  }
  float wsel[8];
  int isel[8];
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    wsel[r] = 0.0f;
    isel[r] = 0;
    if (r >= k) continue;
    Cand c{-INFINITY, 0.0f, 0x7FFFFFFF};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = lane + 64 * j;
      if (e < E) c = better(c, Cand{sel[j], sc[j], e});
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      Cand o{__shfl_xor(c.v, off, 64), __shfl_xor(c.s, off, 64), __shfl_xor(c.i, off, 64)};
      c = better(c, o);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (lane + 64 * j == c.i) sel[j] = -INFINITY;   // remove the winner
    wsel[r] = c.s;
    isel[r] = c.i;
  }
  if (lane == 0) {
    float sum = 0.0f;
#pragma unroll
    for (int r = 0; r < 8; ++r)
      if (r < k) sum = sum + wsel[r];
    const float denom = sum + 1e-20f;
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      if (r < k) {
        ids[(size_t)t * k + r] = isel[r];
        rw[(size_t)t * k + r] = (wsel[r] / denom) * route_scale;
      }
    }
  }
  }
  // ---- QDQ of the row: one 32-wide block per thread per iteration
  const int nb = H / 32;
  for (int b = threadIdx.x; b < nb; b += 256) {
    const uint16_t* src = x + (size_t)t * H + b * 32;
    u32x4 raw[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) raw[i] = *reinterpret_cast<const u32x4*>(src + 8 * i);
    float v[32];
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        v[8 * i + 2 * j] = bits_to_f32(raw[i][j] << 16);
        v[8 * i + 2 * j + 1] = bits_to_f32(raw[i][j] & 0xFFFF0000u);
      }
#pragma unroll
    for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
    const int E8 = qdq_exponent(amax);
    const float inv = exp2_neg(E8);
    u32x4 out[2];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t c0 = qdq_code(v[4 * i], inv), c1 = qdq_code(v[4 * i + 1], inv);
      const uint32_t c2 = qdq_code(v[4 * i + 2], inv), c3 = qdq_code(v[4 * i + 3], inv);
      out[i >> 2][i & 3] = c0 | (c1 << 8) | (c2 << 16) | (c3 << 24);
    }
    u32x4* dst = reinterpret_cast<u32x4*>(x_q + (size_t)t * H + b * 32);
    dst[0] = out[0];
    dst[1] = out[1];
    x_s[(size_t)t * nb + b] = uint8_t(E8 + 127);
  }
}

int router_logit_parts(int M, int H) { return M <= kSmallM ? (H + kChunkH - 1) / kChunkH : 1; }

void launch_router_logits(int M, int H, int E, const uint16_t* x, const float* gate_w, float* logits,
                          hipStream_t s) {
  if (M <= kSmallM) {
    router_logits_small<<<dim3((E + 3) / 4, router_logit_parts(M, H)), dim3(256), 0, s>>>(M, H, E, x, gate_w, logits);
  } else {
    router_logits_tiled<<<dim3((M + 31) / 32, (E + 127) / 128), dim3(256), 0, s>>>(M, H, E, x, gate_w, logits);
  }
}

void launch_router_select_qdq(int M, int H, int E, int k, float route_scale, const float* logits,
                              const float* gate_b, const uint16_t* x, int32_t* ids, float* rw,
                              uint8_t* x_q, uint8_t* x_s, hipStream_t s) {
  router_select_qdq<<<dim3(M), dim3(256), 0, s>>>(M, H, E, k, route_scale, router_logit_parts(M, H),
                                                            logits, gate_b, x, ids, rw, x_q, x_s);
}

}  // namespace moe
