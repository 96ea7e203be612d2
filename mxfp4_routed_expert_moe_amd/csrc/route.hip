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
// butterfly, then the chunks added in ascending order; large M: per quarter of H, 32-wide FMA chains
// summed into a running total, then the quarters added in ascending order); the normalising sum adds
// the k weights in slot order.
#include "kernels.h"
#include "moe_device.h"
#include "route_device.h"

namespace moe {

constexpr int kSmallM = kRouterSmallM;
constexpr int kChunkH = 512;   // H columns per partial logit at small M

// Small M: one wave per (expert, 512-wide chunk of H); lane l covers 8 consecutive columns. Every
// wave handles all M <= 64 tokens, so each gate element is read once. The wave's fp32 partial sum
// (8 FMA chain per lane, then a butterfly over the 64 lanes) goes to part[chunk][t][e]; the select
// kernel adds the chunks in ascending order. The same blocks also QDQ the rows of x: block (b, chunk)
// takes the chunk's 32-wide blocks of tokens b, b + gridDim.x, ...
__global__ __launch_bounds__(256) void router_logits_small(int M, int H, int E, const uint16_t* __restrict__ x,
                                                           const float* __restrict__ gate_w,
                                                           float* __restrict__ part, uint8_t* __restrict__ x_q,
                                                           uint8_t* __restrict__ x_s) {
  const int lane = threadIdx.x & 63;
  const int e = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int chunk = blockIdx.y;
  const int h = chunk * kChunkH + lane * 8;
  const bool ok = h < H && e < E;
  float4 w0 = make_float4(0.f, 0.f, 0.f, 0.f), w1 = w0;
  if (ok) {   // the gate loads go out first
    w0 = *reinterpret_cast<const float4*>(gate_w + (size_t)e * H + h);
    w1 = *reinterpret_cast<const float4*>(gate_w + (size_t)e * H + h + 4);
  }
  {  // the QDQ of this chunk's 32-wide blocks of tokens blockIdx.x, blockIdx.x + gridDim.x, ...
    const int nb = min(kChunkH, H - chunk * kChunkH) / 32, b0 = chunk * (kChunkH / 32);
    for (int it = threadIdx.x;; it += 256) {
      const int t = blockIdx.x + (it / nb) * gridDim.x, b = b0 + it % nb;
      if (t >= M) break;
      qdq_block32(x + (size_t)t * H + b * 32, x_q + (size_t)t * H + b * 32, x_s + (size_t)t * (H / 32) + b);
    }
  }
  if (e >= E) return;
  const size_t plane = (size_t)M * E;
  // one token's partial: an 8-FMA chain per lane, then a butterfly over the 64 lanes. Four tokens at a
  // time, so that their butterflies overlap (each token's order is unchanged).
  auto dot8 = [&](int t) {
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
    return a;
  };
  int t = 0;
  for (; t + 4 <= M; t += 4) {
    float a[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) a[u] = dot8(t + u);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1)
#pragma unroll
      for (int u = 0; u < 4; ++u) a[u] += __shfl_xor(a[u], off, 64);
    if (lane == 0)
#pragma unroll
      for (int u = 0; u < 4; ++u) part[(size_t)chunk * plane + (size_t)(t + u) * E + e] = a[u];
  }
  for (; t < M; ++t) {
    float a = dot8(t);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) a += __shfl_xor(a, off, 64);
    if (lane == 0) part[(size_t)chunk * plane + (size_t)t * E + e] = a;
  }
}

// Larger M: a block computes 64 tokens x 128 experts over one quarter of H (the quarters are added in
// ascending order by the select kernel). Per 32-column chunk, x (transposed, fp32) and the gate tile
// (transposed) sit in LDS; thread (tg, eg) owns tokens 8 tg .. 8 tg + 7 and experts 4 eg .. 4 eg + 3,
// reads two float4 of x and one float4 of the gate per column, and runs 32 FMA chains. Each chunk's
// 32-term chain is added to a running fp32 total.
constexpr int kLargeParts = 4;

__global__ __launch_bounds__(256) void router_logits_tiled(int M, int H, int E, const uint16_t* __restrict__ x,
                                                           const float* __restrict__ gate_w,
                                                           float* __restrict__ part) {
  __shared__ __align__(16) float xs[32][64];
  __shared__ __align__(16) float ws[32][128];
  const int tid = threadIdx.x;
  const int t0 = blockIdx.x * 64, e0 = blockIdx.z * 128;
  const int hq = H / kLargeParts, hbeg = blockIdx.y * hq;
  const int tg = tid >> 5, eg = tid & 31;
  float acc[8][4];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = 0.0f;
  for (int h0 = hbeg; h0 < hbeg + hq; h0 += 32) {
    {  // x tile: 64 tokens x 32 columns; thread loads 8 columns of one token
      const int r = tid >> 2, c = (tid & 3) * 8;
      u32x4 v = {0u, 0u, 0u, 0u};
      if (t0 + r < M) v = *reinterpret_cast<const u32x4*>(x + (size_t)(t0 + r) * H + h0 + c);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        xs[c + 2 * j][r] = bits_to_f32(v[j] << 16);
        xs[c + 2 * j + 1][r] = bits_to_f32(v[j] & 0xFFFF0000u);
      }
    }
    {  // gate tile: 128 experts x 32 columns; thread loads 16 columns of one expert
      const int r = tid >> 1, c = (tid & 1) * 16;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        float4 w = make_float4(0.f, 0.f, 0.f, 0.f);
        if (e0 + r < E) w = *reinterpret_cast<const float4*>(gate_w + (size_t)(e0 + r) * H + h0 + c + 4 * q);
        ws[c + 4 * q][r] = w.x;
        ws[c + 4 * q + 1][r] = w.y;
        ws[c + 4 * q + 2][r] = w.z;
        ws[c + 4 * q + 3][r] = w.w;
      }
    }
    __syncthreads();
    float p[8][4];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) p[i][j] = 0.0f;
#pragma unroll 8
    for (int kk = 0; kk < 32; ++kk) {
      const float4 xa = *reinterpret_cast<const float4*>(&xs[kk][8 * tg]);
      const float4 xb = *reinterpret_cast<const float4*>(&xs[kk][8 * tg + 4]);
      const float4 wv = *reinterpret_cast<const float4*>(&ws[kk][4 * eg]);
      const float xv[8] = {xa.x, xa.y, xa.z, xa.w, xb.x, xb.y, xb.z, xb.w};
      const float wr[4] = {wv.x, wv.y, wv.z, wv.w};
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) p[i][j] = __builtin_fmaf(xv[i], wr[j], p[i][j]);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] += p[i][j];
    __syncthreads();
  }
  const size_t plane = (size_t)M * E;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int t = t0 + 8 * tg + i;
    if (t >= M) continue;
    const int e = e0 + 4 * eg;
    float* dst = part + (size_t)blockIdx.y * plane + (size_t)t * E + e;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (e + j < E) dst[j] = acc[i][j];
  }
}

// One block per token. Wave 0: scores, biased top-k, normalisation; at M > 64 all four waves also
// QDQ the token's row (one 32-wide block per thread); at M <= 64 the logits kernel has done it.
__global__ __launch_bounds__(256) void router_select_qdq(int M, int H, int E, int k, float route_scale,
                                                         int nparts, const float* __restrict__ logits,
                                                         const float* __restrict__ gate_b,
                                                         const uint16_t* __restrict__ x,
                                                         int32_t* __restrict__ ids, float* __restrict__ rw,
                                                         uint8_t* __restrict__ x_q, uint8_t* __restrict__ x_s) {
  const int t = blockIdx.x;
  if (threadIdx.x < 64)
    select_token(t, M, E, k, route_scale, nparts, logits, gate_b, threadIdx.x, ids, rw, nullptr, nullptr);
  if (M <= kSmallM) return;
  const int nb = H / 32;
  for (int b = threadIdx.x; b < nb; b += 256)
    qdq_block32(x + (size_t)t * H + b * 32, x_q + (size_t)t * H + b * 32, x_s + (size_t)t * nb + b);
}

int router_logit_parts(int M, int H) { return M <= kSmallM ? (H + kChunkH - 1) / kChunkH : kLargeParts; }

void launch_router_logits(int M, int H, int E, const uint16_t* x, const float* gate_w, float* logits,
                          uint8_t* x_q, uint8_t* x_s, hipStream_t s) {
  if (M <= kSmallM) {
    router_logits_small<<<dim3((E + 3) / 4, router_logit_parts(M, H)), dim3(256), 0, s>>>(M, H, E, x, gate_w, logits,
                                                                                           x_q, x_s);
  } else {
    router_logits_tiled<<<dim3((M + 63) / 64, kLargeParts, (E + 127) / 128), dim3(256), 0, s>>>(M, H, E, x, gate_w,
                                                                                            logits);
  }
}

void launch_router_select_qdq(int M, int H, int E, int k, float route_scale, const float* logits,
                              const float* gate_b, const uint16_t* x, int32_t* ids, float* rw,
                              uint8_t* x_q, uint8_t* x_s, hipStream_t s) {
  router_select_qdq<<<dim3(M), dim3(256), 0, s>>>(M, H, E, k, route_scale, router_logit_parts(M, H),
                                                            logits, gate_b, x, ids, rw, x_q, x_s);
}

}  // namespace moe
