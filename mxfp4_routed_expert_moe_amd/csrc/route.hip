// Router of the routed-MoE layer on gfx950, and the per-32 E4M3 QDQ of its input rows.
//
// Gate (page "Native 1017 DSpark draft on the NVLink pair (N1-NATIVE)", section 2 "Gate"): fp32 logits of the raw bf16 x
// against the fp32 gate weight, scores sqrt(softplus(l)), top-k of scores + bias (the bias only
// selects), gathered scores normalised by their sum + 1e-20 and scaled by the route scale.
// Activation QDQ (same section, "Quantized linear"): per 32 inputs, E8M0 scale
// 2^ceil(log2(max(amax, 1e-4) / 448)) and E4M3 codes; done once per row and shared by every expert.
//
// Fixed fp32 orders (recorded so routing is reproducible): each logit is accumulated in fp32 as
// strided partial sums (small M: per 512-wide chunk of H, 64 lanes x an 8-FMA chain, then a
// butterfly, then the chunks added in ascending order; large M: per quarter of H, the bf16 matrix
// cores' 32-wide K steps in ascending order, three exact split-gate products per step, then the
// quarters added in ascending order); the normalising sum adds the k weights in slot order.
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
  // time, so that their butterflies overlap, and the x slices of the next four are loaded before the current
  // four are added up (each token's order is unchanged).
  auto xload = [&](int t) {
    return (ok && t < M) ? *reinterpret_cast<const u32x4*>(x + (size_t)t * H + h) : u32x4{0u, 0u, 0u, 0u};
  };
  auto dot8v = [&](const u32x4& xv) {
    float a = 0.0f;
    if (ok) {
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
  u32x4 xn[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) xn[u] = xload(u);
  int t = 0;
  for (; t + 4 <= M; t += 4) {
    u32x4 xc[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      xc[u] = xn[u];
      xn[u] = xload(t + 4 + u);   // the next group (zeros past M)
    }
    float a[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) a[u] = wave_sum_lane0(dot8v(xc[u]));   // the butterfly, as lane 0 forms it
    if (lane == 0)
#pragma unroll
      for (int u = 0; u < 4; ++u) part[(size_t)chunk * plane + (size_t)(t + u) * E + e] = a[u];
  }
  // the last M % 4 tokens: their slices are in xn[0 .. M % 4 - 1]
#pragma unroll
  for (int u = 0; u < 3; ++u) {
    if (t + u >= M) break;
    const float a = wave_sum_lane0(dot8v(xn[u]));
    if (lane == 0) part[(size_t)chunk * plane + (size_t)(t + u) * E + e] = a;
  }
}

// Larger M, on the bf16 matrix cores. Each fp32 gate value is split into three bf16 parts whose sum is
// exactly the value (hi = the top 8 significand bits, mid = the next 8 of the remainder, lo = the rest,
// which has at most 8 bits): every product x * part is exact in fp32 (bf16 x bf16), so only the fp32
// accumulation rounds, as in the vector path. The split is made in registers from the fp32 gate tile in
// LDS, so the gate is read as it is stored and nothing is prepared or written per call.
constexpr int kLargeParts = 4;

__device__ __forceinline__ void split_gate8(const f32x4& lo4, const f32x4& hi4, u32x4& p_hi, u32x4& p_mid,
                                            u32x4& p_lo) {
  uint32_t h[8], m[8], l[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float v = i < 4 ? lo4[i] : hi4[i - 4];
    const uint32_t vh = __float_as_uint(v) & 0xFFFF0000u;
    const float r1 = v - __uint_as_float(vh);                       // exact: the low 16 significand bits
    const uint32_t vm = __float_as_uint(r1) & 0xFFFF0000u;
    const float r2 = r1 - __uint_as_float(vm);                      // exact, at most 8 significant bits
    h[i] = vh >> 16;
    m[i] = vm >> 16;
    l[i] = __float_as_uint(r2) >> 16;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    p_hi[i] = h[2 * i] | (h[2 * i + 1] << 16);
    p_mid[i] = m[2 * i] | (m[2 * i + 1] << 16);
    p_lo[i] = l[2 * i] | (l[2 * i + 1] << 16);
  }
}

// Block: 128 tokens x 128 experts over one quarter of H (the quarters are added in ascending order by the
// select kernel). Per 32-wide K step, the block's x tile (128 rows x 64 B, bf16) and fp32 gate tile
// (128 rows x 128 B) stream into a three-stage LDS ring through direct global -> LDS copies, issued two
// steps ahead; per wave one x copy (16 rows) and two gate copies (8 rows each). The 16-byte chunks of each
// LDS row are XOR-swizzled (x: chunk ^ ((r ^ r >> 2) & 3); gate: chunk ^ (r & 7)) so that the 16 rows of a
// fragment read distinct banks.
// Wave w computes all 128 tokens (eight A tiles) x experts 16 w .. + 15 (one B tile, so each gate fragment is
// split once per block): per step and tile the hi, mid and lo products, in that order (v_mfma_f32_16x16x32_bf16: lane l
// supplies row l % 16 of A and column l % 16 of B, inputs 8 (l / 16) .. + 7 of the step; the result
// (4 (l / 16) + v, l % 16) is accumulator v of lane l).
constexpr int kRtStages = 3;
struct RouterStage {
  uint16_t x[128 * 32];
  float g[128 * 32];
};

__device__ __forceinline__ int rt_key(int r) { return (r ^ (r >> 2)) & 3; }

__global__ __launch_bounds__(512, 1) void router_logits_mfma(int M, int H, int E, const uint16_t* __restrict__ x,
                                                             const float* __restrict__ gate, float* __restrict__ part) {
  __shared__ __align__(16) RouterStage ring[kRtStages];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, r16 = lane & 15, g = lane >> 4;
  const int t0 = blockIdx.x * 128, e0 = blockIdx.z * 128;
  const int hq = H / kLargeParts, hbeg = blockIdx.y * hq, nk = hq / 32;
  // copy sources (rows past M or E repeat the last row): x - lane i of wave w fills LDS row 16 w + i / 4,
  // physical chunk i % 4 (logical (i % 4) ^ key); gate copy c - lane i fills row 16 w + 8 c + i / 8,
  // physical chunk i % 8 (logical (i % 8) ^ (row & 7))
  const int dr = 16 * wave + (lane >> 2), lc = (lane & 3) ^ rt_key(dr);
  const uint16_t* xsrc = x + (size_t)min(t0 + dr, M - 1) * H + hbeg + 8 * lc;
  const float* gsrc[2];
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const int gr = 16 * wave + 8 * c + (lane >> 3), gc = (lane & 7) ^ (gr & 7);
    gsrc[c] = gate + (size_t)min(e0 + gr, E - 1) * H + hbeg + 4 * gc;
  }
  auto copy16 = [](const void* src, void* lds) {
    __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)lds, 16, 0, 0);
  };
  auto issue = [&](int s) {
    RouterStage& st = ring[s % kRtStages];
    const int h = s * 32;
    copy16(xsrc + h, &st.x[16 * wave * 32]);
#pragma unroll
    for (int c = 0; c < 2; ++c) copy16(gsrc[c] + h, &st.g[(16 * wave + 8 * c) * 32]);
  };
  // wave w: experts 16 w .. 16 w + 15 (one B fragment, split once per block) for all 128 tokens
  f32x4 acc[8];
#pragma unroll
  for (int a = 0; a < 8; ++a) acc[a] = f32x4{0.f, 0.f, 0.f, 0.f};
  issue(0);
  if (nk > 1) issue(1);
  for (int s = 0; s < nk; ++s) {
    // this wave's copies of step s have landed (those of step s + 1 may still be in flight), then meet
    if (s + 1 < nk) asm volatile("s_waitcnt vmcnt(3) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    else asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    if (s + 2 < nk) issue(s + 2);   // into the slot read at step s - 1: every wave is past it
    const RouterStage& st = ring[s % kRtStages];
    u32x4 A[8], B[3];
#pragma unroll
    for (int a = 0; a < 8; ++a) {
      const int r = 16 * a + r16;
      A[a] = *reinterpret_cast<const u32x4*>(&st.x[r * 32 + 8 * (g ^ rt_key(r))]);
    }
    {
      const int r = 16 * wave + r16;
      const f32x4 lo4 = *reinterpret_cast<const f32x4*>(&st.g[r * 32 + 4 * ((2 * g) ^ (r & 7))]);
      const f32x4 hi4 = *reinterpret_cast<const f32x4*>(&st.g[r * 32 + 4 * ((2 * g + 1) ^ (r & 7))]);
      split_gate8(lo4, hi4, B[0], B[1], B[2]);
    }
#pragma unroll
    for (int a = 0; a < 8; ++a)
#pragma unroll
      for (int q = 0; q < 3; ++q)
        acc[a] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, A[a]),
                                                         __builtin_bit_cast(bf16x8, B[q]), acc[a], 0, 0, 0);
  }
  float* out = part + (size_t)blockIdx.y * M * E;
  const int e = e0 + 16 * wave + r16;
#pragma unroll
  for (int a = 0; a < 8; ++a)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int t = t0 + 16 * a + 4 * g + v;
      if (t < M && e < E) out[(size_t)t * E + e] = acc[a][v];
    }
}

// One wave per token, four tokens per block: scores, biased top-k, normalisation; with qdq the wave also
// QDQs the token's row (one 32-wide block per lane per pass); otherwise the logits kernel has.
template <int NJ>
__global__ __launch_bounds__(256) void router_select_qdq(int M, int H, int E, int k, float route_scale,
                                                         int nparts, int qdq, const float* __restrict__ logits,
                                                         const float* __restrict__ gate_b,
                                                         const uint16_t* __restrict__ x,
                                                         int32_t* __restrict__ ids, float* __restrict__ rw,
                                                         uint8_t* __restrict__ x_q, uint8_t* __restrict__ x_s) {
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (t >= M) return;
  select_token<NJ>(t, M, E, k, route_scale, nparts, logits, gate_b, lane, ids, rw, nullptr, nullptr);
  if (!qdq) return;
  const int nb = H / 32;
  for (int b = lane; b < nb; b += 64)
    qdq_block32(x + (size_t)t * H + b * 32, x_q + (size_t)t * H + b * 32, x_s + (size_t)t * nb + b);
}

int router_logit_parts(int M, int H, bool mfma_order) {
  return (M <= kSmallM && !mfma_order) ? (H + kChunkH - 1) / kChunkH : kLargeParts;
}

void launch_router_logits(int M, int H, int E, const uint16_t* x, const float* gate_w, float* logits,
                          uint8_t* x_q, uint8_t* x_s, bool mfma_order, hipStream_t s) {
  if (M <= kSmallM && !mfma_order) {
    router_logits_small<<<dim3((E + 3) / 4, router_logit_parts(M, H)), dim3(256), 0, s>>>(M, H, E, x, gate_w, logits,
                                                                                           x_q, x_s);
  } else {
    router_logits_mfma<<<dim3((M + 127) / 128, kLargeParts, (E + 127) / 128), dim3(512), 0, s>>>(M, H, E, x, gate_w,
                                                                                                logits);
  }
}

void launch_router_select_qdq(int M, int H, int E, int k, float route_scale, const float* logits,
                              const float* gate_b, const uint16_t* x, int32_t* ids, float* rw,
                              uint8_t* x_q, uint8_t* x_s, bool mfma_order, hipStream_t s) {
  const int parts = router_logit_parts(M, H, mfma_order);
  const int qdq = (M > kSmallM || mfma_order) ? 1 : 0;   // at decode widths the small logits kernel QDQs x
  if (E <= 128)
    router_select_qdq<2><<<dim3((M + 3) / 4), dim3(256), 0, s>>>(M, H, E, k, route_scale, parts, qdq, logits, gate_b,
                                                                 x, ids, rw, x_q, x_s);
  else
    router_select_qdq<4><<<dim3((M + 3) / 4), dim3(256), 0, s>>>(M, H, E, k, route_scale, parts, qdq, logits, gate_b,
                                                                 x, ids, rw, x_q, x_s);
}

}  // namespace moe
