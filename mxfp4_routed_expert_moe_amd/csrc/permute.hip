// Token-to-expert permutation: a stable counting sort of the M*k (token, slot) pairs by expert id.
//
// The expert GEMMs process the rows of one expert together (the grouped layout of the paper
// "DeepSeek-V4-Flash on AMD gfx90a", section 7.1, and the route-direct chain of the page "DeepSeek V4 Flash
// REAP/XPU B70 Handoff"); the order inside an expert is ascending pair id t*k + j, so results never depend on
// scheduling. No global atomics and no in-kernel counter resets: block e counts the pairs of expert e and of
// the experts below it (per lane, then over the wave), finds its rank among the active experts from a
// presence mask of all ids, and compacts the pairs of expert e with wave ballots.
#include "kernels.h"
#include "moe_device.h"
#include "route_device.h"

namespace moe {

constexpr int kPermWaves = 16;
constexpr int kPermVec = 12;   // 16-byte id vectors per lane and batch: a batch is 3,072 ids per wave

// One batch of a wave's segment: lane l holds ids b0 + 256 u + 4 l .. + 3 in v[u] (-1 past end) for the
// vectors u that start before end (the others are left as they are and never read). With VEC each vector is
// one 16-byte load (ids 16-byte aligned); the batch's loads all go out before any is used.
template <bool VEC>
__device__ __forceinline__ void load_id_batch(const int32_t* __restrict__ ids, int b0, int end, int lane, int4* v) {
#pragma unroll
  for (int u = 0; u < kPermVec; ++u) {
    if (b0 + 256 * u >= end) break;   // (wave-uniform)
    const int i = b0 + 256 * u + 4 * lane;
    if (VEC && i + 4 <= end) {
      v[u] = *reinterpret_cast<const int4*>(ids + i);
    } else {
      v[u].x = i < end ? ids[i] : -1;
      v[u].y = i + 1 < end ? ids[i + 1] : -1;
      v[u].z = i + 2 < end ? ids[i + 2] : -1;
      v[u].w = i + 3 < end ? ids[i + 3] : -1;
    }
  }
}

// ACTIVE = false (active == nullptr: a caller whose expert GEMMs read the row-tile map instead): no presence
// mask and no active list, a third less work per id.
template <bool VEC, bool ACTIVE>
__global__ __launch_bounds__(1024) void permute_kernel(int P, int E, const int32_t* __restrict__ ids,
                                                       int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
                                                       int32_t* __restrict__ pairs, int32_t* __restrict__ inv,
                                                       int32_t* __restrict__ active) {
  __shared__ unsigned long long present[4];   // bit x: some pair has expert id x (x < 256)
  __shared__ int wave_cnt[kPermWaves], wave_below[kPermWaves];
  __shared__ int base_off;
  const int e = blockIdx.x;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  if (tid < 4) present[tid] = 0ull;
  __syncthreads();
  // each wave owns a contiguous segment of the pair list (a multiple of 256 long), read in batches of
  // kPermVec vectors per lane. Block e counts the pairs of expert e and those of lower experts (per lane,
  // then over the wave), and every block collects which ids occur (a 256-bit mask: its rank among the
  // active experts and their number).
  constexpr int kBatch = 256 * kPermVec;
  const int seg = ((P + kPermWaves * 256 - 1) / (kPermWaves * 256)) * 256;
  const int beg = wave * seg, end = min(P, beg + seg);
  int mine = 0, lower = 0;
  unsigned long long pm0 = 0ull, pm1 = 0ull, pm2 = 0ull, pm3 = 0ull;
  int4 v[kPermVec];
  auto count = [&](int x) {
    const bool ok = x >= 0 && x < E;
    mine += (ok && x == e) ? 1 : 0;
    lower += (ok && x < e) ? 1 : 0;
    if constexpr (!ACTIVE) return;
    const unsigned long long bit = ok ? 1ull << (x & 63) : 0ull;
    const int q = x >> 6;
    pm0 |= q == 0 ? bit : 0ull;
    pm1 |= q == 1 ? bit : 0ull;
    pm2 |= q == 2 ? bit : 0ull;
    pm3 |= q == 3 ? bit : 0ull;
  };
  for (int b0 = beg; b0 < end; b0 += kBatch) {
    load_id_batch<VEC>(ids, b0, end, lane, v);
#pragma unroll
    for (int u = 0; u < kPermVec; ++u) {
      if (b0 + 256 * u >= end) break;   // (wave-uniform)
      count(v[u].x);
      count(v[u].y);
      count(v[u].z);
      count(v[u].w);
    }
  }
  // sums and ORs over the wave, then over the block (integer: order-free)
  for (int off = 32; off >= 1; off >>= 1) {
    mine += __shfl_xor(mine, off, 64);
    lower += __shfl_xor(lower, off, 64);
    if constexpr (ACTIVE) {
      pm0 |= __shfl_xor(pm0, off, 64);
      pm1 |= __shfl_xor(pm1, off, 64);
      pm2 |= __shfl_xor(pm2, off, 64);
      pm3 |= __shfl_xor(pm3, off, 64);
    }
  }
  if (lane == 0) {
    wave_cnt[wave] = mine;
    wave_below[wave] = lower;
    if constexpr (ACTIVE) {
      atomicOr(&present[0], pm0);
      atomicOr(&present[1], pm1);
      atomicOr(&present[2], pm2);
      atomicOr(&present[3], pm3);
    }
  }
  __syncthreads();
  if (tid == 0) {
    int off = 0, cnt = 0;
    for (int w = 0; w < kPermWaves; ++w) {
      off += wave_below[w];
      cnt += wave_cnt[w];
    }
    base_off = off;
    counts[e] = cnt;
    offsets[e] = off;
    if constexpr (ACTIVE) {   // rank of e among the active experts (ascending id), and their number
      int rank = 0, n_active = 0;
      for (int q = 0; q < 4; ++q) {
        const unsigned long long m = present[q];
        n_active += __popcll(m);
        if (64 * q + 63 < e) rank += __popcll(m);
        else if (64 * q <= e) rank += __popcll(m & ((1ull << (e & 63)) - 1ull));
      }
      if (cnt > 0) active[rank] = e;   // positions < n_active
      if (e >= n_active) active[e] = -1;   // padding: positions >= n_active, disjoint from the above
    }
    if (e == E - 1) offsets[E] = off + cnt;
  }
  __syncthreads();
  if (wave_cnt[wave] == 0) return;   // (wave-uniform) no pair of expert e in this segment
  int base = base_off;
  for (int w = 0; w < wave; ++w) base += wave_cnt[w];
  // stable compaction: pair i goes to base + (hits of expert e before it in the segment). Per vector,
  // lane l's rank = hits in lanes below l (one ballot per component) + hits in its own earlier components.
  const unsigned long long below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int b0 = beg; b0 < end; b0 += kBatch) {
    if (end - beg > kBatch) load_id_batch<VEC>(ids, b0, end, lane, v);   // else: the batch is still in v
#pragma unroll
    for (int u = 0; u < kPermVec; ++u) {
      if (b0 + 256 * u >= end) break;   // (wave-uniform)
      const bool h0 = v[u].x == e, h1 = v[u].y == e, h2 = v[u].z == e, h3 = v[u].w == e;
      const unsigned long long m0 = __ballot(h0), m1 = __ballot(h1), m2 = __ballot(h2), m3 = __ballot(h3);
      int pos = base + __popcll(m0 & below) + __popcll(m1 & below) + __popcll(m2 & below) + __popcll(m3 & below);
      const int i = b0 + 256 * u + 4 * lane;
      if (h0) {
        pairs[pos] = i;
        if (inv) inv[i] = pos;
        ++pos;
      }
      if (h1) {
        pairs[pos] = i + 1;
        if (inv) inv[i + 1] = pos;
        ++pos;
      }
      if (h2) {
        pairs[pos] = i + 2;
        if (inv) inv[i + 2] = pos;
        ++pos;
      }
      if (h3) {
        pairs[pos] = i + 3;
        if (inv) inv[i + 3] = pos;
      }
      base += __popcll(m0) + __popcll(m1) + __popcll(m2) + __popcll(m3);
    }
  }
}

// Up to 1024 pairs (decode widths): one block. LDS histogram, block scan of the counts and of the
// active flags, and the stable rank of pair p inside its expert = the number of earlier pairs with the
// same id (one LDS sweep per thread).
constexpr int kSmallPairs = 1024;

// Thread tid holds the id of pair tid in v (-1 past P); sid, hist, scan, ascan are the block's LDS.
// Called by all threads of the block.
__device__ __forceinline__ void counting_sort_small(int P, int E, int v, int* sid, int* hist, int* scan, int* ascan,
                                                    int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
                                                    int32_t* __restrict__ pairs, int32_t* __restrict__ inv,
                                                    int32_t* __restrict__ active) {
  const int tid = threadIdx.x;
  if (tid < 256) hist[tid] = 0;
  const bool ok = v >= 0 && v < E;
  sid[tid] = ok ? v : -1;
  __syncthreads();
  if (ok) atomicAdd(&hist[v], 1);   // integer counts: order-free
  __syncthreads();
  if (tid < 256) {
    scan[tid] = tid < E ? hist[tid] : 0;
    ascan[tid] = (tid < E && hist[tid] > 0) ? 1 : 0;
  }
  __syncthreads();
  for (int d = 1; d < 256; d <<= 1) {   // inclusive Hillis-Steele scans
    int a = 0, b = 0;
    if (tid < 256 && tid >= d) {
      a = scan[tid - d];
      b = ascan[tid - d];
    }
    __syncthreads();
    if (tid < 256) {
      scan[tid] += a;
      ascan[tid] += b;
    }
    __syncthreads();
  }
  const int n_active = ascan[255];
  if (tid < E) {
    const int c = hist[tid];
    counts[tid] = c;
    offsets[tid] = scan[tid] - c;
    if (active != nullptr) {
      if (c > 0) active[ascan[tid] - 1] = tid;   // positions < n_active
      if (tid >= n_active) active[tid] = -1;      // padding: positions >= n_active, disjoint from the above
    }
  }
  if (tid == 0) offsets[E] = scan[255];
  if (ok) {
    int r = 0;
    for (int q = 0; q < tid; ++q) r += (sid[q] == v) ? 1 : 0;
    const int pos = scan[v] - hist[v] + r;
    pairs[pos] = tid;
    if (inv) inv[tid] = pos;
  }
}

__global__ __launch_bounds__(1024) void permute_small_kernel(int P, int E, const int32_t* __restrict__ ids,
                                                             int32_t* __restrict__ counts,
                                                             int32_t* __restrict__ offsets,
                                                             int32_t* __restrict__ pairs, int32_t* __restrict__ inv,
                                                             int32_t* __restrict__ active) {
  __shared__ int sid[kSmallPairs];
  __shared__ int hist[256];
  __shared__ int scan[256];
  __shared__ int ascan[256];
  const int v = threadIdx.x < P ? ids[threadIdx.x] : -1;
  counting_sort_small(P, E, v, sid, hist, scan, ascan, counts, offsets, pairs, inv, active);
}

// Decode widths (M <= 64): wave w selects the experts of tokens w, w + 16, ... with the router's own
// selection code (so ids and route weights equal the separate select kernel's bit for bit). A token's
// k experts are distinct, so expert e's pairs are one per token: bit t of the LDS mask of expert e says
// that token t chose it. The count is the mask's popcount, and the stable rank of pair (t, j) inside its
// expert is the number of set bits below t. One wave scans the counts; no per-pair sweep.
template <int NJ>
__global__ __launch_bounds__(1024) void select_permute_small_kernel(
    int M, int E, int k, float route_scale, int nparts, const float* __restrict__ logits,
    const float* __restrict__ gate_b, int32_t* __restrict__ ids, float* __restrict__ rw, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ pairs, int32_t* __restrict__ inv,
    int32_t* __restrict__ active, int32_t* __restrict__ out_rows) {
  __shared__ int sid[kSmallPairs];
  __shared__ unsigned long long emask[256];
  __shared__ int soff[256];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  if (tid < 256) emask[tid] = 0ull;
  __syncthreads();
  for (int t = wave; t < M; t += kSmallPairs / 64)
    select_token<NJ>(t, M, E, k, route_scale, nparts, logits, gate_b, lane, ids, rw, sid, emask);
  __syncthreads();
  if (wave == 0) {   // counts, offsets and the active list: lane l owns experts 4l .. 4l + 3
    int c[4], csum = 0, fsum = 0;
    unsigned long long em[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) em[i] = emask[4 * lane + i];   // all four reads in flight (256 entries)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = 4 * lane + i;
      c[i] = e < E ? __popcll(em[i]) : 0;
      csum += c[i];
      fsum += c[i] > 0 ? 1 : 0;
    }
    const int ic = wave_incl_scan(csum), ifl = wave_incl_scan(fsum);   // inclusive scans over the lanes
    int oc = ic - csum, of = ifl - fsum;
    const int total = __builtin_amdgcn_readlane(ic, 63), n_active = __builtin_amdgcn_readlane(ifl, 63);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = 4 * lane + i;
      if (e < E) {
        counts[e] = c[i];
        offsets[e] = oc;
        soff[e] = oc;
        if (c[i] > 0) active[of++] = e;   // positions < n_active
        oc += c[i];
      }
    }
    for (int i = n_active + lane; i < E; i += 64) active[i] = -1;   // padding, disjoint from the above
    if (lane == 0) offsets[E] = total;
  }
  __syncthreads();
  const int P = M * k;
  if (tid < P) {
    const int t = tid / k, v = sid[tid];
    const int pos = soff[v] + __popcll(emask[v] & ((1ull << t) - 1ull));
    pairs[pos] = tid;
    if (inv) inv[tid] = pos;
    if (out_rows) {   // rank of this expert among the token's k (distinct) ids
      int r = 0;
      for (int j = 0; j < k; ++j) r += sid[t * k + j] < v ? 1 : 0;
      out_rows[pos] = t * k + r;
    }
  }
}

void launch_permute(int P, int E, const int32_t* ids, int32_t* counts, int32_t* offsets, int32_t* pairs,
                    int32_t* inv, int32_t* active, hipStream_t s) {
  if (P <= kSmallPairs)
    permute_small_kernel<<<dim3(1), dim3(kSmallPairs), 0, s>>>(P, E, ids, counts, offsets, pairs, inv, active);
  else {
    const bool vec = (reinterpret_cast<uintptr_t>(ids) & 15u) == 0;
    const dim3 g(E), b(kPermWaves * 64);
    if (vec && active) permute_kernel<true, true><<<g, b, 0, s>>>(P, E, ids, counts, offsets, pairs, inv, active);
    else if (vec) permute_kernel<true, false><<<g, b, 0, s>>>(P, E, ids, counts, offsets, pairs, inv, active);
    else if (active) permute_kernel<false, true><<<g, b, 0, s>>>(P, E, ids, counts, offsets, pairs, inv, active);
    else permute_kernel<false, false><<<g, b, 0, s>>>(P, E, ids, counts, offsets, pairs, inv, active);
  }
}

void launch_select_permute_small(int M, int H, int E, int k, float route_scale, const float* logits,
                                 const float* gate_b, int32_t* ids, float* rw, int32_t* counts,
                                 int32_t* offsets, int32_t* pairs, int32_t* inv, int32_t* active, int32_t* out_rows,
                                 hipStream_t s) {
  const int parts = router_logit_parts(M, H);
  if (E <= 128)
    select_permute_small_kernel<2><<<dim3(1), dim3(kSmallPairs), 0, s>>>(M, E, k, route_scale, parts, logits, gate_b,
                                                                         ids, rw, counts, offsets, pairs, inv, active,
                                                                         out_rows);
  else
    select_permute_small_kernel<4><<<dim3(1), dim3(kSmallPairs), 0, s>>>(M, E, k, route_scale, parts, logits, gate_b,
                                                                         ids, rw, counts, offsets, pairs, inv, active,
                                                                         out_rows);
}

}  // namespace moe
