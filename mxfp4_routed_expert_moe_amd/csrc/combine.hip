// Fixed-order combine of the routed experts (page "Native 1017 DSpark draft on the NVLink pair (N1-NATIVE)", section 2
// "MoE"): y = 0 in fp32; for the token's expert ids in ascending order, y += that expert's bf16
// output (as fp32); then y += the shared expert's bf16 output; out = bf16(y). A block covers 512 columns
// of one token (8 per thread); no atomics: the order of the adds is fixed by the ids, so the result is
// run-to-run identical.
#include "kernels.h"
#include "moe_device.h"

namespace moe {

__global__ __launch_bounds__(64) void combine_kernel(int H, int k, const int32_t* __restrict__ ids,
                                                     const uint16_t* __restrict__ slot_out,
                                                     const uint16_t* __restrict__ shared_out,
                                                     uint16_t* __restrict__ out) {
  const int t = blockIdx.y;
  // slots of this token sorted by ascending expert id (stable in slot order; k <= 8)
  // (ids == nullptr: the rows are already in ascending-id order, as the decode-width layer writes them, and
  // no id needs to be read)
  int order[8], key[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    order[j] = j;
    key[j] = (j < k && ids) ? ids[(size_t)t * k + j] : 0x7FFFFFFF;
  }
  if (ids) {
#pragma unroll
    for (int a = 1; a < 8; ++a)
#pragma unroll
      for (int b = a; b > 0; --b)
        if (key[b] < key[b - 1]) {
          const int tk = key[b]; key[b] = key[b - 1]; key[b - 1] = tk;
          const int to = order[b]; order[b] = order[b - 1]; order[b - 1] = to;
        }
  }
  {
    const int c = blockIdx.x * 512 + threadIdx.x * 8;   // H is a multiple of 128, so c + 8 <= H or c >= H
    if (c >= H) return;
    float acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = 0.0f;
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      if (r < k) {
        // each slot row is read once: non-temporal loads (M = 8192: 106 -> 90 us, alternating builds)
        const u32x4 v = __builtin_nontemporal_load(
            reinterpret_cast<const u32x4*>(slot_out + ((size_t)t * k + order[r]) * H + c));
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          acc[2 * i] = acc[2 * i] + bits_to_f32(v[i] << 16);
          acc[2 * i + 1] = acc[2 * i + 1] + bits_to_f32(v[i] & 0xFFFF0000u);
        }
      }
    }
    if (shared_out) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(shared_out + (size_t)t * H + c);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc[2 * i] = acc[2 * i] + bits_to_f32(v[i] << 16);
        acc[2 * i + 1] = acc[2 * i + 1] + bits_to_f32(v[i] & 0xFFFF0000u);
      }
    }
    u32x4 o;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      o[i] = uint32_t(f32_to_bf16_rne(acc[2 * i])) | (uint32_t(f32_to_bf16_rne(acc[2 * i + 1])) << 16);
    *reinterpret_cast<u32x4*>(out + (size_t)t * H + c) = o;
  }
}

// The same walk over fp32 slot partials (SLOT mode): OFFICIAL rounds each slot (and an fp32 shared
// partial) to bf16 before adding it and writes bf16; otherwise the fp32 slots are summed unrounded, then
// the optional fp32 add input, and the fp32 sums are written.
template <bool OFFICIAL>
__global__ __launch_bounds__(64) void combine_f32_kernel(int H, int k, const int32_t* __restrict__ ids,
                                                         const float* __restrict__ slot, const float* __restrict__ extra,
                                                         const uint16_t* __restrict__ shared_bf16,
                                                         uint16_t* __restrict__ out_bf16, float* __restrict__ out_f32) {
  const int t = blockIdx.y;
  int order[8], key[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    order[j] = j;
    key[j] = (j < k) ? ids[(size_t)t * k + j] : 0x7FFFFFFF;
  }
#pragma unroll
  for (int a = 1; a < 8; ++a)
#pragma unroll
    for (int b = a; b > 0; --b)
      if (key[b] < key[b - 1]) {
        const int tk = key[b]; key[b] = key[b - 1]; key[b - 1] = tk;
        const int to = order[b]; order[b] = order[b - 1]; order[b - 1] = to;
      }
  const int c = blockIdx.x * 512 + threadIdx.x * 8;
  if (c >= H) return;
  float acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = 0.0f;
  auto add8 = [&](const float* src, bool round) {
    const f32x4 v0 = *reinterpret_cast<const f32x4*>(src), v1 = *reinterpret_cast<const f32x4*>(src + 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc[i] = acc[i] + (round ? round_bf16(v0[i]) : v0[i]);
      acc[4 + i] = acc[4 + i] + (round ? round_bf16(v1[i]) : v1[i]);
    }
  };
#pragma unroll
  for (int r = 0; r < 8; ++r)
    if (r < k) add8(slot + ((size_t)t * k + order[r]) * H + c, OFFICIAL);
  if (extra) add8(extra + (size_t)t * H + c, OFFICIAL);
  if (OFFICIAL) {
    if (shared_bf16) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(shared_bf16 + (size_t)t * H + c);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc[2 * i] = acc[2 * i] + bits_to_f32(v[i] << 16);
        acc[2 * i + 1] = acc[2 * i + 1] + bits_to_f32(v[i] & 0xFFFF0000u);
      }
    }
    u32x4 o;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      o[i] = uint32_t(f32_to_bf16_rne(acc[2 * i])) | (uint32_t(f32_to_bf16_rne(acc[2 * i + 1])) << 16);
    *reinterpret_cast<u32x4*>(out_bf16 + (size_t)t * H + c) = o;
  } else {
    float* o = out_f32 + (size_t)t * H + c;
    *reinterpret_cast<f32x4*>(o) = f32x4{acc[0], acc[1], acc[2], acc[3]};
    *reinterpret_cast<f32x4*>(o + 4) = f32x4{acc[4], acc[5], acc[6], acc[7]};
  }
}

void launch_combine_official_f32(int M, int H, int k, const int32_t* ids, const float* slot_f32,
                                 const float* shared_f32, const uint16_t* shared_bf16, uint16_t* out, hipStream_t s) {
  combine_f32_kernel<true><<<dim3((H + 511) / 512, M), dim3(64), 0, s>>>(H, k, ids, slot_f32, shared_f32, shared_bf16,
                                                                         out, nullptr);
}

void launch_combine_sum_f32(int M, int H, int k, const int32_t* ids, const float* slot_f32, const float* add,
                            float* out, hipStream_t s) {
  combine_f32_kernel<false><<<dim3((H + 511) / 512, M), dim3(64), 0, s>>>(H, k, ids, slot_f32, add, nullptr, nullptr,
                                                                          out);
}

void launch_combine(int M, int H, int k, const int32_t* ids, const uint16_t* slot_out, const uint16_t* shared_out,
                    uint16_t* out, hipStream_t s) {
  combine_kernel<<<dim3((H + 511) / 512, M), dim3(64), 0, s>>>(H, k, ids, slot_out, shared_out, out);
}

}  // namespace moe
