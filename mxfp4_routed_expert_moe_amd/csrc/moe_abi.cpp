// C ABI of libmoe (declared in include/moe.h): host-side validation, workspace layout and the
// launch sequence of the routed-MoE layer. No entry point allocates, synchronizes or reads device
// data; every check runs before the first launch and a refusal enqueues nothing.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <mutex>

#include "../../include/moe.h"
#include "kernels.h"

namespace {

using moe::GemmProblem;

// Average rows per expert (M * k / E) from which the routed GEMMs run over the row-tile list. Swept on the
// full-size layer (E 128, k 6) with the 8-row decode passes: M = 128 561 us streamed against 563-565 us tiled,
// M = 192 720 against 567, M = 256 888 against 563-575, M = 384 1220 against 573-585, M = 512 1530 against
// 587-598 us; at M = 64 both 450 us.
constexpr int kTiledRowsPerExpert = MOE_TILED_ROWS_PER_EXPERT;

// Size of the library-owned workspace of moe_forward_noalloc (per GPU).
constexpr size_t kScratchBytes = (size_t)MOE_NOALLOC_SCRATCH_BYTES;

struct WsLayout {
  size_t logits, ids, rw, x_q, x_s, counts, offsets, pairs, inv, out_rows, active, tile_e, tile_r0, tile_info, h_q, h_s, slot,
      sh_q, sh_s, sh_out, scales, xs_sm;
  size_t total;
};

inline size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// Batch-invariant mode: the router runs its matrix-core kernel (one summation order) at every M.
inline bool batch_invariant(const moe_dims* d) { return (d->flags & MOE_FLAG_BATCH_INVARIANT) != 0u; }

WsLayout ws_layout(const moe_dims* d, int64_t M) {
  WsLayout L{};
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += round_up(bytes, 256);
    return o;
  };
  const size_t E = d->num_experts, H = d->hidden, I = d->inter, k = d->top_k, m = (size_t)M;
  // router logits: partial planes at small M; sized so the total never shrinks as M grows (a
  // workspace sized for max_tokens serves every M <= max_tokens)
  const size_t small_rows = std::min<size_t>(m, 64) * (size_t)moe::router_logit_parts(1, (int)H);
  L.logits = take(std::max(m * (size_t)moe::router_logit_parts(1 << 20, (int)H), small_rows) * E * 4);
  L.ids = take(m * k * 4);
  L.rw = take(m * k * 4);
  L.x_q = take(m * H);
  L.x_s = take(m * H / 32);
  L.counts = take(E * 4);
  L.offsets = take((E + 1) * 4);
  L.pairs = take(m * k * 4);
  L.inv = take(m * k * 4);
  L.out_rows = take(m * k * 4);
  L.active = take(E * 4);
  L.tile_e = take((size_t)moe::mfma_max_tiles((int)(m * k), (int)E) * 4);
  L.tile_r0 = take((size_t)moe::mfma_max_tiles((int)(m * k), (int)E) * 4);
  L.tile_info = take((1 + 2 * E) * 4);
  L.h_q = take(m * k * I);
  L.h_s = take(m * k * I / 32);
  L.slot = take(m * k * H * 2);
  L.sh_q = take(m * I);
  L.sh_s = take(m * I / 32);
  L.sh_out = take(m * H * 2);
  // stage-major copies of the routed w1, w3 and w2 scales for the prefill-width GEMMs
  L.scales = take(m * k >= (size_t)kTiledRowsPerExpert * E ? 3 * E * I * H / 32 : 0);
  // the activation scales of the sorted pairs, stage-major (prefill width: x_s gathered for GEMM1, or a
  // caller's row-major h_s for GEMM2)
  L.xs_sm = take(m * k >= (size_t)kTiledRowsPerExpert * E ? m * k * std::max(H, I) / 32 : 0);
  L.total = off;
  return L;
}

template <typename T>
inline T* at(void* ws, size_t off) {
  return reinterpret_cast<T*>(static_cast<char*>(ws) + off);
}

inline bool al(const void* p, uintptr_t a) { return p != nullptr && (reinterpret_cast<uintptr_t>(p) % a) == 0; }

moe_status check_dims(const moe_dims* d, int32_t M) {
  if (d == nullptr || M < 0) return MOE_ERR_INVALID_ARG;
  const int E = d->num_experts, H = d->hidden, I = d->inter, k = d->top_k;
  if (E <= 0 || H <= 0 || I <= 0 || k <= 0 || !std::isfinite(d->route_scale)) return MOE_ERR_INVALID_ARG;
  if ((d->flags & ~MOE_FLAG_BATCH_INVARIANT) != 0u) return MOE_ERR_INVALID_ARG;
  if (E > 256 || k > 8 || k > E) return MOE_ERR_UNSUPPORTED;
  if (H % 128 != 0 || I % 128 != 0) return MOE_ERR_UNSUPPORTED;
  if (H > 8192 || I > 8192) return MOE_ERR_UNSUPPORTED;   // decode-width LDS staging stays within 64 KB
  if ((int64_t)H * I > (int64_t(1) << 31)) return MOE_ERR_UNSUPPORTED;
  if (M > (1 << 24) || (int64_t)M * k > (int64_t(1) << 26)) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

moe_status check_ws(const moe_dims* d, int32_t M, const void* ws, size_t ws_bytes) {
  if (!al(ws, 256)) return MOE_ERR_INVALID_ARG;
  if (ws_bytes < ws_layout(d, M).total) return MOE_ERR_WORKSPACE;
  return MOE_OK;
}

moe_status launched() { return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

#define MOE_TRY(expr)                   \
  do {                                  \
    const moe_status st_ = (expr);      \
    if (st_ != MOE_OK) return st_;      \
  } while (0)

// The weight codes come from w1, w3, w2 or, when given, from the fragment-order copy (then the three
// row-major pointers may be NULL); the scales always from s1, s3, s2.
moe_status check_packed(const moe_mxfp4_experts* w) {
  if (!w || !al(w->s1, 16) || !al(w->s3, 16) || !al(w->s2, 16)) return MOE_ERR_INVALID_ARG;
  if (w->tiled_weights != nullptr) {
    if (!al(w->tiled_weights, 16)) return MOE_ERR_INVALID_ARG;
  } else if (!al(w->w1, 16) || !al(w->w3, 16) || !al(w->w2, 16)) {
    return MOE_ERR_INVALID_ARG;
  }
  if (w->stage_scales != nullptr && !al(w->stage_scales, 16)) return MOE_ERR_INVALID_ARG;
  return MOE_OK;
}

// Offset of w1, w3, w2 inside moe_prepare_mxfp4_weights output (each matrix stack is E * I * H / 2 bytes).
inline size_t tiled_off(const moe_dims* d, int which) {
  return (size_t)which * d->num_experts * (size_t)d->inter * (d->hidden / 2);
}

// Offsets of the s1, s3, s2 stage-major copies inside moe_prepare_mxfp4_scales output (and the
// workspace copy).
inline size_t stage_scales_off(const moe_dims* d, int which) {
  return (size_t)which * d->num_experts * (size_t)d->inter * (d->hidden / 32);
}

moe_status check_decoded(const moe_bf16_experts* w) {
  if (!w || !al(w->w1, 16) || !al(w->w3, 16) || !al(w->w2, 16)) return MOE_ERR_INVALID_ARG;
  return MOE_OK;
}

moe_status check_shared(const moe_fp8_expert* w) {
  if (!w || !al(w->w1, 16) || !al(w->w3, 16) || !al(w->w2, 16) || !al(w->s1, 16) || !al(w->s3, 16) || !al(w->s2, 16))
    return MOE_ERR_INVALID_ARG;
  return MOE_OK;
}

// ---- launch sequences (arguments already validated) ------------------------------------------
// Kernel variant: a pure function of (dims, M) and the arm. Once the experts hold kTiledRowsPerExpert rows on average
// (prefill widths) the grouped GEMMs over the row-tile list: block-scaled MFMA for the packed experts,
// bf16 MFMA for the decoded-BF16 arm. Below, the weight-streaming kernels (packed) and the per-expert
// vector kernel (decoded).
inline bool routed_tiled(const moe_dims* d, int M) {
  return (int64_t)M * d->top_k >= kTiledRowsPerExpert * (int64_t)d->num_experts;
}
inline bool routed_mfma(const moe_dims* d, int M, const moe_mxfp4_experts* packed) {
  return packed != nullptr && routed_tiled(d, M);
}
inline bool shared_mfma(int M) { return M > 64; }
// The 512 x 128 tile kernels (expert_wide.hip) serve the fragment-order MXFP4 copy at prefill width while every
// operand they address stays below 2^31 bytes (32-bit buffer offsets); beyond that the register kernel of
// expert_mfma.hip takes over.
inline bool routed_wide(const moe_dims* d, int M, const moe_mxfp4_experts* packed) {
  if (!routed_mfma(d, M, packed) || packed->tiled_weights == nullptr) return false;
  const int64_t P = (int64_t)M * d->top_k, lim = int64_t(1) << 31;
  return (int64_t)M * d->hidden < lim && P * d->inter < lim && P * d->hidden / 32 < lim &&
         (int64_t)d->inter * d->hidden / 2 < lim;
}

struct TileMap {
  int max_tiles = 0;
  const int32_t* tile_e = nullptr;
  const int32_t* tile_r0 = nullptr;
  const int32_t* info = nullptr;
  uint8_t* scales = nullptr;   // workspace room for the stage-major w1, w3, w2 scales
  uint8_t* xs_sm = nullptr;    // workspace room for the stage-major activation scales of GEMM1
  bool act_sm = false;         // GEMM1 reads stage-major activation scales and writes h_s stage-major
};

TileMap make_tile_map(const moe_dims* d, int M, const int32_t* offsets, void* ws, hipStream_t s) {
  const WsLayout L = ws_layout(d, M);
  TileMap t;
  t.max_tiles = moe::mfma_max_tiles(M * d->top_k, d->num_experts);
  int32_t* te = at<int32_t>(ws, L.tile_e);
  int32_t* tr = at<int32_t>(ws, L.tile_r0);
  int32_t* ti = at<int32_t>(ws, L.tile_info);
  moe::launch_tile_map(d->num_experts, t.max_tiles, offsets, te, tr, ti, s);
  t.tile_e = te;
  t.tile_r0 = tr;
  t.info = ti;
  t.scales = at<uint8_t>(ws, L.scales);
  t.xs_sm = at<uint8_t>(ws, L.xs_sm);
  return t;
}
void do_route(const moe_dims* d, int M, const uint16_t* x, const float* gw, const float* gb, int32_t* ids,
              float* rw, uint8_t* xq, uint8_t* xs, void* ws, hipStream_t s) {
  const WsLayout L = ws_layout(d, M);
  float* logits = at<float>(ws, L.logits);
  moe::launch_router_logits(M, d->hidden, d->num_experts, x, gw, logits, xq, xs, batch_invariant(d), s);
  moe::launch_router_select_qdq(M, d->hidden, d->num_experts, d->top_k, d->route_scale, logits, gb, x, ids, rw, xq,
                                xs, batch_invariant(d), s);
}

// GEMM1: I rows of w1 and w3 over H inputs; activation row = token of the pair; output h rows at
// sorted positions.
void do_gemm1(const moe_dims* d, int M, const uint8_t* xq, const uint8_t* xs, const moe_mxfp4_experts* packed,
              const moe_bf16_experts* decoded, const float* rw, const int32_t* offsets, const int32_t* pairs,
              const int32_t* active, uint8_t* hq, uint8_t* hs, const TileMap& tm, hipStream_t s) {
  const int E = d->num_experts, H = d->hidden, I = d->inter, k = d->top_k;
  const int max_active = (int)std::min<int64_t>(E, (int64_t)M * k);
  GemmProblem p{};
  p.dense = 0; p.M = M; p.k = k; p.num_experts = E;
  p.offsets = offsets; p.pairs = pairs; p.active = active; p.rw = rw;
  moe::WeightFormat f;
  if (packed) {
    f = moe::W_MXFP4;
    p.wa = packed->w1; p.sa = packed->s1; p.wb = packed->w3; p.sb = packed->s3;
    p.w_expert_stride = (long long)I * H / 2; p.s_expert_stride = (long long)I * H / 32;
    if (packed->tiled_weights != nullptr) {
      p.wa = packed->tiled_weights + tiled_off(d, 0);
      p.wb = packed->tiled_weights + tiled_off(d, 1);
      p.w_tiled = 1;
    }
  } else {
    f = moe::W_BF16;
    p.wa = decoded->w1; p.sa = nullptr; p.wb = decoded->w3; p.sb = nullptr;
    p.w_expert_stride = (long long)I * H; p.s_expert_stride = 0;
  }
  p.N = I; p.K = H;
  p.act_q = xq; p.act_s = xs; p.act_by_token = 1;
  p.h_q = hq; p.h_s = hs;
  if (routed_mfma(d, M, packed)) {
    if (packed->stage_scales != nullptr) {
      p.sa = packed->stage_scales + stage_scales_off(d, 0);
      p.sb = packed->stage_scales + stage_scales_off(d, 1);
    } else {
      uint8_t* s1 = tm.scales + stage_scales_off(d, 0);
      uint8_t* s3 = tm.scales + stage_scales_off(d, 1);
      moe::launch_scales_stage_major(E, I, H, packed->s1, s1, s);
      moe::launch_scales_stage_major(E, I, H, packed->s3, s3, s);
      p.sa = s1; p.sb = s3;
    }
    p.s_stage_major = 1;
    const bool wide = routed_wide(d, M, packed);
    if (wide || tm.act_sm) {   // the activation scales of the sorted pairs, stage-major
      moe::launch_gather_act_scales(M * k, k, H, pairs, xs, tm.xs_sm, s);
      p.act_s = tm.xs_sm; p.a_stage_major = 1;
    }
    p.h_s_stage_major = tm.act_sm ? 1 : 0;   // h stays in the workspace: GEMM2 reads its scales stage-major
    if (wide) moe::launch_gemm1_wide(p, tm.max_tiles, tm.tile_e, tm.tile_r0, tm.info, s);
    else moe::launch_gemm1_mfma(f, p, tm.max_tiles, tm.tile_e, tm.tile_r0, tm.info, s);
  }
  else if (packed) moe::launch_gemm1_stream(f, p, max_active, s);
  else if (routed_tiled(d, M)) moe::launch_gemm1_bf16(p, tm.max_tiles, tm.tile_e, tm.tile_r0, tm.info, s);
  else moe::launch_gemm1_small(f, p, max_active, s);
}

// GEMM2: H rows of w2 over I inputs; activation row = sorted position; output row = pair id.
void do_gemm2(const moe_dims* d, int M, const uint8_t* hq, const uint8_t* hs, const moe_mxfp4_experts* packed,
              const moe_bf16_experts* decoded, const int32_t* offsets, const int32_t* pairs, const int32_t* active,
              uint16_t* slot, float* slot_f32, const TileMap& tm, hipStream_t s, const int32_t* out_rows = nullptr) {
  const int E = d->num_experts, H = d->hidden, I = d->inter, k = d->top_k;
  const int max_active = (int)std::min<int64_t>(E, (int64_t)M * k);
  GemmProblem q{};
  q.dense = 0; q.M = M; q.k = k; q.num_experts = E;
  q.offsets = offsets; q.pairs = pairs; q.active = active; q.rw = nullptr;
  moe::WeightFormat f;
  if (packed) {
    f = moe::W_MXFP4;
    q.wa = packed->w2; q.sa = packed->s2;
    q.w_expert_stride = (long long)H * I / 2; q.s_expert_stride = (long long)H * I / 32;
    if (packed->tiled_weights != nullptr) {
      q.wa = packed->tiled_weights + tiled_off(d, 2);
      q.w_tiled = 1;
    }
  } else {
    f = moe::W_BF16;
    q.wa = decoded->w2; q.sa = nullptr;
    q.w_expert_stride = (long long)H * I; q.s_expert_stride = 0;
  }
  q.N = H; q.K = I;
  q.act_q = hq; q.act_s = hs; q.act_by_token = 0;
  q.out = slot; q.out_f32 = slot_f32;
  // (out_rows: the decode-width kernels only; the caller passes it only when no prefill-width kernel runs)
  q.out_rows = routed_tiled(d, M) ? nullptr : out_rows;
  if (routed_mfma(d, M, packed)) {
    if (packed->stage_scales != nullptr) {
      q.sa = packed->stage_scales + stage_scales_off(d, 2);
    } else {
      uint8_t* s2 = tm.scales + stage_scales_off(d, 2);
      moe::launch_scales_stage_major(E, H, I, packed->s2, s2, s);
      q.sa = s2;
    }
    q.s_stage_major = 1;
    q.a_stage_major = tm.act_sm ? 1 : 0;
    if (routed_wide(d, M, packed)) {
      if (!tm.act_sm) {   // a caller's h_s [P, I/32] by sorted position: re-laid out stage-major first
        moe::launch_gather_act_scales(M * k, 1, I, nullptr, hs, tm.xs_sm, s);
        q.act_s = tm.xs_sm; q.a_stage_major = 1;
      }
      moe::launch_gemm2_wide(q, tm.max_tiles, tm.tile_e, tm.tile_r0, tm.info, s);
    } else {
      moe::launch_gemm2_mfma(f, q, tm.max_tiles, tm.tile_e, tm.tile_r0, tm.info, s);
    }
  }
  else if (packed) moe::launch_gemm2_stream(f, q, max_active, s);
  else if (routed_tiled(d, M)) moe::launch_gemm2_bf16(q, tm.max_tiles, tm.tile_e, tm.tile_r0, tm.info, s);
  else moe::launch_gemm2_small(f, q, max_active, s);
}

// h_internal: h_q / h_s are workspace buffers no caller reads, so the prefill GEMMs may keep h_s in
// their own stage-major layout.
void do_expert_ffn(const moe_dims* d, int M, const uint8_t* xq, const uint8_t* xs, const moe_mxfp4_experts* packed,
                   const moe_bf16_experts* decoded, const float* rw, const int32_t* offsets, const int32_t* pairs,
                   const int32_t* active, uint16_t* slot, float* slot_f32, uint8_t* hq, uint8_t* hs, bool h_internal,
                   void* ws, hipStream_t s,
                   const int32_t* out_rows = nullptr) {
  TileMap tm;
  if (routed_tiled(d, M)) {
    tm = make_tile_map(d, M, offsets, ws, s);
    tm.act_sm = h_internal && packed != nullptr;   // the bf16 kernels keep h_s row-major
  }
  do_gemm1(d, M, xq, xs, packed, decoded, rw, offsets, pairs, active, hq, hs, tm, s);
  do_gemm2(d, M, hq, hs, packed, decoded, offsets, pairs, active, slot, slot_f32, tm, s, out_rows);
}

void do_shared(const moe_dims* d, int M, const uint8_t* xq, const uint8_t* xs, const moe_fp8_expert* sh,
               uint8_t* shq, uint8_t* shs, uint16_t* out, float* out_f32, hipStream_t s) {
  const int H = d->hidden, I = d->inter;
  GemmProblem p{};
  p.dense = 1; p.M = M; p.k = 1; p.num_experts = 1;
  p.wa = sh->w1; p.sa = sh->s1; p.wb = sh->w3; p.sb = sh->s3;
  p.w_expert_stride = 0; p.s_expert_stride = 0;
  p.N = I; p.K = H;
  p.act_q = xq; p.act_s = xs; p.act_by_token = 1;
  p.h_q = shq; p.h_s = shs;
  const TileMap none;
  if (shared_mfma(M)) moe::launch_gemm1_mfma(moe::W_FP8_BLOCK32, p, 0, none.tile_e, none.tile_r0, none.info, s);
  else moe::launch_gemm1_stream(moe::W_FP8_BLOCK32, p, 1, s);
  GemmProblem q = p;
  q.wa = sh->w2; q.sa = sh->s2; q.wb = nullptr; q.sb = nullptr;
  q.N = H; q.K = I;
  q.act_q = shq; q.act_s = shs; q.act_by_token = 0;
  q.out = out; q.out_f32 = out_f32;
  if (shared_mfma(M)) moe::launch_gemm2_mfma(moe::W_FP8_BLOCK32, q, 0, none.tile_e, none.tile_r0, none.info, s);
  else moe::launch_gemm2_stream(moe::W_FP8_BLOCK32, q, 1, s);
}

// Argument checks of moe_forward and moe_forward_noalloc (everything except the workspace).
moe_status check_forward(const moe_dims* dims, int32_t M, const uint16_t* x, const float* gate_w, const float* gate_b,
                         const moe_mxfp4_experts* packed, const moe_bf16_experts* decoded,
                         const moe_fp8_expert* shared, const uint16_t* out, const int32_t* ids_out,
                         const float* rw_out, const uint16_t* shared_out) {
  MOE_TRY(check_dims(dims, M));
  if ((packed == nullptr) == (decoded == nullptr)) return MOE_ERR_INVALID_ARG;
  if (M == 0) return MOE_OK;
  MOE_TRY(packed ? check_packed(packed) : check_decoded(decoded));
  if (shared != nullptr) MOE_TRY(check_shared(shared));
  if (!al(x, 16) || !al(gate_w, 16) || !al(gate_b, 4) || !al(out, 16)) return MOE_ERR_INVALID_ARG;
  if ((ids_out && !al(ids_out, 4)) || (rw_out && !al(rw_out, 4)) || (shared_out && !al(shared_out, 16)))
    return MOE_ERR_INVALID_ARG;
  if (shared_out != nullptr && shared == nullptr) return MOE_ERR_INVALID_ARG;
  return MOE_OK;
}

// The whole layer on a validated workspace of ws_layout(dims, M).total bytes. No kernel relies on the
// workspace's previous contents: every buffer is written before it is read within the call.
// ---- the shared expert beside the routed experts ---------------------------------------------------
// At prefill widths the FP8 shared expert (288 / 320 blocks of its two GEMMs at M = 2048, a second wave of blocks
// that fills a ninth of the chip) runs on a second stream of the same device, forked from the caller's stream
// after the router and joined before the combine, so its blocks fill the CUs the routed GEMMs leave idle. One
// such stream and two events per device, created on first use and kept; the fork / join sequence of a call is
// enqueued under a lock, so calls from several host threads pair their own records and waits. (Graph capture:
// the fork event brings the second stream into the caller's capture and the join returns it.)
struct SideStream {
  hipStream_t stream = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
  bool failed = false;
};
constexpr int kMaxSideDevices = 64;
std::mutex g_side_mu;
SideStream g_side[kMaxSideDevices];

// The device's side stream (nullptr if it cannot be made: the shared expert then runs on the caller's stream).
// Called with g_side_mu held.
SideStream* side_stream_locked() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxSideDevices) return nullptr;
  SideStream& ss = g_side[dev];
  if (ss.stream == nullptr && !ss.failed) {
    if (hipStreamCreateWithFlags(&ss.stream, hipStreamNonBlocking) != hipSuccess ||
        hipEventCreateWithFlags(&ss.fork, hipEventDisableTiming) != hipSuccess ||
        hipEventCreateWithFlags(&ss.join, hipEventDisableTiming) != hipSuccess) {
      ss.failed = true;
      (void)hipGetLastError();
      return nullptr;
    }
  }
  return ss.failed ? nullptr : &ss;
}

void forward_impl(const moe_dims* dims, int32_t M, const uint16_t* x, const float* gate_w, const float* gate_b,
                  const moe_mxfp4_experts* packed, const moe_bf16_experts* decoded, const moe_fp8_expert* shared,
                  uint16_t* out, int32_t* ids_out, float* rw_out, uint16_t* shared_out, void* ws, hipStream_t s,
                  bool side_ok = true) {
  const WsLayout L = ws_layout(dims, M);
  int32_t* ids = ids_out ? ids_out : at<int32_t>(ws, L.ids);
  float* rw = rw_out ? rw_out : at<float>(ws, L.rw);
  uint8_t* xq = at<uint8_t>(ws, L.x_q);
  uint8_t* xs = at<uint8_t>(ws, L.x_s);
  int32_t* offsets = at<int32_t>(ws, L.offsets);
  int32_t* pairs = at<int32_t>(ws, L.pairs);
  int32_t* active = at<int32_t>(ws, L.active);
  const bool fused = M <= moe::kRouterSmallM && !batch_invariant(dims);
  if (fused) {   // decode widths: logits + QDQ, then selection and permutation in one block
    float* logits = at<float>(ws, L.logits);
    moe::launch_router_logits(M, dims->hidden, dims->num_experts, x, gate_w, logits, xq, xs, false, s);
    moe::launch_select_permute_small(M, dims->hidden, dims->num_experts, dims->top_k, dims->route_scale, logits,
                                     gate_b, ids, rw, at<int32_t>(ws, L.counts), offsets, pairs,
                                     at<int32_t>(ws, L.inv), active, at<int32_t>(ws, L.out_rows), s);
  } else {
    do_route(dims, M, x, gate_w, gate_b, ids, rw, xq, xs, ws, s);
    // at the row-tiled widths the expert GEMMs read the row-tile map, so the active list is not built
    moe::launch_permute(M * dims->top_k, dims->num_experts, ids, at<int32_t>(ws, L.counts), offsets, pairs,
                        at<int32_t>(ws, L.inv), routed_tiled(dims, M) ? nullptr : active, s);
  }
  uint16_t* slot = at<uint16_t>(ws, L.slot);
  uint16_t* sh_out = shared != nullptr ? (shared_out ? shared_out : at<uint16_t>(ws, L.sh_out)) : nullptr;
  // the shared expert on the device's second stream (prefill widths), else after the routed experts
  std::unique_lock<std::mutex> side_lock;
  SideStream* side = nullptr;
  if (shared != nullptr && side_ok && shared_mfma(M)) {
    side_lock = std::unique_lock<std::mutex>(g_side_mu);
    side = side_stream_locked();
    if (side != nullptr && (hipEventRecord(side->fork, s) != hipSuccess ||
                            hipStreamWaitEvent(side->stream, side->fork, 0) != hipSuccess)) {
      (void)hipGetLastError();
      side = nullptr;
    }
    if (side != nullptr) {
      do_shared(dims, M, xq, xs, shared, at<uint8_t>(ws, L.sh_q), at<uint8_t>(ws, L.sh_s), sh_out, nullptr,
                side->stream);
      (void)hipEventRecord(side->join, side->stream);
    }
  }
  // decode widths on the decode-width kernels: each token's slot rows are written in ascending expert-id order
  // (rows from the selection kernel), so the combine reads no ids
  const bool ranked = fused && !routed_tiled(dims, M);
  do_expert_ffn(dims, M, xq, xs, packed, decoded, rw, offsets, pairs, active, slot, nullptr, at<uint8_t>(ws, L.h_q),
                at<uint8_t>(ws, L.h_s), true, ws, s, ranked ? at<int32_t>(ws, L.out_rows) : nullptr);
  if (side != nullptr) {
    (void)hipStreamWaitEvent(s, side->join, 0);
    side_lock.unlock();
  } else if (shared != nullptr) {
    do_shared(dims, M, xq, xs, shared, at<uint8_t>(ws, L.sh_q), at<uint8_t>(ws, L.sh_s), sh_out, nullptr, s);
  }
  moe::launch_combine(M, dims->hidden, dims->top_k, ranked ? nullptr : ids, slot, sh_out, out, s);
}

}  // namespace

// ---- the library-owned workspace of moe_forward_noalloc ---------------------------------------------
// One array per GPU the library runs on, held until the process ends. In host code the name `scratch`
// only stands in for the symbol: its device address comes from hipGetSymbolAddress, once per device with
// that device current, and only that address is ever passed to kernels.
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of this device's scratch array for work on stream s (NULL = the current device's
// default stream). The stream must belong to the current device.
moe_status scratch_for_stream(hipStream_t s, void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return MOE_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return MOE_ERR_UNSUPPORTED;
  if (s != nullptr) {
    hipDevice_t sdev = -1;
    if (hipStreamGetDevice(s, &sdev) != hipSuccess) return MOE_ERR_INVALID_ARG;
    if (sdev != dev) return MOE_ERR_INVALID_ARG;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return MOE_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MOE_OK;
}

}  // namespace

extern "C" {

size_t moe_workspace_bytes(const moe_dims* dims, int32_t max_tokens) {
  if (check_dims(dims, max_tokens) != MOE_OK) return 0;
  return ws_layout(dims, max_tokens).total;
}

const char* moe_status_str(moe_status status) {
  switch (status) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_INVALID_ARG: return "MOE_ERR_INVALID_ARG";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED";
    case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE";
    case MOE_ERR_HIP: return "MOE_ERR_HIP";
    default: return "MOE_ERR_UNKNOWN";
  }
}

moe_status moe_route(const moe_dims* dims, int32_t M, const uint16_t* x, const float* gate_w, const float* gate_b,
                     int32_t* ids, float* rw, uint8_t* x_q, uint8_t* x_s, void* ws, size_t ws_bytes, void* stream) {
  MOE_TRY(check_dims(dims, M));
  if (M == 0) return MOE_OK;
  if (!al(x, 16) || !al(gate_w, 16) || !al(gate_b, 4) || !al(ids, 4) || !al(rw, 4) || !al(x_q, 16) || !al(x_s, 16))
    return MOE_ERR_INVALID_ARG;
  MOE_TRY(check_ws(dims, M, ws, ws_bytes));
  do_route(dims, M, x, gate_w, gate_b, ids, rw, x_q, x_s, ws, static_cast<hipStream_t>(stream));
  return launched();
}

moe_status moe_permute(const moe_dims* dims, int32_t M, const int32_t* ids, int32_t* counts, int32_t* offsets,
                       int32_t* pairs, int32_t* inv, int32_t* active, void* stream) {
  MOE_TRY(check_dims(dims, M));
  if (M == 0) return MOE_OK;
  if (!al(ids, 4) || !al(counts, 4) || !al(offsets, 4) || !al(pairs, 4) || !al(active, 4)) return MOE_ERR_INVALID_ARG;
  if (inv != nullptr && !al(inv, 4)) return MOE_ERR_INVALID_ARG;
  moe::launch_permute(M * dims->top_k, dims->num_experts, ids, counts, offsets, pairs, inv, active,
                      static_cast<hipStream_t>(stream));
  return launched();
}

moe_status moe_expert_ffn(const moe_dims* dims, int32_t M, const uint8_t* x_q, const uint8_t* x_s,
                          const moe_mxfp4_experts* packed, const moe_bf16_experts* decoded, const float* rw,
                          const int32_t* offsets, const int32_t* pairs, const int32_t* active, uint16_t* slot_out,
                          uint8_t* h_q, uint8_t* h_s, void* ws, size_t ws_bytes, void* stream) {
  MOE_TRY(check_dims(dims, M));
  if ((packed == nullptr) == (decoded == nullptr)) return MOE_ERR_INVALID_ARG;
  if (M == 0) return MOE_OK;
  MOE_TRY(packed ? check_packed(packed) : check_decoded(decoded));
  if (!al(x_q, 16) || !al(x_s, 16) || !al(rw, 4) || !al(offsets, 4) || !al(pairs, 4) || !al(active, 4) || !al(slot_out, 16))
    return MOE_ERR_INVALID_ARG;
  if ((h_q == nullptr) != (h_s == nullptr)) return MOE_ERR_INVALID_ARG;
  if (h_q != nullptr && !al(h_q, 16)) return MOE_ERR_INVALID_ARG;
  MOE_TRY(check_ws(dims, M, ws, ws_bytes));
  const WsLayout L = ws_layout(dims, M);
  const bool h_internal = h_q == nullptr;
  if (h_internal) {
    h_q = at<uint8_t>(ws, L.h_q);
    h_s = at<uint8_t>(ws, L.h_s);
  }
  do_expert_ffn(dims, M, x_q, x_s, packed, decoded, rw, offsets, pairs, active, slot_out, nullptr, h_q, h_s,
                h_internal, ws, static_cast<hipStream_t>(stream));
  return launched();
}

moe_status moe_expert_gemm1(const moe_dims* dims, int32_t M, const uint8_t* x_q, const uint8_t* x_s,
                            const moe_mxfp4_experts* packed, const moe_bf16_experts* decoded, const float* rw,
                            const int32_t* offsets, const int32_t* pairs, const int32_t* active, uint8_t* h_q,
                            uint8_t* h_s, void* ws, size_t ws_bytes, void* stream) {
  MOE_TRY(check_dims(dims, M));
  if ((packed == nullptr) == (decoded == nullptr)) return MOE_ERR_INVALID_ARG;
  if (M == 0) return MOE_OK;
  MOE_TRY(packed ? check_packed(packed) : check_decoded(decoded));
  if (!al(x_q, 16) || !al(x_s, 16) || !al(rw, 4) || !al(offsets, 4) || !al(pairs, 4) || !al(active, 4) || !al(h_q, 16) ||
      !al(h_s, 16))
    return MOE_ERR_INVALID_ARG;
  MOE_TRY(check_ws(dims, M, ws, ws_bytes));
  hipStream_t s = static_cast<hipStream_t>(stream);
  TileMap tm;
  if (routed_tiled(dims, M)) tm = make_tile_map(dims, M, offsets, ws, s);
  do_gemm1(dims, M, x_q, x_s, packed, decoded, rw, offsets, pairs, active, h_q, h_s, tm, s);
  return launched();
}

moe_status moe_expert_gemm2(const moe_dims* dims, int32_t M, const uint8_t* h_q, const uint8_t* h_s,
                            const moe_mxfp4_experts* packed, const moe_bf16_experts* decoded,
                            const int32_t* offsets, const int32_t* pairs, const int32_t* active,
                            uint16_t* slot_out, void* ws, size_t ws_bytes, void* stream) {
  MOE_TRY(check_dims(dims, M));
  if ((packed == nullptr) == (decoded == nullptr)) return MOE_ERR_INVALID_ARG;
  if (M == 0) return MOE_OK;
  MOE_TRY(packed ? check_packed(packed) : check_decoded(decoded));
  if (!al(h_q, 16) || !al(h_s, 16) || !al(offsets, 4) || !al(pairs, 4) || !al(active, 4) || !al(slot_out, 16))
    return MOE_ERR_INVALID_ARG;
  MOE_TRY(check_ws(dims, M, ws, ws_bytes));
  hipStream_t s = static_cast<hipStream_t>(stream);
  TileMap tm;
  if (routed_tiled(dims, M)) tm = make_tile_map(dims, M, offsets, ws, s);
  do_gemm2(dims, M, h_q, h_s, packed, decoded, offsets, pairs, active, slot_out, nullptr, tm, s);
  return launched();
}

moe_status moe_shared_expert(const moe_dims* dims, int32_t M, const uint8_t* x_q, const uint8_t* x_s,
                             const moe_fp8_expert* shared, uint16_t* shared_out, void* ws, size_t ws_bytes,
                             void* stream) {
  MOE_TRY(check_dims(dims, M));
  if (M == 0) return MOE_OK;
  MOE_TRY(check_shared(shared));
  if (!al(x_q, 16) || !al(x_s, 16) || !al(shared_out, 16)) return MOE_ERR_INVALID_ARG;
  MOE_TRY(check_ws(dims, M, ws, ws_bytes));
  const WsLayout L = ws_layout(dims, M);
  do_shared(dims, M, x_q, x_s, shared, at<uint8_t>(ws, L.sh_q), at<uint8_t>(ws, L.sh_s), shared_out, nullptr,
            static_cast<hipStream_t>(stream));
  return launched();
}

moe_status moe_combine(const moe_dims* dims, int32_t M, const int32_t* ids, const uint16_t* slot_out,
                       const uint16_t* shared_out, uint16_t* out, void* stream) {
  MOE_TRY(check_dims(dims, M));
  if (M == 0) return MOE_OK;
  if (!al(ids, 4) || !al(slot_out, 16) || !al(out, 16)) return MOE_ERR_INVALID_ARG;
  if (shared_out != nullptr && !al(shared_out, 16)) return MOE_ERR_INVALID_ARG;
  moe::launch_combine(M, dims->hidden, dims->top_k, ids, slot_out, shared_out, out, static_cast<hipStream_t>(stream));
  return launched();
}

moe_status moe_forward(const moe_dims* dims, int32_t M, const uint16_t* x, const float* gate_w, const float* gate_b,
                       const moe_mxfp4_experts* packed, const moe_bf16_experts* decoded, const moe_fp8_expert* shared,
                       uint16_t* out, int32_t* ids_out, float* rw_out, uint16_t* shared_out, void* ws,
                       size_t ws_bytes, void* stream) {
  MOE_TRY(check_forward(dims, M, x, gate_w, gate_b, packed, decoded, shared, out, ids_out, rw_out, shared_out));
  if (M == 0) return MOE_OK;
  MOE_TRY(check_ws(dims, M, ws, ws_bytes));
  forward_impl(dims, M, x, gate_w, gate_b, packed, decoded, shared, out, ids_out, rw_out, shared_out, ws,
               static_cast<hipStream_t>(stream));
  return launched();
}

moe_status moe_forward_noalloc(const moe_dims* dims, int32_t M, const uint16_t* x, const float* gate_w,
                               const float* gate_b, const moe_mxfp4_experts* packed, const moe_bf16_experts* decoded,
                               const moe_fp8_expert* shared, uint16_t* out, int32_t* ids_out, float* rw_out,
                               uint16_t* shared_out, void* stream) {
  MOE_TRY(check_forward(dims, M, x, gate_w, gate_b, packed, decoded, shared, out, ids_out, rw_out, shared_out));
  if (M == 0) return MOE_OK;
  if (ws_layout(dims, M).total > kScratchBytes) return MOE_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  void* ws = nullptr;
  MOE_TRY(scratch_for_stream(s, &ws));
  // (no second stream here: creating it would allocate)
  forward_impl(dims, M, x, gate_w, gate_b, packed, decoded, shared, out, ids_out, rw_out, shared_out, ws, s, false);
  return launched();
}

moe_status moe_expert_ffn_f32(const moe_dims* dims, int32_t M, const uint8_t* x_q, const uint8_t* x_s,
                              const moe_mxfp4_experts* packed, const moe_bf16_experts* decoded, const float* rw,
                              const int32_t* offsets, const int32_t* pairs, const int32_t* active, float* slot_f32,
                              void* ws, size_t ws_bytes, void* stream) {
  MOE_TRY(check_dims(dims, M));
  if ((packed == nullptr) == (decoded == nullptr)) return MOE_ERR_INVALID_ARG;
  if (M == 0) return MOE_OK;
  MOE_TRY(packed ? check_packed(packed) : check_decoded(decoded));
  if (!al(x_q, 16) || !al(x_s, 16) || !al(rw, 4) || !al(offsets, 4) || !al(pairs, 4) || !al(active, 4) ||
      !al(slot_f32, 16))
    return MOE_ERR_INVALID_ARG;
  MOE_TRY(check_ws(dims, M, ws, ws_bytes));
  const WsLayout L = ws_layout(dims, M);
  do_expert_ffn(dims, M, x_q, x_s, packed, decoded, rw, offsets, pairs, active, nullptr, slot_f32,
                at<uint8_t>(ws, L.h_q), at<uint8_t>(ws, L.h_s), true, ws, static_cast<hipStream_t>(stream));
  return launched();
}

moe_status moe_shared_expert_f32(const moe_dims* dims, int32_t M, const uint8_t* x_q, const uint8_t* x_s,
                                 const moe_fp8_expert* shared, float* shared_f32, void* ws, size_t ws_bytes,
                                 void* stream) {
  MOE_TRY(check_dims(dims, M));
  if (M == 0) return MOE_OK;
  MOE_TRY(check_shared(shared));
  if (!al(x_q, 16) || !al(x_s, 16) || !al(shared_f32, 16)) return MOE_ERR_INVALID_ARG;
  MOE_TRY(check_ws(dims, M, ws, ws_bytes));
  const WsLayout L = ws_layout(dims, M);
  do_shared(dims, M, x_q, x_s, shared, at<uint8_t>(ws, L.sh_q), at<uint8_t>(ws, L.sh_s), nullptr, shared_f32,
            static_cast<hipStream_t>(stream));
  return launched();
}

moe_status moe_combine_sum_f32(const moe_dims* dims, int32_t M, const int32_t* ids, const float* slot_f32,
                               const float* add, float* out_f32, void* stream) {
  MOE_TRY(check_dims(dims, M));
  if (M == 0) return MOE_OK;
  if (!al(ids, 4) || !al(slot_f32, 16) || !al(out_f32, 16)) return MOE_ERR_INVALID_ARG;
  if (add != nullptr && !al(add, 16)) return MOE_ERR_INVALID_ARG;
  moe::launch_combine_sum_f32(M, dims->hidden, dims->top_k, ids, slot_f32, add, out_f32,
                              static_cast<hipStream_t>(stream));
  return launched();
}

moe_status moe_combine_official_f32(const moe_dims* dims, int32_t M, const int32_t* ids, const float* slot_f32,
                                    const float* shared_f32, const uint16_t* shared_bf16, uint16_t* out,
                                    void* stream) {
  MOE_TRY(check_dims(dims, M));
  if (M == 0) return MOE_OK;
  if (!al(ids, 4) || !al(slot_f32, 16) || !al(out, 16)) return MOE_ERR_INVALID_ARG;
  if (shared_f32 != nullptr && shared_bf16 != nullptr) return MOE_ERR_INVALID_ARG;
  if ((shared_f32 != nullptr && !al(shared_f32, 16)) || (shared_bf16 != nullptr && !al(shared_bf16, 16)))
    return MOE_ERR_INVALID_ARG;
  moe::launch_combine_official_f32(M, dims->hidden, dims->top_k, ids, slot_f32, shared_f32, shared_bf16, out,
                                   static_cast<hipStream_t>(stream));
  return launched();
}

// ---- dense FP8 linear -------------------------------------------------------------------------
namespace {

moe_status check_linear(int32_t M, int32_t N, int32_t K) {
  if (M < 0 || N <= 0 || K <= 0) return MOE_ERR_INVALID_ARG;
  if (N % 128 != 0 || K % 128 != 0 || N > 65536 || K > 65536) return MOE_ERR_UNSUPPORTED;
  if (M > (1 << 24) || (int64_t)M * K > (int64_t(1) << 31) || (int64_t)M * N > (int64_t(1) << 31))
    return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

struct LinearLayout {
  size_t xq, xs, part, total;
};

LinearLayout linear_layout(int32_t M, int32_t N, int32_t K) {
  LinearLayout L{};
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += round_up(bytes, 256);
    return o;
  };
  const size_t m = (size_t)M;
  L.xq = take(m * K);
  L.xs = take(m * K / 32);
  size_t part = 0;
  if (M > 0 && M <= 64) {
    const moe::DensePlan pl = moe::dense_plan(M, N, K);
    if (pl.runs > 1) part = (size_t)pl.runs * m * N * 4;
  }
  L.part = take(part);
  L.total = off;
  return L;
}

}  // namespace

size_t moe_fp8_linear_workspace_bytes(int32_t M, int32_t N, int32_t K) {
  if (check_linear(M, N, K) != MOE_OK) return 0;
  return std::max<size_t>(linear_layout(M, N, K).total, 256);
}

namespace {

moe_status fp8_linear_impl(int32_t M, int32_t N, int32_t K, const uint16_t* x, const uint8_t* w, bool w_tiled,
                           const uint8_t* s, uint16_t* y, float* y_f32, void* ws, size_t ws_bytes, void* stream) {
  MOE_TRY(check_linear(M, N, K));
  if ((y == nullptr) == (y_f32 == nullptr)) return MOE_ERR_INVALID_ARG;
  if (w_tiled && M > 64) return MOE_ERR_UNSUPPORTED;   // the fragment-order copy feeds the decode-width kernel
  if (M == 0) return MOE_OK;
  if (!al(x, 16) || !al(w, 16) || !al(s, 16) || !al(ws, 256)) return MOE_ERR_INVALID_ARG;
  if ((y != nullptr && !al(y, 16)) || (y_f32 != nullptr && !al(y_f32, 16))) return MOE_ERR_INVALID_ARG;
  const LinearLayout L = linear_layout(M, N, K);
  if (ws_bytes < L.total) return MOE_ERR_WORKSPACE;
  hipStream_t st = static_cast<hipStream_t>(stream);
  uint8_t* xq = at<uint8_t>(ws, L.xq);
  uint8_t* xs = at<uint8_t>(ws, L.xs);
  if (M <= 64) {   // the blocks QDQ their own runs of x
    moe::launch_fp8_linear_stream(M, N, K, x, nullptr, nullptr, w, w_tiled, s, at<float>(ws, L.part), y, y_f32, st);
  } else {
    moe::launch_qdq_rows(M, K, x, xq, xs, st);
    GemmProblem q{};
    q.dense = 1; q.M = M; q.k = 1; q.num_experts = 1;
    q.wa = w; q.sa = s; q.w_expert_stride = 0; q.s_expert_stride = 0;
    q.N = N; q.K = K;
    q.act_q = xq; q.act_s = xs; q.act_by_token = 0;
    q.out = y; q.out_f32 = y_f32;
    moe::launch_gemm2_mfma(moe::W_FP8_BLOCK32, q, 0, nullptr, nullptr, nullptr, st);
  }
  return launched();
}

}  // namespace

moe_status moe_fp8_linear(int32_t M, int32_t N, int32_t K, const uint16_t* x, const uint8_t* w, const uint8_t* s,
                          uint16_t* y, float* y_f32, void* ws, size_t ws_bytes, void* stream) {
  return fp8_linear_impl(M, N, K, x, w, false, s, y, y_f32, ws, ws_bytes, stream);
}

moe_status moe_fp8_linear_tiled(int32_t M, int32_t N, int32_t K, const uint16_t* x, const uint8_t* w_tiled,
                                const uint8_t* s, uint16_t* y, float* y_f32, void* ws, size_t ws_bytes,
                                void* stream) {
  return fp8_linear_impl(M, N, K, x, w_tiled, true, s, y, y_f32, ws, ws_bytes, stream);
}

size_t moe_fp8_tiled_weights_bytes(int32_t N, int32_t K) {
  if (check_linear(0, N, K) != MOE_OK) return 0;
  return (size_t)N * (size_t)K;
}

moe_status moe_prepare_fp8_weights(int32_t N, int32_t K, const uint8_t* w, uint8_t* out, void* stream) {
  MOE_TRY(check_linear(0, N, K));
  if (!al(w, 16) || !al(out, 16)) return MOE_ERR_INVALID_ARG;
  const size_t n = (size_t)N * (size_t)K;
  const uintptr_t o = reinterpret_cast<uintptr_t>(out), p = reinterpret_cast<uintptr_t>(w);
  if (p < o + n && o < p + n) return MOE_ERR_INVALID_ARG;
  // an E4M3 row of K bytes has the byte layout of an E2M1 row of 2 K values
  moe::launch_tile_mxfp4(1, N, 2 * K, w, out, static_cast<hipStream_t>(stream));
  return launched();
}

size_t moe_mxfp4_stage_scales_bytes(const moe_dims* dims) {
  if (check_dims(dims, 0) != MOE_OK) return 0;
  return stage_scales_off(dims, 3);
}

moe_status moe_prepare_mxfp4_scales(const moe_dims* dims, const moe_mxfp4_experts* w, uint8_t* out, void* stream) {
  MOE_TRY(check_dims(dims, 0));
  if (!w || !al(w->s1, 16) || !al(w->s3, 16) || !al(w->s2, 16) || !al(out, 16)) return MOE_ERR_INVALID_ARG;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int E = dims->num_experts, H = dims->hidden, I = dims->inter;
  moe::launch_scales_stage_major(E, I, H, w->s1, out + stage_scales_off(dims, 0), s);
  moe::launch_scales_stage_major(E, I, H, w->s3, out + stage_scales_off(dims, 1), s);
  moe::launch_scales_stage_major(E, H, I, w->s2, out + stage_scales_off(dims, 2), s);
  return launched();
}

size_t moe_mxfp4_tiled_weights_bytes(const moe_dims* dims) {
  if (check_dims(dims, 0) != MOE_OK) return 0;
  return tiled_off(dims, 3);
}

moe_status moe_prepare_mxfp4_weights(const moe_dims* dims, const moe_mxfp4_experts* w, uint8_t* out, void* stream) {
  MOE_TRY(check_dims(dims, 0));
  if (!w || !al(w->w1, 16) || !al(w->w3, 16) || !al(w->w2, 16) || !al(out, 16)) return MOE_ERR_INVALID_ARG;
  const size_t n = tiled_off(dims, 3), per = tiled_off(dims, 1);
  auto overlaps = [&](const uint8_t* a) {
    const uintptr_t o = reinterpret_cast<uintptr_t>(out), p = reinterpret_cast<uintptr_t>(a);
    return p < o + n && o < p + per;
  };
  if (overlaps(w->w1) || overlaps(w->w3) || overlaps(w->w2)) return MOE_ERR_INVALID_ARG;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int E = dims->num_experts, H = dims->hidden, I = dims->inter;
  moe::launch_tile_mxfp4(E, I, H, w->w1, out + tiled_off(dims, 0), s);
  moe::launch_tile_mxfp4(E, I, H, w->w3, out + tiled_off(dims, 1), s);
  moe::launch_tile_mxfp4(E, H, I, w->w2, out + tiled_off(dims, 2), s);
  return launched();
}

moe_status moe_expand_mxfp4(int64_t rows, int32_t cols, const uint8_t* w, const uint8_t* s, uint16_t* out,
                            void* stream) {
  if (rows < 0 || cols <= 0) return MOE_ERR_INVALID_ARG;
  if (cols % 32 != 0) return MOE_ERR_UNSUPPORTED;
  if (rows == 0) return MOE_OK;
  if (!al(w, 16) || !al(s, 16) || !al(out, 16)) return MOE_ERR_INVALID_ARG;
  moe::launch_expand_mxfp4(rows, cols, w, s, out, static_cast<hipStream_t>(stream));
  return launched();
}

}  // extern "C"
