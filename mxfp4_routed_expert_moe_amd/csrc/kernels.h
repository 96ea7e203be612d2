// Host-side launchers of the gfx950 kernels (internal to libmoe; the public C ABI is include/moe.h).
// Every launcher enqueues on the given stream, never synchronizes and never allocates; the caller
// (moe_abi.cpp) has validated shapes, pointers and workspace sizes before any launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "dense_plan.h"

namespace moe {

// ---- router (route.hip) --------------------------------------------------------------------
// Batches of at most kRouterSmallM tokens take the decode-width router: the logits kernel also does
// the per-32 E4M3 QDQ of x, and the selection may run fused with the permutation.
constexpr int kRouterSmallM = 64;
// fp32 logits of the raw bf16 activations against the fp32 gate weight [E, H], as
// router_logit_parts(M, H, mfma_order) partial planes [parts, M, E] (summed in order by the select kernel).
// At M <= kRouterSmallM it also writes x_q / x_s (ignored otherwise). mfma_order: the matrix-core kernel (and its
// summation order) at every M, the decode widths included; then the selection QDQs x.
int router_logit_parts(int M, int H, bool mfma_order = false);
void launch_router_logits(int M, int H, int E, const uint16_t* x, const float* gate_w, float* logits,
                          uint8_t* x_q, uint8_t* x_s, bool mfma_order, hipStream_t s);
// sqrt(softplus) scores, biased top-k, normalised route weights; at M > kRouterSmallM, or with mfma_order, also
// the per-32 E4M3 QDQ of x.
void launch_router_select_qdq(int M, int H, int E, int k, float route_scale, const float* logits,
                              const float* gate_b, const uint16_t* x, int32_t* ids, float* rw,
                              uint8_t* x_q, uint8_t* x_s, bool mfma_order, hipStream_t s);

// ---- permutation (permute.hip) -------------------------------------------------------------
// Stable counting sort of the M*k (token, slot) pairs by expert id. active may be null (no active list: for
// callers whose expert GEMMs read the row-tile map).
void launch_permute(int P, int E, const int32_t* ids, int32_t* counts, int32_t* offsets,
                    int32_t* pairs, int32_t* inv, int32_t* active, hipStream_t s);
// M <= kRouterSmallM only: the router's selection (from the partial logit planes) and the counting sort in
// one block; ids and rw equal launch_router_select_qdq's bit for bit.
// out_rows (nullable) [M*k]: for each sorted position, the row t*k + r of its pair (t, j), r = the rank of
// ids[t, j] among the token's k ids (ascending): slot rows written there are in ascending-id order per token.
void launch_select_permute_small(int M, int H, int E, int k, float route_scale, const float* logits,
                                 const float* gate_b, int32_t* ids, float* rw, int32_t* counts,
                                 int32_t* offsets, int32_t* pairs, int32_t* inv, int32_t* active, int32_t* out_rows,
                                 hipStream_t s);

// ---- expert GEMMs (expert_gemm.hip) --------------------------------------------------------
enum WeightFormat { W_MXFP4 = 0, W_FP8_BLOCK32 = 1, W_BF16 = 2 };

struct GemmProblem {
  // weights: GEMM1 uses wa = w1, wb = w3; GEMM2 uses wa = w2 (wb unused). Per-expert strides in
  // elements of the storage type (bytes for MXFP4/FP8, bf16 elements for BF16).
  const void* wa; const uint8_t* sa;
  const void* wb; const uint8_t* sb;
  long long w_expert_stride;   // storage elements per expert matrix
  long long s_expert_stride;   // scale bytes per expert matrix
  int N;                       // weight rows (output features)
  int K;                       // inner dimension
  // activations: E4M3 codes [rows, K] and E8M0 scales [rows, K/32]
  const uint8_t* act_q; const uint8_t* act_s;
  // routing: dense = one pseudo-expert over rows 0..M-1 in order (shared expert)
  int dense; int M; int k;
  int num_experts;             // E (routed problems)
  const int32_t* offsets;      // [E + 1]
  const int32_t* pairs;        // [M * k]: pair id t * k + j at each sorted position
  const int32_t* active;       // [E]: active expert ids (ascending, -1 padded)
  const float* rw;             // [M * k] route weight per pair (GEMM1, routed only)
  int act_by_token;            // 1: activation row = token of the pair; 0: row = sorted position
  // outputs
  uint8_t* h_q; uint8_t* h_s;  // GEMM1: QDQ'd h codes [rows, N] and scales [rows, N/32]
  uint16_t* out;               // GEMM2: bf16 [*, N]; row = pair id (routed) or token (dense)
  const int32_t* out_rows;     // GEMM2 (routed, decode-width kernels only): if set, the output row of each sorted
                               // position instead of its pair id
  float* out_f32;              // GEMM2: if set, the unrounded fp32 sums [*, N] instead of out
  // MXFP4 scales in the stage-major copy made by launch_scales_stage_major (block-scaled MFMA kernels
  // only): [E][K/128][N][4] instead of [E][N][K/32]
  int s_stage_major;
  // activation scales stage-major by sorted position, [K/128][M*k][4] (routed block-scaled MFMA only)
  int a_stage_major;
  // GEMM1 output scales h_s written stage-major, [N/128][M*k][4], for a GEMM2 with a_stage_major
  int h_s_stage_major;
  // MXFP4 weight codes in fragment order (launch_tile_mxfp4): per expert [N/16][K/128][64 lanes][16 B]
  // instead of [N][K/2]; same expert stride
  int w_tiled;
};
// GEMM1: g = w1 x, u = w3 x -> bf16 -> SwiGLU (x rw) -> bf16 -> QDQ per 32 -> h_q, h_s
void launch_gemm1_small(WeightFormat f, const GemmProblem& p, int max_active, hipStream_t s);
// GEMM2: y = w2 h -> bf16 rows
void launch_gemm2_small(WeightFormat f, const GemmProblem& p, int max_active, hipStream_t s);
// The same at decode width on the block-scaled matrix cores (MXFP4 or FP8 weights only).
void launch_gemm1_stream(WeightFormat f, const GemmProblem& p, int max_active, hipStream_t s);
void launch_gemm2_stream(WeightFormat f, const GemmProblem& p, int max_active, hipStream_t s);

// ---- decoded-BF16 arm at prefill widths (expert_bf16.hip) ---------------------------------------
// The routed problems of the *_small launchers with W_BF16 weights on the bf16 matrix cores, over the row-tile
// list of launch_tile_map; activation scales and h_s row-major.
void launch_gemm1_bf16(const GemmProblem& p, int max_tiles, const int32_t* tile_e, const int32_t* tile_r0,
                       const int32_t* info, hipStream_t s);
void launch_gemm2_bf16(const GemmProblem& p, int max_tiles, const int32_t* tile_e, const int32_t* tile_r0,
                       const int32_t* info, hipStream_t s);

// ---- expert GEMMs on the block-scaled matrix cores (expert_mfma.hip) ---------------------------
// Upper bound of the row-tile list for P (token, slot) pairs over E experts.
int mfma_max_tiles(int P, int E);
// Row-tile list from the expert offsets: tile_e [max_tiles] (-1 past the end), tile_r0 [max_tiles],
// info [1 + 2E] (tile count, first tile and tile count of each expert).
void launch_tile_map(int E, int max_tiles, const int32_t* offsets, int32_t* tile_e, int32_t* tile_r0, int32_t* info,
                     hipStream_t s);
// Same problems as the *_small launchers (MXFP4 or FP8 weights only); routed problems take the tile list.
// Stage-major copy of MXFP4 E8M0 scales for the block-scaled MFMA kernels: mats matrices s[m][N][K/32]
// -> S[m][K/128][N][4], so the 4 scale bytes of one 128-wide K step of consecutive rows are contiguous
// (one stage's scales of 64 rows are 256 contiguous bytes instead of 64 strided dwords).
void launch_scales_stage_major(int mats, int N, int K, const uint8_t* s, uint8_t* S, hipStream_t st);
// Activation scales of the P = M*k sorted pairs, stage-major: out[K/128][P][4] from x_s[token][K/32],
// token = pairs[pos] / k (pairs == nullptr: token = pos, i.e. rows already in sorted order).
void launch_gather_act_scales(int P, int k, int K, const int32_t* pairs, const uint8_t* x_s, uint8_t* out,
                              hipStream_t st);
// MXFP4 weights in the fragment-order copy with stage-major scales of both operands (expert_wide.hip): the
// 512 x 128 block tile, one wave per SIMD. Routed problems only.
void launch_gemm1_wide(const GemmProblem& p, int max_tiles, const int32_t* tile_e, const int32_t* tile_r0,
                       const int32_t* info, hipStream_t s);
void launch_gemm2_wide(const GemmProblem& p, int max_tiles, const int32_t* tile_e, const int32_t* tile_r0,
                       const int32_t* info, hipStream_t s);
void launch_gemm1_mfma(WeightFormat f, const GemmProblem& p, int max_tiles, const int32_t* tile_e,
                       const int32_t* tile_r0, const int32_t* info, hipStream_t s);
void launch_gemm2_mfma(WeightFormat f, const GemmProblem& p, int max_tiles, const int32_t* tile_e,
                       const int32_t* tile_r0, const int32_t* info, hipStream_t s);

// ---- combine (combine.hip) -----------------------------------------------------------------
// fp32 slot partials (the SLOT mode of the expert FFN). official: y = 0; y += float(bf16(slot)) over the
// token's slots in ascending id; y += float(bf16(shared_f32)) or float(shared_bf16) if given; out_bf16 =
// bf16(y). sum: out_f32 = fp32 sum of the slots in ascending id, then + add if given (no rounding).
void launch_combine_official_f32(int M, int H, int k, const int32_t* ids, const float* slot_f32,
                                 const float* shared_f32, const uint16_t* shared_bf16, uint16_t* out, hipStream_t s);
void launch_combine_sum_f32(int M, int H, int k, const int32_t* ids, const float* slot_f32, const float* add,
                            float* out, hipStream_t s);
// ---- dense FP8 linear (dense.hip) ----------------------------------------------------------
// Per-32 E4M3 QDQ of every row of x [M, K].
void launch_qdq_rows(int M, int K, const uint16_t* x, uint8_t* xq, uint8_t* xs, hipStream_t s);
// y = bf16(x_hat W^T) (or fp32 into y32) for M <= 64: W FP8 [N, K] with E8M0 [N/32, K/32]; N % 64 == 0.
// With x (bf16 [M, K]) the blocks QDQ their runs themselves and xq / xs are not read. w_tiled: w is the
// fragment-order copy (launch_tile_mxfp4(1, N, 2 K, ...) of the row-major codes).
void launch_fp8_linear_stream(int M, int N, int K, const uint16_t* x, const uint8_t* xq, const uint8_t* xs,
                              const uint8_t* w, bool w_tiled, const uint8_t* s, float* part, uint16_t* y, float* y32,
                              hipStream_t st);

// ids == nullptr: the token's k slot rows t*k .. t*k + k - 1 are already in ascending expert-id order.
void launch_combine(int M, int H, int k, const int32_t* ids, const uint16_t* slot_out,
                    const uint16_t* shared_out, uint16_t* out, hipStream_t s);

// ---- expansion of packed experts to bf16 (expand.hip) --------------------------------------
// Fragment order of packed E2M1 codes: mats matrices w[m][N][K/2] -> T[m][N/16][K/128][64][16] with
// T[m][f][q][l][b] = w[m][16 f + l % 16][64 q + 16 (l / 16) + b] (N % 16 == 0, K % 128 == 0).
void launch_tile_mxfp4(int mats, int N, int K, const uint8_t* w, uint8_t* out, hipStream_t s);
void launch_expand_mxfp4(long long rows, int cols, const uint8_t* w, const uint8_t* sc, uint16_t* out,
                         hipStream_t s);

}  // namespace moe
