/*
 * moe.h - C ABI of the MI355X (gfx950) routed-MoE FFN layer library (libmoe.so).
 *
 * The layer is the DeepSeek-V4-Flash-style routed mixture-of-experts FFN defined on the
 * page "Native 1017 DSpark draft on the NVLink pair (N1-NATIVE)":
 *   section 2 "Official semantics" - quantized linear, activation QDQ, Gate, Expert, MoE;
 *   section 4 "Kernel contract"    - inputs, packed/expanded weight formats, per-(t, j) math, outputs.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Every pointer argument is a DEVICE pointer owned by the caller, unless stated otherwise
 *   (the dims and weight-set structs themselves live in host memory). Tensors are dense, row-major,
 *   16-byte aligned; the workspace is 256-byte aligned.
 * - `stream` is a hipStream_t (NULL = the default stream). Work is only enqueued: no entry point
 *   synchronizes, allocates device memory or copies device data to the host. Routing never leaves
 *   the device.
 * - Arguments are validated on the host before anything is launched; a failed check returns a
 *   negative moe_status and enqueues nothing. There is no fallback path: an unsupported shape is
 *   refused. A failing launch returns MOE_ERR_HIP; faults inside kernels surface at the caller's
 *   next synchronization.
 * - Launch geometry depends only on (dims, M), never on routed data.
 * - A workspace must not be used by two calls in flight at the same time.
 * - M = 0 is a valid empty call (returns MOE_OK, enqueues nothing).
 *
 * Supported domain: 1 <= E <= 256, 1 <= k <= min(E, 8), H and I multiples of 128 and at most 8192, 0 <= M <= 2^24,
 * M * k <= 2^26, H * I <= 2^31.
 * H and I are inner dimensions of the matrix-core steps, which take 128 inputs at a time. An I that is a
 * multiple of 32 only (e.g. a quarter of 2304) is refused; widen it to the next multiple of 128 with
 * zero weight codes (w1 / w3 rows and w2 inputs of code 0, any valid scale): the padded rows give g = u =
 * h = 0 and the padded w2 inputs multiply zero codes, so every output keeps its value.
 * E8M0 scale bytes must be in 1..254 (255 is NaN; 0 is outside the supported range); E4M3 weight bytes
 * must be finite (not 0x7F/0xFF).
 *
 * Data formats (section 2):
 * - bf16: uint16 bit pattern. fp32: float.
 * - MXFP4 matrix [rows, cols]: uint8 [rows, cols/2]; byte j of a row holds input 2j in the low nibble
 *   and input 2j+1 in the high nibble; E2M1 magnitudes 0, .5, 1, 1.5, 2, 3, 4, 6, bit 3 = sign;
 *   one E8M0 scale byte per 32 inputs of a row, uint8 [rows, cols/32]; value = e2m1 * 2^(b-127).
 * - FP8 matrix [rows, cols]: E4M3fn bytes uint8 [rows, cols]; one E8M0 byte per 32x32 block,
 *   uint8 [rows/32, cols/32].
 * - QDQ'd activations (x_q/x_s, h_q/h_s): E4M3 codes uint8 [rows, n] and E8M0 bytes [rows, n/32],
 *   value = e4m3(code) * 2^(b-127); s = 2^ceil(log2(max(amax, 1e-4) / 448)) per 32 inputs.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

/* Kernel family of the routed GEMMs, a function of (dims, M) only: while M * top_k is below
 * MOE_TILED_ROWS_PER_EXPERT * num_experts (fewer than that many rows per expert on average) the weights
 * stream through the decode-width kernels (each expert's rows in passes of up to 8); from there on the
 * GEMMs run over a row-tile list of 128 rows per expert tile. Outputs stay within the stated tolerance
 * on either side; their bits can change where M crosses the boundary (the fp32 summation order differs). */
#define MOE_TILED_ROWS_PER_EXPERT 6

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t moe_status;
#define MOE_OK 0
#define MOE_ERR_INVALID_ARG (-1) /* null or misaligned pointer, negative size, bad dims       */
#define MOE_ERR_UNSUPPORTED (-2) /* shape outside the supported domain                        */
#define MOE_ERR_WORKSPACE (-3)   /* workspace smaller than moe_workspace_bytes(dims, M)       */
#define MOE_ERR_HIP (-4)         /* a kernel launch failed                                    */

/* Layer dimensions (host struct). */
typedef struct {
  int32_t num_experts; /* E: routed experts                         */
  int32_t hidden;      /* H: model width (x and output columns)     */
  int32_t inter;       /* I: expert intermediate width              */
  int32_t top_k;       /* k: experts per token                      */
  float route_scale;   /* multiplies the normalised route weights   */
  uint32_t flags;      /* MOE_FLAG_* bits; 0 = default              */
} moe_dims;

/* Batch invariance. Every stage after the router computes each token's rows with the same arithmetic in the
 * same order whatever the batch (the streamed and row-tiled GEMMs give the same bits per row), but the router
 * sums its fp32 logits in one order up to M = 64 tokens (512-wide chunks, 64 lanes' 8-term FMA chains) and in
 * another above (the matrix cores over 32-wide steps of exact bf16 parts), so a token's route weights, and
 * rarely its output bits, can change when a batch crosses M = 64 / 65. With MOE_FLAG_BATCH_INVARIANT the
 * router takes its matrix-core kernel at every M (at decode widths slower: about 33 us more at M = 8 on the
 * full-size layer, through the separate selection and permutation kernels): a token's ids, route weights and
 * outputs are then the same bits in every batch. Above 64 tokens the flag changes nothing. Unknown flag bits
 * are refused (MOE_ERR_INVALID_ARG). */
#define MOE_FLAG_BATCH_INVARIANT 1u

/* Routed experts in packed MXFP4 (section 1 table, section 2 formats). Host struct of device pointers. */
typedef struct {
  const uint8_t* w1; /* [E, I, H/2]  gate projection  */
  const uint8_t* s1; /* [E, I, H/32]                  */
  const uint8_t* w3; /* [E, I, H/2]  up projection    */
  const uint8_t* s3; /* [E, I, H/32]                  */
  const uint8_t* w2; /* [E, H, I/2]  down projection  */
  const uint8_t* s2; /* [E, H, I/32]                  */
  /* Optional (NULL = none): the output of moe_prepare_mxfp4_scales for these scales. The prefill-width
   * kernels read the scales from it; without it every prefill-width call re-lays them out in the
   * workspace. */
  const uint8_t* stage_scales;
  /* Optional (NULL = none): the output of moe_prepare_mxfp4_weights for w1, w3, w2. When given, every
   * routed GEMM reads the weight codes from it (each 128-bit load then covers 1 KB of contiguous bytes)
   * and w1, w3, w2 may be NULL; the scales are still read from s1, s3, s2 (and stage_scales). */
  const uint8_t* tiled_weights;
} moe_mxfp4_experts;

/* Routed experts expanded to bf16 (section 4 "expanded weights": exactly code * 2^(b-127)). */
typedef struct {
  const uint16_t* w1; /* [E, I, H] */
  const uint16_t* w3; /* [E, I, H] */
  const uint16_t* w2; /* [E, H, I] */
} moe_bf16_experts;

/* Shared expert in FP8 E4M3 with E8M0 32x32 block scales (section 1 table, section 2). */
typedef struct {
  const uint8_t* w1; /* [I, H]        */
  const uint8_t* s1; /* [I/32, H/32]  */
  const uint8_t* w3; /* [I, H]        */
  const uint8_t* s3; /* [I/32, H/32]  */
  const uint8_t* w2; /* [H, I]        */
  const uint8_t* s2; /* [H/32, I/32]  */
} moe_fp8_expert;

/* Bytes of workspace the entry points need for up to max_tokens rows; 0 if dims are invalid.
 * Holds the router logits, routing, QDQ'd x, permutation, QDQ'd h of every (token, slot), the
 * per-slot bf16 expert outputs and the shared expert's intermediates. */
size_t moe_workspace_bytes(const moe_dims* dims, int32_t max_tokens);

/* Human-readable name of a status code (static string). */
const char* moe_status_str(moe_status status);

/* Router + activation QDQ (section 2 "Gate" and "Quantized linear").
 * x bf16 [M, H] (raw, not QDQ'd), gate_w fp32 [E, H], gate_b fp32 [E] ->
 * ids int32 [M, k]: the k largest sqrt(softplus(x W^T)) + bias, descending, ties to the lower id;
 * rw fp32 [M, k]: route_scale * s[ids] / (sum_j s[ids_j] + 1e-20), the sum taken in slot order;
 * x_q uint8 [M, H], x_s uint8 [M, H/32]: QDQ of x per 32 inputs (shared by all experts). */
moe_status moe_route(const moe_dims* dims, int32_t M, const uint16_t* x, const float* gate_w, const float* gate_b,
                     int32_t* ids, float* rw, uint8_t* x_q, uint8_t* x_s, void* ws, size_t ws_bytes, void* stream);

/* Token-to-expert permutation: a stable counting sort of the M*k pairs p = t*k + j by ids[p]. The layer's
 * math (section 2 "MoE") sums each token's k expert outputs; grouping the pairs by expert is how the
 * expert GEMMs read each expert's packed weights once for all its rows: the expert sorter of the paper
 * "DeepSeek-V4-Flash on AMD gfx90a" (section 7.1, rows of one expert gathered into blocks) and the
 * (token, expert) emitter and the grouped route-direct chain screened on the page "DeepSeek V4 Flash
 * REAP/XPU B70 Handoff". The order is stable, so the result does not depend on how the sort is scheduled.
 * counts int32 [E]; offsets int32 [E+1] (exclusive prefix sum, offsets[E] = number of valid pairs);
 * pairs int32 [M*k]: pair ids grouped by expert, ascending within an expert; inv int32 [M*k]
 * (nullable): position of each pair in `pairs`; active int32 [E]: experts with counts > 0 in
 * ascending order, then -1. Ids outside [0, E) are ignored. */
moe_status moe_permute(const moe_dims* dims, int32_t M, const int32_t* ids, int32_t* counts, int32_t* offsets,
                       int32_t* pairs, int32_t* inv, int32_t* active, void* stream);

/* Routed experts (section 4 math per (t, j)): for each pair p at sorted position q with expert e,
 * g = bf16(x_hat w1[e]^T), u = bf16(x_hat w3[e]^T), h = rw[p] * silu(min(g, 10)) * clamp(u, -10, 10)
 * in fp32, h16 = bf16(h), (h_q, h_s) = QDQ(h16), slot_out[p] = bf16(h_hat w2[e]^T).
 * Exactly one of `packed` / `decoded` is non-NULL (the decoded-BF16 arm computes the same values
 * from expanded weights). x_q/x_s from moe_route; rw [M*k]; offsets/pairs/active from moe_permute.
 * slot_out bf16 [M*k, H] indexed by pair id. h_q uint8 [M*k, I] / h_s uint8 [M*k, I/32] indexed
 * by sorted position: both NULL = kept in the workspace, or both given to receive them. */
moe_status moe_expert_ffn(const moe_dims* dims, int32_t M, const uint8_t* x_q, const uint8_t* x_s,
                          const moe_mxfp4_experts* packed, const moe_bf16_experts* decoded, const float* rw,
                          const int32_t* offsets, const int32_t* pairs, const int32_t* active,
                          uint16_t* slot_out, uint8_t* h_q, uint8_t* h_s, void* ws, size_t ws_bytes,
                          void* stream);

/* The two halves of moe_expert_ffn, for callers that time or schedule them separately.
 * moe_expert_gemm1: h_q uint8 [M*k, I] and h_s uint8 [M*k, I/32] (rows = sorted positions) from
 *   x_q/x_s: g, u, clamped SwiGLU times rw, bf16, QDQ per 32 (section 4 math up to hq).
 * moe_expert_gemm2: slot_out bf16 [M*k, H] (rows = pair ids) = bf16(h_hat w2[e]^T).
 * Same argument rules as moe_expert_ffn. The workspace (moe_workspace_bytes(dims, M)) holds the
 * row-tile list the prefill-width kernels build from `offsets`; each call builds its own. */
moe_status moe_expert_gemm1(const moe_dims* dims, int32_t M, const uint8_t* x_q, const uint8_t* x_s,
                            const moe_mxfp4_experts* packed, const moe_bf16_experts* decoded, const float* rw,
                            const int32_t* offsets, const int32_t* pairs, const int32_t* active, uint8_t* h_q,
                            uint8_t* h_s, void* ws, size_t ws_bytes, void* stream);
moe_status moe_expert_gemm2(const moe_dims* dims, int32_t M, const uint8_t* h_q, const uint8_t* h_s,
                            const moe_mxfp4_experts* packed, const moe_bf16_experts* decoded,
                            const int32_t* offsets, const int32_t* pairs, const int32_t* active,
                            uint16_t* slot_out, void* ws, size_t ws_bytes, void* stream);

/* Shared expert (section 2 "Expert", FP8 weights, no route weight) on every row:
 * shared_out bf16 [M, H] = bf16(QDQ(bf16(silu(min(g,10)) * clamp(u,-10,10))) w2^T). */
moe_status moe_shared_expert(const moe_dims* dims, int32_t M, const uint8_t* x_q, const uint8_t* x_s,
                             const moe_fp8_expert* shared, uint16_t* shared_out, void* ws, size_t ws_bytes,
                             void* stream);

/* Combine (section 2 "MoE"): out[t] = bf16(fp32 sum of slot_out[t*k + j] over the token's slots in
 * ascending ids[t, j] order, then + shared_out[t] if shared_out is not NULL). out bf16 [M, H]. */
moe_status moe_combine(const moe_dims* dims, int32_t M, const int32_t* ids, const uint16_t* slot_out,
                       const uint16_t* shared_out, uint16_t* out, void* stream);

/* The whole layer: moe_route -> moe_permute -> moe_expert_ffn -> (moe_shared_expert) -> moe_combine.
 * Exactly one of packed / decoded is non-NULL; shared may be NULL. out bf16 [M, H].
 * ids_out [M, k], rw_out [M, k] and shared_out [M, H] are optional (NULL = workspace only). */
moe_status moe_forward(const moe_dims* dims, int32_t M, const uint16_t* x, const float* gate_w, const float* gate_b,
                       const moe_mxfp4_experts* packed, const moe_bf16_experts* decoded, const moe_fp8_expert* shared,
                       uint16_t* out, int32_t* ids_out, float* rw_out, uint16_t* shared_out, void* ws,
                       size_t ws_bytes, void* stream);

/* For callers that cannot allocate device memory or pass a workspace: code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation. The same layer as moe_forward (same arguments
 * minus ws / ws_bytes, same kernels, bit-identical results), with its workspace in a library-owned device
 * array of MOE_NOALLOC_SCRATCH_BYTES per GPU (held from the first call on a device until the process
 * ends). It calls no allocating routine.
 * Limit: the call is refused with MOE_ERR_WORKSPACE (nothing enqueued) when moe_workspace_bytes(dims, M)
 * exceeds MOE_NOALLOC_SCRATCH_BYTES; the full-size layer (E 128, H 5120, I 2304, k 6) fits up to M = 64 with
 * or without the shared expert. The stream must belong to the current device (else MOE_ERR_INVALID_ARG).
 * Every call on one GPU uses that GPU's one array, and nothing in it needs clearing between calls (each
 * call writes every buffer before reading it); calls that overlap in time on one GPU (different streams or
 * threads) race on it and must be serialised by the caller. */
#define MOE_NOALLOC_SCRATCH_BYTES (16u << 20)
moe_status moe_forward_noalloc(const moe_dims* dims, int32_t M, const uint16_t* x, const float* gate_w,
                               const float* gate_b, const moe_mxfp4_experts* packed, const moe_bf16_experts* decoded,
                               const moe_fp8_expert* shared, uint16_t* out, int32_t* ids_out, float* rw_out,
                               uint16_t* shared_out, void* stream);

/* ---- fp32 partial outputs for a tensor-parallel split of I (section 3 "combine modes"; section 4 "outputs",
 * modes SLOT and COMBINE). A rank holding I/G of every expert's w1/w3 rows and w2 inputs (dims.inter =
 * I/G; QDQ blocks never straddle the cut) produces fp32 partial sums; after an all-reduce of the
 * partials, the exact-official combine rounds each (row, slot) sum to bf16 and adds them in ascending
 * expert id, as the single-device layer does. */

/* Mode SLOT: as moe_expert_ffn, but slot_f32 [M*k, H] (rows = pair ids t*k + j) receives the unrounded
 * fp32 sums of h_hat w2[e]^T. h stays in the workspace. */
moe_status moe_expert_ffn_f32(const moe_dims* dims, int32_t M, const uint8_t* x_q, const uint8_t* x_s,
                              const moe_mxfp4_experts* packed, const moe_bf16_experts* decoded, const float* rw,
                              const int32_t* offsets, const int32_t* pairs, const int32_t* active, float* slot_f32,
                              void* ws, size_t ws_bytes, void* stream);

/* The shared expert with the unrounded fp32 sums of its w2 (shared_f32 [M, H]) instead of bf16. */
moe_status moe_shared_expert_f32(const moe_dims* dims, int32_t M, const uint8_t* x_q, const uint8_t* x_s,
                                 const moe_fp8_expert* shared, float* shared_f32, void* ws, size_t ws_bytes,
                                 void* stream);

/* Mode COMBINE: out_f32 [M, H] = the token's fp32 slot sums added in fp32 in ascending ids[t, j] order,
 * then + add[t] (fp32 [M, H], e.g. a shared partial) if add is not NULL. No rounding. */
moe_status moe_combine_sum_f32(const moe_dims* dims, int32_t M, const int32_t* ids, const float* slot_f32,
                               const float* add, float* out_f32, void* stream);

/* Exact-official combine of (all-reduced) fp32 slot sums: y = 0 (fp32); y += float(bf16(slot)) over the
 * token's slots in ascending id order; then y += float(bf16(shared_f32[t])) or float(shared_bf16[t])
 * (at most one of the two; both NULL = no shared expert); out bf16 [M, H] = bf16(y). With one rank this
 * equals moe_combine on the bf16 slot outputs bit for bit. */
moe_status moe_combine_official_f32(const moe_dims* dims, int32_t M, const int32_t* ids, const float* slot_f32,
                                    const float* shared_f32, const uint16_t* shared_bf16, uint16_t* out,
                                    void* stream);

/* ---- Dense FP8 linear (section 4 "Dense", the projection family wq_a 1280 x 5120, wkv 512 x 5120,
 * wq_b 16384 x 1280, wo_b 5120 x 4096, main_proj 5120 x 15360, shared w1/w3/w2): y = bf16(act_qdq(x) W^T)
 * with W FP8 E4M3 uint8 [N, K] and one E8M0 scale per 32x32 block, s uint8 [N/32, K/32]; act_qdq is the
 * per-32 E4M3 QDQ of each row of x (section 2 "Quantized linear"). x bf16 [M, K]; exactly one of y
 * (bf16 [M, N]) or y_f32 (the unrounded fp32 sums [M, N], e.g. a tensor-parallel partial) is given.
 * N and K multiples of 128 (at most 65536), M*K and M*N at most 2^31. The workspace holds the QDQ'd x
 * and, at M <= 64, the partial sums of the split inner dimension. */
size_t moe_fp8_linear_workspace_bytes(int32_t M, int32_t N, int32_t K);
moe_status moe_fp8_linear(int32_t M, int32_t N, int32_t K, const uint16_t* x, const uint8_t* w, const uint8_t* s,
                          uint16_t* y, float* y_f32, void* ws, size_t ws_bytes, void* stream);

/* Bytes of moe_prepare_fp8_weights output: N * K (0 for a shape moe_fp8_linear refuses). */
size_t moe_fp8_tiled_weights_bytes(int32_t N, int32_t K);

/* One-time re-layout of a dense FP8 weight matrix (the operand of section 4 "Dense") for the decode-width
 * kernel: w uint8 E4M3 [N, K] row-major -> out[f][q][l][b] = w[16 f + l % 16][64 q + 16 (l / 16) + b]
 * (f < N / 16 row fragments, q < K / 64 chunks of 64 bytes, lane l < 64, byte b < 16), so that every weight
 * load of a wave reads 1 KB of consecutive bytes. Same values in another order, done once (e.g. at load).
 * w and out: device, 16-byte aligned, not overlapping; out holds moe_fp8_tiled_weights_bytes(N, K) bytes
 * and is owned by the caller. Errors: INVALID_ARG (NULL, misaligned or overlapping pointers),
 * UNSUPPORTED (a shape moe_fp8_linear refuses). */
moe_status moe_prepare_fp8_weights(int32_t N, int32_t K, const uint8_t* w, uint8_t* out, void* stream);

/* moe_fp8_linear with the weights given as the moe_prepare_fp8_weights copy (w_tiled), for decode widths:
 * M <= 64, UNSUPPORTED above (the prefill-width kernel reads the row-major codes). Outputs are bit-identical
 * to moe_fp8_linear's on the same inputs; same scales s, workspace and errors otherwise. */
moe_status moe_fp8_linear_tiled(int32_t M, int32_t N, int32_t K, const uint16_t* x, const uint8_t* w_tiled,
                                const uint8_t* s, uint16_t* y, float* y_f32, void* ws, size_t ws_bytes,
                                void* stream);

/* Bytes of moe_prepare_mxfp4_scales output: 3 * E * I * H / 32 (0 if dims are invalid). */
size_t moe_mxfp4_stage_scales_bytes(const moe_dims* dims);

/* One-time re-layout of the routed experts' E8M0 scales for the prefill-width (block-scaled matrix
 * core) kernels, which read one 128-wide K step of many rows at a time. For each of s1, s3, s2 in that
 * order (matrix m = [E, N, K/32]: N = I, K = H for s1 and s3; N = H, K = I for s2), out holds
 * [E, K/128, N, 4] with out[e][q][n][b] = s[e][n][4q + b]. The scales are constant, so this is done
 * once (e.g. when the weights are loaded); the values are unchanged, only their order. out: device,
 * 16-byte aligned, moe_mxfp4_stage_scales_bytes(dims) bytes, owned by the caller. w's weight
 * pointers are not read (w->stage_scales is ignored). */
moe_status moe_prepare_mxfp4_scales(const moe_dims* dims, const moe_mxfp4_experts* w, uint8_t* out, void* stream);

/* Bytes of moe_prepare_mxfp4_weights output: 3 * E * I * H / 2 (0 if dims are invalid). */
size_t moe_mxfp4_tiled_weights_bytes(const moe_dims* dims);

/* One-time re-layout of the routed experts' packed E2M1 codes (section 2 MXFP4 format: w1, w3, w2; scales
 * untouched) into
 * matrix-core fragment order. The values are unchanged, only their order. For each matrix m in the order
 * w1, w3, w2 (m = [E, N, K/2] bytes: N = I, K = H for w1 and w3; N = H, K = I for w2), stored one after
 * the other (each E * I * H / 2 bytes), out holds [E, N/16, K/128, 64, 16]:
 *   out[e][f][q][l][b] = m[e][16 f + l % 16][64 q + 16 (l / 16) + b],
 * i.e. fragment (f, q) is the 16 rows 16f.. by the 128 inputs 128q.. in 1024 contiguous bytes, 16 per
 * lane l of the block-scaled matrix-core instruction (lane l: row l % 16, inputs 32 (l / 16) .. + 31).
 * Done once (e.g. when the weights are loaded). out: device, 16-byte aligned,
 * moe_mxfp4_tiled_weights_bytes(dims) bytes, owned by the caller; must not overlap w's weights.
 * w's scale pointers and w->stage_scales / w->tiled_weights are not read. Errors (nothing enqueued):
 * MOE_ERR_INVALID_ARG for NULL or misaligned w1, w3, w2 or out, or an out that overlaps them;
 * MOE_ERR_INVALID_ARG / MOE_ERR_UNSUPPORTED for dims outside the supported domain. */
moe_status moe_prepare_mxfp4_weights(const moe_dims* dims, const moe_mxfp4_experts* w, uint8_t* out, void* stream);

/* Expand one packed MXFP4 matrix (or a stack of them) to bf16: w uint8 [rows, cols/2], s uint8
 * [rows, cols/32] -> out bf16 [rows, cols], exactly code * 2^(b-127) (section 4 "expanded weights").
 * cols a multiple of 32, rows >= 0. w is in the stored row-major layout (not the tiled one). */
moe_status moe_expand_mxfp4(int64_t rows, int32_t cols, const uint8_t* w, const uint8_t* s, uint16_t* out,
                            void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H */
