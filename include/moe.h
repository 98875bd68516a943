/*
 * moe.h -- C ABI of the MI355X (gfx950) mixture-of-experts feed-forward layer.
 *
 * The layer (per token x, already normalized by the block's pre-norm):
 *   router   l = W_r x over the E routed and S shared experts, a linear scoring of the
 *            experts ("Qwen3.8-2.4T-A95B vs Inkling", component table, router row);
 *   select   either the softmax top-k router (softmax over the routed experts, keep the
 *            top k, renormalize; Qwen3.8 column of that row) or the sigmoid router with a
 *            shared-expert sink (sigmoid scores, top-k of the routed experts steered by a
 *            per-expert selection bias, weights normalized jointly over the k + S active
 *            experts then multiplied by route_scale = k + S; Inkling column of that row,
 *            and "Inkling vs Gemma 4 31B", component table, shared-expert row);
 *   experts  SwiGLU FFNs E_j(x) = W_down,j (SiLU(W_gate,j x) * W_up,j x)
 *            ("Inkling vs Gemma 4 31B", routed-expert row; SiLU per the Qwen3.8 2.4T A95B
 *            atlas page, hidden_act);
 *   combine  y = sum over active j of w_j E_j(x), optionally added to a residual
 *            ("Qwen3.5-397B-A17B vs Inkling", block diagram, residual add after the MoE).
 *
 * Conventions shared by every entry point
 *   - All tensor pointers are DEVICE pointers to caller-owned, contiguous, row-major
 *     buffers.  The library never allocates, frees or synchronizes; every call only
 *     enqueues kernels on `stream` and returns.
 *   - bf16 tensors hold IEEE bfloat16 bit patterns; f32 tensors IEEE binary32.  The
 *     selection bias, logit offset, combine weights, outputs and the per-row expert
 *     outputs are always f32.
 *   - Layouts:  x [T, d];  w_router [E + S, d] (shared experts' rows last);
 *     w_gate, w_up [E + S, I, d];  w_down [E + S, d, I];  every weight matrix is
 *     contiguous along the reduction dimension.
 *   - Rows: the T (k + S) expert-input rows are grouped by expert.  Group g < E holds the
 *     tokens routed to expert g in ascending token order; group E + s (shared expert s)
 *     holds every token in order, rows [T k + s T, T k + (s + 1) T).
 *   - Pointers to tensors read with 16-byte vector loads (x, weights, y_rows, out,
 *     residual, ws) must be 16-byte aligned; ws must be 256-byte aligned.
 *   - Errors: argument problems are reported synchronously, before anything is enqueued
 *     (MOE_ERR_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE).  A failed launch returns
 *     MOE_ERR_HIP.  T = 0 is a no-op returning MOE_OK.  No C++ exception crosses the ABI.
 *   - Supported shapes: d % 256 == 0, I % 128 == 0, 1 <= k <= min(E, 32),
 *     E + S <= 1024, 0 <= S <= 8; the softmax router requires route_scale == 1 and
 *     bias_on_logits == 0 (its S shared experts are ungated).
 *     Token counts: R = T (k + S) grouped rows with R * max(d, I) <= 2^31, and x [T, d]
 *     and the intermediate [R, I + 64] each under 2^31 bytes in the layer's dtype
 *     (MOE_ERR_UNSUPPORTED otherwise).
 *   - Calls that share a workspace must be ordered on one stream.  The library holds no
 *     global mutable state, so distinct streams with distinct workspaces are independent.
 *   - Every entry point only enqueues kernels on `stream` (no allocation, copy, memset or
 *     synchronization; the counters the kernels use live in the workspace and are reset
 *     by a kernel of the same call), so calls can be captured into a HIP graph and
 *     replayed.  The one exception is a debugging switch: with the environment variable
 *     MOE_DEBUG_SYNC=1 every entry point synchronizes its stream after its launches and
 *     reports a failed kernel as MOE_ERR_HIP.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_ARG = 1,          /* null/misaligned pointer, bad size or enum value */
  MOE_ERR_UNSUPPORTED = 2,  /* valid layer, but a shape this build does not tile */
  MOE_ERR_WORKSPACE = 3,    /* ws_bytes below moe_workspace_size() */
  MOE_ERR_HIP = 4           /* a kernel launch failed */
} moe_status_t;

typedef enum {
  MOE_ROUTER_SOFTMAX_TOPK = 0,    /* softmax over E, top-k, renormalize; S ungated shared
                                     experts (weight 1, no router rows) */
  MOE_ROUTER_SIGMOID_SHARED = 1   /* sigmoid over E + S, bias-steered top-k, joint norm */
} moe_router_t;

typedef enum { MOE_F32 = 0, MOE_BF16 = 1 } moe_dtype_t;

typedef struct {
  int32_t d_model;         /* d: model width */
  int32_t n_experts;       /* E: routed experts */
  int32_t d_ff;            /* I: expert intermediate size */
  int32_t top_k;           /* k: routed experts per token */
  int32_t n_shared;        /* S: shared (always-active) experts, 0..8 */
  int32_t router;          /* moe_router_t */
  int32_t dtype;           /* moe_dtype_t of x, w_router and the expert weights */
  int32_t bias_on_logits;  /* sigmoid router: 0 = selection bias added to the score
                              sigmoid(l) (default reading), 1 = added to the logit */
  float route_scale;       /* sigmoid: factor after the joint normalization (k + S);
                              softmax: must be 1 */
} moe_config_t;

/* Human-readable name of a status code (static storage; never NULL). */
const char* moe_status_str(moe_status_t status);

/* Bytes of device workspace every entry point below needs for `T` tokens (host only,
 * never touches the GPU).  The same workspace serves all entry points. */
moe_status_t moe_workspace_size(const moe_config_t* cfg, int64_t T, size_t* bytes);

/* Router: logits with f32 accumulation of exact products, selection, and combine
 * weights (definition: the router row of the component table of "Qwen3.8-2.4T-A95B vs
 * Inkling"; shared-expert weighting: "Inkling vs Gemma 4 31B", shared-expert row, which
 * sets Inkling's router-weighted shared experts against the blueprint's ungated one).
 *   x [T, d] (dtype)
 *   w_router [NR, d] (dtype): sigmoid router NR = E + S (shared experts' rows last);
 *            softmax router NR = E (its shared experts are ungated and have no row)
 *   sel_bias [E] f32 or NULL: sigmoid router only; steers selection, not the weights
 *   logit_offset [E] f32 or NULL: added to the routed experts' logits before scoring
 *   topk_idx [T, k] int32 out: routed experts in descending selection score; equal
 *            scores keep the lower index first
 *   weights  [T, k + S] f32 out: the routed experts' weights in topk_idx order, then the
 *            shared experts' weights; sigmoid: all k + S sum to route_scale; softmax: the
 *            k routed weights sum to 1 and each shared weight is exactly 1
 *   ws: workspace of at least moe_workspace_size() bytes. */
moe_status_t moe_route(const moe_config_t* cfg, int64_t T, const void* x,
                       const void* w_router, const float* sel_bias,
                       const float* logit_offset, int32_t* topk_idx, float* weights,
                       void* ws, size_t ws_bytes, hipStream_t stream);

/* Grouping of the T (k + S) expert-input rows by expert: per-expert token histogram,
 * exclusive prefix scan and a stable (ascending token) permutation.  This step is the
 * GPU method's own; it has no counterpart on the pages.
 *   topk_idx [T, k] int32 in: entries must lie in [0, E) and be distinct per token
 *            (out-of-range entries are skipped and leave rows unassigned)
 *   counts   [E + S] int32 out: rows per group (shared groups hold T)
 *   offsets  [E + S + 1] int32 out: exclusive prefix of counts; offsets[E + S] = T(k + S)
 *   row_token [T (k + S)] int32 out: token of each grouped row
 *   slot_row  [T (k + S)] int32 out: slot_row[t (k + S) + j] = row of token t's j-th
 *             active expert (j < k routed in topk_idx order, then the shared experts) */
moe_status_t moe_permute(const moe_config_t* cfg, int64_t T, const int32_t* topk_idx,
                         int32_t* counts, int32_t* offsets, int32_t* row_token,
                         int32_t* slot_row, void* ws, size_t ws_bytes, hipStream_t stream);

/* Grouped SwiGLU experts over the grouped rows ("Inkling vs Gemma 4 31B", routed- and
 * shared-expert rows): for every group g and each of its rows r (token t = row_token[r]),
 *   h = SiLU(W_gate,g x_t) * (W_up,g x_t)      (f32 accumulation; bf16 dtype rounds h to
 *                                                bf16 once, to nearest even)
 *   y_rows[r] = W_down,g h                      (f32 accumulation, f32 out)
 *   offsets [E + S + 1], row_token [T (k + S)]: as produced by moe_permute
 *   y_rows [T (k + S), d] f32 out. */
moe_status_t moe_grouped_swiglu(const moe_config_t* cfg, int64_t T, const void* x,
                                const int32_t* offsets, const int32_t* row_token,
                                const void* w_gate, const void* w_up, const void* w_down,
                                float* y_rows, void* ws, size_t ws_bytes,
                                hipStream_t stream);

/* Weighted combine back to token order, reading each token's k + S rows (no scatter):
 *   out[t] = [residual[t] +] sum_{j < k + S} weights[t, j] * y_rows[slot_row[t (k+S) + j]]
 * summed in the fixed order j = 0 .. k + S - 1 ("Qwen3.5-397B-A17B vs Inkling", block
 * diagram, residual add).  residual [T, d] f32 or NULL; out [T, d] f32. */
moe_status_t moe_combine(const moe_config_t* cfg, int64_t T, const float* y_rows,
                         const int32_t* slot_row, const float* weights,
                         const float* residual, float* out, hipStream_t stream);

/* The whole layer: route, group, grouped SwiGLU experts, combine, on one stream.
 *   out [T, d] f32; residual [T, d] f32 or NULL;
 *   topk_idx_out [T, k] int32 or NULL, counts_out [E + S] int32 or NULL: optional copies
 *   of the routing for inspection. */
moe_status_t moe_forward(const moe_config_t* cfg, int64_t T, const void* x,
                         const void* w_router, const float* sel_bias,
                         const float* logit_offset, const void* w_gate, const void* w_up,
                         const void* w_down, const float* residual, float* out,
                         int32_t* topk_idx_out, int32_t* counts_out, void* ws,
                         size_t ws_bytes, hipStream_t stream);

/* Pre-norm RMSNorm of the layer input, the step that pre-norm blocks run before the
 * layer ("Qwen3.5-397B-A17B vs Inkling" and "Qwen3.8-2.4T-A95B vs Inkling", residual-stream
 * rows and block diagrams; zero-centred gains for Qwen3.8; rms_norm_eps on the Qwen3.8
 * atlas page):
 *   y[t, c] = x[t, c] / sqrt(mean_c x[t, c]^2 + eps) * (zero_centred + gain[c])
 * with the sum of squares accumulated in f32; bf16 layers round y once to bf16 (nearest
 * even).  x, y [T, d] and gain [d] in the config's dtype; eps > 0; zero_centred 0 or 1.
 * d <= 16384 (MOE_ERR_UNSUPPORTED above).  y may not alias x. */
moe_status_t moe_rmsnorm(const moe_config_t* cfg, int64_t T, const void* x,
                         const void* gain, float eps, int32_t zero_centred, void* y,
                         hipStream_t stream);

/* The pre-norm block's branch in one call: moe_rmsnorm of the raw hidden states x into the
 * workspace, then moe_forward on the normalized input.  Arguments as in moe_rmsnorm and
 * moe_forward (the residual, if given, is added to the layer's output). */
moe_status_t moe_forward_rmsnorm(const moe_config_t* cfg, int64_t T, const void* x,
                                 const void* norm_gain, float eps, int32_t zero_centred,
                                 const void* w_router, const float* sel_bias,
                                 const float* logit_offset, const void* w_gate,
                                 const void* w_up, const void* w_down, const float* residual,
                                 float* out, int32_t* topk_idx_out, int32_t* counts_out,
                                 void* ws, size_t ws_bytes, hipStream_t stream);

/* Packed MXFP4 scales.  The MXFP4 entry points below take each weight tensor's E8M0
 * scales, defined row-major as [E, N, K/32] (row n, MX block kb = elements 32 kb .. +31 of
 * K), in a packed order: for each expert e, each block of 64 rows nb and each run of 8 MX
 * blocks kr, a 512-byte record of 64 rows x 8 bytes,
 *   packed[(((e * N/64 + nb) * KR + kr) * 64 + r) * 8 + j] = scale[e, 64 nb + r, 8 kr + j]
 * with KR = ceil(K / 256) and zero bytes where 8 kr + j >= K/32.  One wave's scales for 32
 * rows and 256 elements of K are then 256 contiguous bytes.  Weights are packed once, when
 * they are loaded.
 *
 * moe_mxfp4_scales_bytes (host only): size of the packed tensor, E * (N/64) * KR * 512.
 * moe_mxfp4_pack_scales: scales (device, [E, N, K/32] uint8) -> packed (device, that
 * size, 16-byte aligned, not overlapping scales), enqueued on stream.
 * Both: MOE_ERR_ARG for E, N or K <= 0 or a NULL / misaligned pointer; MOE_ERR_UNSUPPORTED
 * unless N % 64 == 0 and K % 32 == 0, or if one expert's packed scales reach 2 GiB. */
moe_status_t moe_mxfp4_scales_bytes(int64_t E, int64_t N, int64_t K, size_t* bytes);
moe_status_t moe_mxfp4_pack_scales(int64_t E, int64_t N, int64_t K, const uint8_t* scales,
                                   uint8_t* packed, hipStream_t stream);

/* MXFP4 routed experts (next to the decode shape's HBM bound: ~4.25 bits per weight).
 * The routed experts' weights arrive block-scaled FP4: Inkling's FP4 checkpoint keeps its
 * shared experts in BF16 ("Inkling vs Gemma 4 31B", shared-expert row) and the pages name
 * MXFP4/NVFP4 ("Qwen3.5-397B-A17B vs Inkling", block diagram, FP4 training box) without
 * defining it; the OCP Microscaling definition is used: per 32 consecutive K elements one
 * E8M0 scale byte s (2^(s - 127), 255 = NaN), elements E2M1 (sign, 2 exponent bits with
 * bias 1, 1 mantissa bit), two per byte with element 2i in the low nibble.  The experts
 * compute on the exactly dequantized weights with bf16 x, as in moe_grouped_swiglu.
 *   wq_gate, wq_up [E, I, d/2] uint8; ws_gate, ws_up the packed scales of [E, I, d/32]
 *   (moe_mxfp4_pack_scales with N = I, K = d); wq_down [E, d, I/2] uint8; ws_down the
 *   packed scales of [E, d, I/32] (N = d, K = I); codes and scales 16-byte aligned;
 *   w_gate_shared, w_up_shared [S, I, d] bf16, w_down_shared [S, d, I] bf16 (NULL iff
 *   S = 0).  bf16 layers only (MOE_ERR_UNSUPPORTED otherwise). */
moe_status_t moe_grouped_swiglu_mxfp4(const moe_config_t* cfg, int64_t T, const void* x,
                                      const int32_t* offsets, const int32_t* row_token,
                                      const uint8_t* wq_gate, const uint8_t* ws_gate,
                                      const uint8_t* wq_up, const uint8_t* ws_up,
                                      const uint8_t* wq_down, const uint8_t* ws_down,
                                      const void* w_gate_shared, const void* w_up_shared,
                                      const void* w_down_shared, float* y_rows, void* ws,
                                      size_t ws_bytes, hipStream_t stream);

/* The whole layer with MXFP4 routed experts (arguments as in moe_forward and
 * moe_grouped_swiglu_mxfp4). */
moe_status_t moe_forward_mxfp4(const moe_config_t* cfg, int64_t T, const void* x,
                               const void* w_router, const float* sel_bias,
                               const float* logit_offset, const uint8_t* wq_gate,
                               const uint8_t* ws_gate, const uint8_t* wq_up,
                               const uint8_t* ws_up, const uint8_t* wq_down,
                               const uint8_t* ws_down, const void* w_gate_shared,
                               const void* w_up_shared, const void* w_down_shared,
                               const float* residual, float* out, int32_t* topk_idx_out,
                               int32_t* counts_out, void* ws, size_t ws_bytes,
                               hipStream_t stream);

/* For callers that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation): the whole layer as moe_forward, with
 * its scratch space in a static device array inside the library instead of a caller
 * workspace.  Arguments as in moe_forward, without ws and ws_bytes.
 *   - Limit: moe_workspace_size(cfg, T) must not exceed MOE_STATIC_SCRATCH_BYTES (64 MiB:
 *     up to ~230 tokens at the Inkling shape, ~160 at the Qwen3.8 shape); larger token
 *     counts return MOE_ERR_WORKSPACE before anything is enqueued.
 *   - Memory: each GPU the library runs on holds its own copy of the array until the
 *     process ends.  The first call on a device looks up that copy's address (no
 *     allocation); later calls on the device reuse it.  No call allocates or frees.
 *   - Sharing: every call on one GPU uses that GPU's one array, so calls that overlap on
 *     one GPU (on different streams, or from different host threads without ordering)
 *     race and give undefined results; order them on one stream.  Each call rebuilds
 *     every counter and plan it reads, so what an earlier call left in the array does
 *     not matter.
 *   - Errors: as moe_forward; MOE_ERR_HIP also if the device's array cannot be resolved. */
#define MOE_STATIC_SCRATCH_BYTES ((size_t)64 << 20)
moe_status_t moe_forward_static(const moe_config_t* cfg, int64_t T, const void* x,
                                const void* w_router, const float* sel_bias,
                                const float* logit_offset, const void* w_gate,
                                const void* w_up, const void* w_down, const float* residual,
                                float* out, int32_t* topk_idx_out, int32_t* counts_out,
                                hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H */
