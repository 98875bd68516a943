// Host-side launchers of the MoE layer's gfx950 kernels (internal to the library).
// Arguments are validated by the C-ABI layer before any launcher runs.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "moe.h"

namespace moe {

// Every argument check of moe_forward except the workspace's (moe_api.cpp): the config,
// the token count and the pointers, in that order.  If ws_bytes_needed is not NULL and the
// config and token count are valid, it receives moe_workspace_size's value.  T = 0 returns
// MOE_OK after the config and token checks, before the pointer checks.
moe_status_t check_forward_args(const moe_config_t* cfg, int64_t T, const void* x,
                                const void* w_router, const float* sel_bias,
                                const void* w_gate, const void* w_up, const void* w_down,
                                const float* residual, const float* out,
                                size_t* ws_bytes_needed);

// Tile sizes of the grouped expert GEMMs, shared with the workspace planner.
constexpr int kGemmBM = 128;        // grouped rows per tile
constexpr int kGateUpBN = 128;      // h columns per gate/up tile (128 gate + 128 up rows)
constexpr int kDownBN = 256;        // y columns per down tile
constexpr int kPermBlock = 256;     // tokens per permute block
constexpr int kRouterTile = 64;     // tokens and experts per router tile (small batches)
constexpr int kRouterBigTile = 128; // tokens and experts per router tile, bf16, T >= 256

// Router tile edge for a batch: bf16 batches of at least 256 tokens use the LDS-staged
// 128 x 128 tiles.
inline int router_tile(int dtype, int64_t T) {
  return (dtype == 1 && T >= 2 * kRouterBigTile) ? kRouterBigTile : kRouterTile;
}

struct PlanEntry {   // one m-tile of the grouped GEMM
  int32_t group, row0, nrows, pad;
};

// Pre-norm RMSNorm: y = x / sqrt(mean(x^2) + eps) * (gain_offset + gain), per token.
hipError_t launch_rmsnorm(int dtype, const void* x, const void* gain, void* y, int T, int d,
                          float eps, float gain_offset, hipStream_t stream);

// Router partial logits: part[s][t][e] = sum over the s-th K chunk of x[t] . w_router[e].
hipError_t launch_router_logits(int dtype, const void* x, const void* w_router, float* part,
                                int T, int d, int NE, int nsplit, int kchunk,
                                hipStream_t stream);

// Selection and combine weights from the partial logits (summed in split order).
hipError_t launch_topk(const float* part, int nsplit, int T, int E, int S, int k,
                       int router, int bias_on_logits, float route_scale,
                       const float* sel_bias, const float* logit_offset, int32_t* topk_idx,
                       float* weights, hipStream_t stream);

// Histogram, scan and stable scatter of the grouped rows.
hipError_t launch_permute(const int32_t* topk_idx, int T, int E, int S, int k,
                          int32_t* block_hist, int32_t* counts, int32_t* offsets,
                          int32_t* row_token, int32_t* slot_row, hipStream_t stream);

// Grouped gate/up (+SwiGLU) and down GEMMs.  h is [R, I] (dtype) with row pitch
// h_pitch(I), y_rows [R, d] f32.
hipError_t launch_grouped_swiglu(int dtype, const void* x, const int32_t* offsets,
                                 const int32_t* row_token, const void* w_gate,
                                 const void* w_up, const void* w_down, void* h,
                                 float* y_rows, PlanEntry* plan, int T, int d, int I, int G,
                                 int R, hipStream_t stream);

// Packed MXFP4 scales: for each expert, each block of 64 rows of N and each run of 8 MX
// blocks (256 elements) of K, a record of 64 rows x 8 E8M0 bytes (row-major); the last
// record along K is zero-padded when K is not a multiple of 256.
constexpr int kMxRecRows = 64;
constexpr int kMxRecBlocks = 8;
constexpr int kMxRecBytes = kMxRecRows * kMxRecBlocks;
__host__ __device__ inline int64_t mx_rec_k(int64_t K) {
  return (K / 32 + kMxRecBlocks - 1) / kMxRecBlocks;
}
inline int64_t mx_scales_bytes(int64_t E, int64_t N, int64_t K) {
  return E * (N / kMxRecRows) * mx_rec_k(K) * kMxRecBytes;
}

// Row-major scales [E, N, K/32] -> the packed records (N % 64 == 0, K % 32 == 0).
hipError_t launch_pack_mx_scales(const uint8_t* src, uint8_t* dst, int64_t E, int64_t N,
                                 int64_t K, hipStream_t stream);

// MXFP4 routed-expert weights: codes [E, N, K/2] (element 2i in the low nibble) and packed
// E8M0 scales (above) per tensor (gate/up: N = I, K = d; down: N = d, K = I).
struct MxWeights {
  const uint8_t *codes_gate, *scales_gate, *codes_up, *scales_up, *codes_down, *scales_down;
};

// Grouped SwiGLU with MXFP4 routed experts and bf16 shared experts ([S, ...]); bf16 x.
hipError_t launch_grouped_swiglu_mxfp4(const uint16_t* x, const int32_t* offsets,
                                       const int32_t* row_token, const MxWeights& q,
                                       const uint16_t* wg_shared, const uint16_t* wu_shared,
                                       const uint16_t* wd_shared, uint16_t* h, float* y,
                                       PlanEntry* plan, int T, int d, int I, int E, int G,
                                       int R, hipStream_t stream);

// Weighted combine of each token's A = k + S rows, fixed order, optional residual.
hipError_t launch_combine(const float* y_rows, const int32_t* slot_row, const float* weights,
                          const float* residual, float* out, int T, int d, int A, int R,
                          hipStream_t stream);

// Upper bound of the grouped GEMM's m-tiles for R rows in G groups (the smallest m-tile,
// that of the MXFP4 decode tiles, has 16 rows).
constexpr int kMinTileRows = 16;
inline int64_t max_mtiles(int64_t R, int64_t G) { return R / kMinTileRows + G; }

// Row pitch (elements) of the intermediate h [R, I]: 64 elements of padding per row, so
// that the rows one K step of a tile reads do not all share their low address bits.
constexpr int kHPad = 64;
inline int64_t h_pitch(int64_t I) { return I + kHPad; }

// bf16 layers with at most 32 tokens (every group fits one 32-row m-tile) run the
// decode-shaped tiling.
constexpr int kDecodeMaxTokens = 32;

// bf16 layers whose groups average at least 128 rows run the 256-row tiling.
inline bool use_wide_tiles(int dtype, int64_t R, int64_t G) {
  return dtype == 1 && R >= 128 * G;
}

// The plan buffer: entry 0 (m-tile count), the m-tiles, then kSyncEntries entries that
// hold 16 uint32 phase counters (8 XCDs x 2 GEMMs), cleared by the plan kernel.
constexpr int kSyncEntries = 4;
inline int64_t plan_entries(int64_t R, int64_t G) { return 1 + max_mtiles(R, G) + kSyncEntries; }

}  // namespace moe
