// Grouping of the expert-input rows by expert on gfx950: per-block token histogram,
// prefix scan, stable scatter.  Deterministic: no result depends on the order in which
// atomics land (LDS integer adds and bit ORs commute).
//
// Rows: group g < E holds the tokens routed to expert g in ascending token order; group
// E + s (shared expert s) holds all tokens, rows [T k + s T, T k + (s + 1) T).
#include "moe_device.h"
#include "moe_launch.h"

namespace moe {

// Tokens of block b: [b * 256, (b + 1) * 256).  block_hist[b][e] = routed assignments of
// those tokens to expert e.
__global__ __launch_bounds__(256) void perm_hist_kernel(const int32_t* __restrict__ topk_idx,
                                                        int T, int E, int k,
                                                        int32_t* __restrict__ block_hist) {
  extern __shared__ int32_t cnt[];  // [E]
  for (int e = threadIdx.x; e < E; e += blockDim.x) cnt[e] = 0;
  __syncthreads();
  const int t = blockIdx.x * kPermBlock + threadIdx.x;
  if (t < T)
    for (int j = 0; j < k; ++j) {
      const int e = topk_idx[(size_t)t * k + j];
      if (e >= 0 && e < E) atomicAdd(&cnt[e], 1);
    }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += blockDim.x)
    block_hist[(size_t)blockIdx.x * E + e] = cnt[e];
}

// One workgroup of 1024 threads.  counts[e] = sum over blocks; offsets = exclusive scan of
// counts over all E + S groups; block_hist[b][e] becomes the first row of block b's tokens
// within group e.
__global__ __launch_bounds__(1024) void perm_scan_kernel(int32_t* __restrict__ block_hist,
                                                         int nblocks, int T, int E, int S,
                                                         int32_t* __restrict__ counts,
                                                         int32_t* __restrict__ offsets) {
  __shared__ int32_t scan[1024];
  const int G = E + S;
  const int g = threadIdx.x;
  int c = 0;
  if (g < E) {
    for (int b = 0; b < nblocks; ++b) {
      int32_t* p = block_hist + (size_t)b * E + g;
      const int v = *p;
      *p = c;  // exclusive prefix over blocks
      c += v;
    }
  } else if (g < G) {
    c = T;
  }
  // Inclusive Hillis-Steele scan over the groups.
  scan[g] = c;
  __syncthreads();
  for (int o = 1; o < 1024; o <<= 1) {
    const int v = g >= o ? scan[g - o] : 0;
    __syncthreads();
    scan[g] += v;
    __syncthreads();
  }
  const int start = scan[g] - c;
  if (g < G) {
    counts[g] = c;
    offsets[g] = start;
  }
  if (g == G - 1) offsets[G] = scan[g];
  if (g < E)
    for (int b = 0; b < nblocks; ++b) block_hist[(size_t)b * E + g] += start;
}

// Each wave takes 64 consecutive tokens.  For every expert e the wave ORs a 64-bit mask of
// its lanes (tokens) that chose e; a token's rank inside the block's run of group e is
// the popcount of the lower lanes of its own wave plus all lanes of the earlier waves.
__global__ __launch_bounds__(256) void perm_scatter_kernel(
    const int32_t* __restrict__ topk_idx, int T, int E, int S, int k,
    const int32_t* __restrict__ block_base, int32_t* __restrict__ row_token,
    int32_t* __restrict__ slot_row) {
  extern __shared__ unsigned long long mask[];  // [4][E]
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  for (int i = threadIdx.x; i < 4 * E; i += blockDim.x) mask[i] = 0ull;
  __syncthreads();
  const int t = blockIdx.x * kPermBlock + threadIdx.x;
  const bool live = t < T;
  const int A = k + S;
  if (live)
    for (int j = 0; j < k; ++j) {
      const int e = topk_idx[(size_t)t * k + j];
      if (e >= 0 && e < E) atomicOr(&mask[wave * E + e], 1ull << lane);
    }
  __syncthreads();
  if (live) {
    const unsigned long long below = (1ull << lane) - 1ull;
    const int32_t* base = block_base + (size_t)blockIdx.x * E;
    for (int j = 0; j < k; ++j) {
      const int e = topk_idx[(size_t)t * k + j];
      if (e < 0 || e >= E) continue;
      int rank = base[e];
      for (int w = 0; w < wave; ++w) rank += __popcll(mask[w * E + e]);
      rank += __popcll(mask[wave * E + e] & below);
      row_token[rank] = t;
      slot_row[(size_t)t * A + j] = rank;
    }
    for (int s = 0; s < S; ++s) {
      const int row = T * k + s * T + t;
      row_token[row] = t;
      slot_row[(size_t)t * A + k + s] = row;
    }
  }
}

// Batches of at most 256 tokens (one token block): the three steps above in one
// workgroup of 1024 threads, so a decode step pays one launch instead of three.  Waves
// 0..3 hold the tokens (64 each) and build the same per-wave expert masks as
// perm_scatter_kernel, whose popcounts give the histogram; every thread then scans one
// group as perm_scan_kernel does, and the token waves place their rows.  The results
// equal the three-kernel path's.
__global__ __launch_bounds__(1024) void perm_small_kernel(
    const int32_t* __restrict__ topk_idx, int T, int E, int S, int k,
    int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
    int32_t* __restrict__ row_token, int32_t* __restrict__ slot_row) {
  extern __shared__ unsigned long long mask[];  // [4][E]
  __shared__ int32_t scan[1024];
  const int G = E + S, A = k + S;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  for (int i = tid; i < 4 * E; i += blockDim.x) mask[i] = 0ull;
  __syncthreads();
  const int t = tid;
  const bool live = wave < 4 && t < T;
  if (live)
    for (int j = 0; j < k; ++j) {
      const int e = topk_idx[(size_t)t * k + j];
      if (e >= 0 && e < E) atomicOr(&mask[wave * E + e], 1ull << lane);
    }
  __syncthreads();
  const int g = tid;
  int c = 0;
  if (g < E) {
    for (int w = 0; w < 4; ++w) c += __popcll(mask[w * E + g]);
  } else if (g < G) {
    c = T;
  }
  // Inclusive Hillis-Steele scan over the groups.
  scan[g] = c;
  __syncthreads();
  for (int o = 1; o < 1024; o <<= 1) {
    const int v = g >= o ? scan[g - o] : 0;
    __syncthreads();
    scan[g] += v;
    __syncthreads();
  }
  const int start = scan[g] - c;
  if (g < G) {
    counts[g] = c;
    offsets[g] = start;
  }
  if (g == G - 1) offsets[G] = scan[g];
  __syncthreads();
  // scan[e] - (group e's count) is group e's first row; recompute it per row below.
  if (live) {
    const unsigned long long below = (1ull << lane) - 1ull;
    for (int j = 0; j < k; ++j) {
      const int e = topk_idx[(size_t)t * k + j];
      if (e < 0 || e >= E) continue;
      int before = 0, cnt = 0;
      for (int w = 0; w < 4; ++w) {
        const int pc = __popcll(mask[w * E + e]);
        cnt += pc;
        if (w < wave) before += pc;
      }
      const int rank = scan[e] - cnt + before + __popcll(mask[wave * E + e] & below);
      row_token[rank] = t;
      slot_row[(size_t)t * A + j] = rank;
    }
    for (int s = 0; s < S; ++s) {
      const int row = T * k + s * T + t;
      row_token[row] = t;
      slot_row[(size_t)t * A + k + s] = row;
    }
  }
}

hipError_t launch_permute(const int32_t* topk_idx, int T, int E, int S, int k,
                          int32_t* block_hist, int32_t* counts, int32_t* offsets,
                          int32_t* row_token, int32_t* slot_row, hipStream_t stream) {
  const int nb = (T + kPermBlock - 1) / kPermBlock;
  if (nb == 1) {
    hipLaunchKernelGGL(perm_small_kernel, dim3(1), dim3(1024),
                       4 * E * sizeof(unsigned long long), stream, topk_idx, T, E, S, k,
                       counts, offsets, row_token, slot_row);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(perm_hist_kernel, dim3(nb), dim3(kPermBlock), E * sizeof(int32_t),
                     stream, topk_idx, T, E, k, block_hist);
  hipLaunchKernelGGL(perm_scan_kernel, dim3(1), dim3(1024), 0, stream, block_hist, nb, T, E,
                     S, counts, offsets);
  hipLaunchKernelGGL(perm_scatter_kernel, dim3(nb), dim3(kPermBlock),
                     4 * E * sizeof(unsigned long long), stream, topk_idx, T, E, S, k,
                     block_hist, row_token, slot_row);
  return hipGetLastError();
}

}  // namespace moe
