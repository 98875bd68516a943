// Router of the MoE layer on gfx950: logits l = W_r x with f32 accumulation, then a
// wavefront-wide top-k and the combine weights.
//
// Definition followed: the router row of the component table of "Qwen3.8-2.4T-A95B vs
// Inkling" (a linear router; softmax top-k with renormalization for Qwen3.8; sigmoid
// scores over routed + shared experts, bias-steered top-k and weights normalized jointly
// over the active experts then multiplied by their count for Inkling) and the
// shared-expert row of "Inkling vs Gemma 4 31B" (each shared expert weighted by its own
// router score).
#include "moe_device.h"
#include "moe_launch.h"

namespace moe {

// ---------------------------------------------------------------------------------------
// Logits.  One workgroup (4 waves) owns 64 tokens x 64 experts of one K chunk; each wave
// a 32 x 32 block as 2 x 2 MFMA tiles.  bf16 products are exact in f32, so the only
// rounding is the f32 accumulation.  Operands go straight from global memory (x rows and
// router rows are reused out of L2) into the MFMA register layout; no LDS.
// Two accumulator sets (even / odd K steps) halve the length of each f32 sum.
// ---------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void router_logits_bf16(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ wr, float* __restrict__ part,
    int T, int d, int NE, int kchunk) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int t0 = blockIdx.x * kRouterTile + (wave & 1) * 32;
  const int e0 = blockIdx.y * kRouterTile + (wave >> 1) * 32;
  const int split = blockIdx.z;
  const int kbeg = split * kchunk;
  const int kend = min(d, kbeg + kchunk);
  // v_mfma_f32_16x16x32_bf16 operands: lane l holds row (l % 16), K elements
  // [8 (l / 16), 8 (l / 16) + 8) of its 32-wide K step.
  const int r = lane & 15, kq = (lane >> 4) * 8;
  const uint16_t* a0 = x + (size_t)min(t0 + r, T - 1) * d + kq;
  const uint16_t* a1 = x + (size_t)min(t0 + 16 + r, T - 1) * d + kq;
  const uint16_t* b0 = wr + (size_t)min(e0 + r, NE - 1) * d + kq;
  const uint16_t* b1 = wr + (size_t)min(e0 + 16 + r, NE - 1) * d + kq;
  f32x4 c[2][2][2] = {};
  int k = kbeg;
  for (; k + 64 <= kend; k += 64) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      bf16x8 A0 = *reinterpret_cast<const bf16x8*>(a0 + k + 32 * h);
      bf16x8 A1 = *reinterpret_cast<const bf16x8*>(a1 + k + 32 * h);
      bf16x8 B0 = *reinterpret_cast<const bf16x8*>(b0 + k + 32 * h);
      bf16x8 B1 = *reinterpret_cast<const bf16x8*>(b1 + k + 32 * h);
      c[h][0][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A0, B0, c[h][0][0], 0, 0, 0);
      c[h][0][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A0, B1, c[h][0][1], 0, 0, 0);
      c[h][1][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A1, B0, c[h][1][0], 0, 0, 0);
      c[h][1][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A1, B1, c[h][1][1], 0, 0, 0);
    }
  }
  if (k < kend) {  // one trailing 32-wide step
    bf16x8 A0 = *reinterpret_cast<const bf16x8*>(a0 + k);
    bf16x8 A1 = *reinterpret_cast<const bf16x8*>(a1 + k);
    bf16x8 B0 = *reinterpret_cast<const bf16x8*>(b0 + k);
    bf16x8 B1 = *reinterpret_cast<const bf16x8*>(b1 + k);
    c[0][0][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A0, B0, c[0][0][0], 0, 0, 0);
    c[0][0][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A0, B1, c[0][0][1], 0, 0, 0);
    c[0][1][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A1, B0, c[0][1][0], 0, 0, 0);
    c[0][1][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A1, B1, c[0][1][1], 0, 0, 0);
  }
  // Result layout: lane l holds column (l % 16), rows 4 (l / 16) + i.
  float* out = part + (size_t)split * T * NE;
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int ni = 0; ni < 2; ++ni)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        int t = t0 + 16 * mi + 4 * (lane >> 4) + i;
        int e = e0 + 16 * ni + (lane & 15);
        if (t < T && e < NE) out[(size_t)t * NE + e] = c[0][mi][ni][i] + c[1][mi][ni][i];
      }
}

// f32 inputs: the same tiling on v_mfma_f32_16x16x4_f32 (lane l holds row l % 16,
// K element l / 16 of each 4-wide step).
__global__ __launch_bounds__(256) void router_logits_f32(
    const float* __restrict__ x, const float* __restrict__ wr, float* __restrict__ part,
    int T, int d, int NE, int kchunk) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int t0 = blockIdx.x * kRouterTile + (wave & 1) * 32;
  const int e0 = blockIdx.y * kRouterTile + (wave >> 1) * 32;
  const int split = blockIdx.z;
  const int kbeg = split * kchunk;
  const int kend = min(d, kbeg + kchunk);
  const int r = lane & 15, kq = lane >> 4;
  const float* a0 = x + (size_t)min(t0 + r, T - 1) * d + kq;
  const float* a1 = x + (size_t)min(t0 + 16 + r, T - 1) * d + kq;
  const float* b0 = wr + (size_t)min(e0 + r, NE - 1) * d + kq;
  const float* b1 = wr + (size_t)min(e0 + 16 + r, NE - 1) * d + kq;
  f32x4 c[2][2] = {};
  for (int k = kbeg; k < kend; k += 4) {
    float A0 = a0[k], A1 = a1[k], B0 = b0[k], B1 = b1[k];
    c[0][0] = __builtin_amdgcn_mfma_f32_16x16x4f32(A0, B0, c[0][0], 0, 0, 0);
    c[0][1] = __builtin_amdgcn_mfma_f32_16x16x4f32(A0, B1, c[0][1], 0, 0, 0);
    c[1][0] = __builtin_amdgcn_mfma_f32_16x16x4f32(A1, B0, c[1][0], 0, 0, 0);
    c[1][1] = __builtin_amdgcn_mfma_f32_16x16x4f32(A1, B1, c[1][1], 0, 0, 0);
  }
  float* out = part + (size_t)split * T * NE;
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int ni = 0; ni < 2; ++ni)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        int t = t0 + 16 * mi + 4 * (lane >> 4) + i;
        int e = e0 + 16 * ni + (lane & 15);
        if (t < T && e < NE) out[(size_t)t * NE + e] = c[mi][ni][i];
      }
}

// ---------------------------------------------------------------------------------------
// Logits of bf16 batches of at least 256 tokens: one workgroup (4 waves, 2 x 2) owns 128
// tokens x 128 router rows of one K chunk, each wave 64 x 64 as 2 x 2
// v_mfma_f32_32x32x16_bf16 tiles.  Each 64-element K step of both tiles is loaded
// coalesced (8 lanes x 16 bytes per 128-byte row segment) one step ahead into registers
// and stored into the other of two LDS buffers, rows of 128 bytes with chunk c of row r
// at slot c ^ ((r / 2) % 8).  Rows past the batch or the router rows load a copy of the
// last one; their results are not stored.  Compared with the small-batch tiles this
// reads x 4x and the router rows 2x less often out of L2.
// ---------------------------------------------------------------------------------------
constexpr int kRtStage = 2 * kRouterBigTile * kRowBytes;   // A and B tiles, 32 KB

__global__ __launch_bounds__(256) void router_logits_bf16_tiled(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ wr, float* __restrict__ part,
    int T, int d, int NE, int kchunk) {
  __shared__ __attribute__((aligned(1024))) char smem[2 * kRtStage];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int wm = wave & 1, wn = wave >> 1;
  const int t0 = blockIdx.x * kRouterBigTile, e0 = blockIdx.y * kRouterBigTile;
  const int split = blockIdx.z;
  const int kbeg = split * kchunk;
  const int KT = (min(d, kbeg + kchunk) - kbeg) / 64;   // d and kchunk: multiples of 64
  const __amdgpu_buffer_rsrc_t xr = buffer_rsrc(x, static_cast<uint32_t>((size_t)T * d * 2));
  const __amdgpu_buffer_rsrc_t wrr =
      buffer_rsrc(wr, static_cast<uint32_t>((size_t)NE * d * 2));
  // Wave w stages 1 KB blocks 4 w .. 4 w + 3 of each tile; block b holds rows 8 b + l / 8,
  // and lane l's 16 bytes land at slot l % 8 of its row.
  uint32_t a_off[4], b_off[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = 8 * (4 * wave + i) + (lane >> 3);
    const int chunk = (lane & 7) ^ ((row >> 1) & 7);
    a_off[i] = static_cast<uint32_t>((size_t)min(t0 + row, T - 1) * d + 8 * chunk) * 2;
    b_off[i] = static_cast<uint32_t>((size_t)min(e0 + row, NE - 1) * d + 8 * chunk) * 2;
  }
  u32x4 ra[4], rb[4];
  f32x16 acc[2][2];
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int ni = 0; ni < 2; ++ni) acc[mi][ni] = f32x16{};
#define MOE_RT_FETCH(kt)                                                                \
  do {                                                                                  \
    const uint32_t k0_ = static_cast<uint32_t>(kbeg + 64 * (kt)) * 2;                   \
    _Pragma("unroll") for (int i = 0; i < 4; ++i) {                                     \
      ra[i] = load16(xr, a_off[i], k0_);                                                \
      rb[i] = load16(wrr, b_off[i], k0_);                                               \
    }                                                                                   \
  } while (0)
#define MOE_RT_STORE(slot)                                                              \
  do {                                                                                  \
    char* st_ = smem + (slot) * kRtStage + lane * 16;                                   \
    _Pragma("unroll") for (int i = 0; i < 4; ++i) {                                     \
      *reinterpret_cast<u32x4*>(st_ + (4 * wave + i) * 1024) = ra[i];                   \
      *reinterpret_cast<u32x4*>(st_ + kRouterBigTile * kRowBytes + (4 * wave + i) * 1024) = \
          rb[i];                                                                        \
    }                                                                                   \
  } while (0)
  MOE_RT_FETCH(0);
  MOE_RT_STORE(0);
  __syncthreads();
  for (int kt = 0; kt < KT; ++kt) {
    if (kt + 1 < KT) MOE_RT_FETCH(kt + 1);
    const char* sa = smem + (kt & 1) * kRtStage;
    const char* sb = sa + kRouterBigTile * kRowBytes;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      // 16-wide step s: lane l holds row l % 32, K elements 8 (l / 32) .. +8.
      const int chunk = 2 * s + (lane >> 5);
      bf16x8 fa[2], fb[2];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        fa[j] = *reinterpret_cast<const bf16x8*>(sa + swz(wm * 64 + j * 32 + (lane & 31), chunk));
        fb[j] = *reinterpret_cast<const bf16x8*>(sb + swz(wn * 64 + j * 32 + (lane & 31), chunk));
      }
#pragma unroll
      for (int mi = 0; mi < 2; ++mi)
#pragma unroll
        for (int ni = 0; ni < 2; ++ni)
          acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[mi], fb[ni], acc[mi][ni],
                                                                0, 0, 0);
    }
    if (kt + 1 < KT) MOE_RT_STORE((kt + 1) & 1);
    __syncthreads();
  }
#undef MOE_RT_STORE
#undef MOE_RT_FETCH
  // Accumulator layout: lane l, register r -> router row (l % 32), token
  // 8 (r / 4) + 4 (l / 32) + (r % 4) of the 32 x 32 tile.
  float* out = part + (size_t)split * T * NE;
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int ni = 0; ni < 2; ++ni)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int t = t0 + wm * 64 + mi * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        const int e = e0 + wn * 64 + ni * 32 + (lane & 31);
        if (t < T && e < NE) out[(size_t)t * NE + e] = acc[mi][ni][r];
      }
}

hipError_t launch_router_logits(int dtype, const void* x, const void* w_router, float* part,
                                int T, int d, int NE, int nsplit, int kchunk,
                                hipStream_t stream) {
  const int tile = router_tile(dtype, T);
  dim3 grid((T + tile - 1) / tile, (NE + tile - 1) / tile, nsplit);
  if (tile == kRouterBigTile)
    hipLaunchKernelGGL(router_logits_bf16_tiled, grid, dim3(256), 0, stream,
                       static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(w_router),
                       part, T, d, NE, kchunk);
  else if (dtype == 1)
    hipLaunchKernelGGL(router_logits_bf16, grid, dim3(256), 0, stream,
                       static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(w_router),
                       part, T, d, NE, kchunk);
  else
    hipLaunchKernelGGL(router_logits_f32, grid, dim3(256), 0, stream,
                       static_cast<const float*>(x), static_cast<const float*>(w_router), part,
                       T, d, NE, kchunk);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------------
// Selection.  One wave per token; lane l holds experts l, l + 64, ...  Each of the k
// rounds takes the wave-wide maximum of 64-bit keys (order-preserving f32 bits of the
// selection score in the high word, the inverted expert index in the low word, so equal
// scores resolve to the lower index) and retires the winner.
//   sigmoid: s = 1 / (1 + exp(-l)); selection score s + b (or sigmoid(l + b) when the
//            bias applies to the logit); weight route_scale * s_j / sum over the active
//            set (routed in selection order, then shared) of s.
//   softmax: logits over the E routed experts only; selection on the logit (monotone
//            in the probability); weight exp(l_j - l_top) / sum over the top k of
//            exp(l_i - l_top), which equals the renormalized softmax probability; the S
//            shared experts are ungated: weight 1.
// ---------------------------------------------------------------------------------------
template <int MAXV>
__global__ __launch_bounds__(256) void topk_kernel(
    const float* __restrict__ part, int nsplit, int T, int E, int S, int k, int router,
    int bias_on_logits, float route_scale, const float* __restrict__ sel_bias,
    const float* __restrict__ logit_offset, int32_t* __restrict__ topk_idx,
    float* __restrict__ weights) {
  __shared__ float sval[4][64];
  __shared__ float sden[4];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + wave;
  const int NE = router == 1 ? E + S : E;   // logit columns
  const bool live = t < T;
  float raw[MAXV];
  uint64_t key[MAXV];
  // Logits: the nsplit partial sums added in split order.  The loads of 8 splits of every
  // slot are issued together (a runtime-length loop of dependent adds per slot would
  // serialize nsplit x MAXV memory latencies); the adds keep the order, and the padding
  // +0 terms cannot change a sum that starts at +0.
  float lsum[MAXV];
#pragma unroll
  for (int i = 0; i < MAXV; ++i) lsum[i] = 0.f;
  for (int s0 = 0; s0 < nsplit; s0 += 8) {
    float pv[8][MAXV];
#pragma unroll
    for (int u = 0; u < 8; ++u)
#pragma unroll
      for (int i = 0; i < MAXV; ++i) {
        const int e = lane + 64 * i;
        pv[u][i] = (live && e < NE && s0 + u < nsplit)
                       ? part[((size_t)(s0 + u) * T + t) * NE + e]
                       : 0.f;
      }
#pragma unroll
    for (int u = 0; u < 8; ++u)
#pragma unroll
      for (int i = 0; i < MAXV; ++i) lsum[i] += pv[u][i];
  }
#pragma unroll
  for (int i = 0; i < MAXV; ++i) {
    const int e = lane + 64 * i;
    raw[i] = 0.f;
    key[i] = 0;
    if (live && e < NE) {
      float l = lsum[i];
      if (logit_offset != nullptr && e < E) l += logit_offset[e];
      float sel;
      if (router == 1) {
        const float sc = 1.0f / (1.0f + expf(-l));
        raw[i] = sc;
        const float b = (sel_bias != nullptr && e < E) ? sel_bias[e] : 0.0f;
        sel = bias_on_logits ? 1.0f / (1.0f + expf(-(l + b))) : sc + b;
      } else {
        raw[i] = l;
        sel = l;
      }
      if (e < E)
        key[i] = (static_cast<uint64_t>(f32_order_key(sel)) << 32) |
                 (0xffffffffu - static_cast<uint32_t>(e));
    }
  }
  for (int j = 0; j < k; ++j) {
    uint64_t best = 0;
#pragma unroll
    for (int i = 0; i < MAXV; ++i) best = key[i] > best ? key[i] : best;
    best = wave_max_u64(best);
    const int e = static_cast<int>(0xffffffffu - static_cast<uint32_t>(best));
    if (live && lane == (e & 63)) {
      const int slot = e >> 6;
      float v = 0.f;
#pragma unroll
      for (int i = 0; i < MAXV; ++i)
        if (i == slot) {
          v = raw[i];
          key[i] = 0;
        }
      sval[wave][j] = v;
      topk_idx[(size_t)t * k + j] = e;
    }
  }
  // Shared experts' raw scores follow the routed ones.
#pragma unroll
  for (int i = 0; i < MAXV; ++i) {
    const int e = lane + 64 * i;
    if (live && e >= E && e < NE) sval[wave][k + (e - E)] = raw[i];
  }
  __syncthreads();
  const int A = k + S;
  if (live && lane == 0) {
    float den = 0.f;
    if (router == 1) {
      for (int j = 0; j < A; ++j) den += sval[wave][j];
    } else {
      const float top = sval[wave][0];
      for (int j = 0; j < k; ++j) den += expf(sval[wave][j] - top);
    }
    sden[wave] = den;
  }
  __syncthreads();
  if (live && lane < A) {
    const float den = sden[wave];
    const float v = sval[wave][lane];
    const float w = (router == 1) ? route_scale * v / den
                    : (lane < k ? expf(v - sval[wave][0]) / den : 1.0f);
    weights[(size_t)t * A + lane] = w;
  }
}

hipError_t launch_topk(const float* part, int nsplit, int T, int E, int S, int k, int router,
                       int bias_on_logits, float route_scale, const float* sel_bias,
                       const float* logit_offset, int32_t* topk_idx, float* weights,
                       hipStream_t stream) {
  const int per_lane = ((router == 1 ? E + S : E) + 63) / 64;
  dim3 grid((T + 3) / 4);
#define MOE_TOPK(MV)                                                                      \
  hipLaunchKernelGGL(topk_kernel<MV>, grid, dim3(256), 0, stream, part, nsplit, T, E, S, \
                     k, router, bias_on_logits, route_scale, sel_bias, logit_offset,      \
                     topk_idx, weights)
  if (per_lane <= 1) MOE_TOPK(1);
  else if (per_lane <= 2) MOE_TOPK(2);
  else if (per_lane <= 4) MOE_TOPK(4);
  else if (per_lane <= 8) MOE_TOPK(8);
  else MOE_TOPK(16);
#undef MOE_TOPK
  return hipGetLastError();
}

}  // namespace moe
