// Grouped SwiGLU expert GEMMs on gfx950 (MFMA, LDS-staged tiles).
//
// Expert j computes E_j(x) = W_down,j (SiLU(W_gate,j x) * W_up,j x) ("Inkling vs Gemma 4
// 31B", component table, routed- and shared-expert rows; SiLU per the Qwen3.8 2.4T A95B
// atlas page, hidden_act).  Rows are grouped by expert, so each group is a dense
// NT-GEMM against that expert's weights (all operands contiguous along K).
//
//   gate/up:  h[r, n] = SiLU(sum_c x[tok(r), c] Wg[n, c]) * (sum_c x[tok(r), c] Wu[n, c])
//             x rows gathered on load through row_token; f32 accumulation; bf16 layers
//             round h to bf16 once (nearest even).
//   down:     y[r, n] = sum_i h[r, i] Wd[n, i], f32 accumulation and f32 output.
//
// Work decomposition.  A device-built plan lists the m-tiles (up to 128 rows of one
// group).  Tiles are ordered group by group, n-tile by n-tile, with the m-tiles of a
// group fastest, so the workgroups that run together share one expert's weight slice
// (read from HBM once, then from L2) and read the gathered rows at the same K offsets.
// The grid is an upper bound of the tile count; workgroup ids past the real count exit,
// and the real ones are remapped so that each XCD walks one contiguous range of tiles.
//
// Tile: 128 rows x 256 B-rows (gate/up: 128 gate + 128 up rows; down: 256 outputs).  K
// moves 128 bytes per row per step (64 bf16 / 32 f32) through a 3-stage LDS ring filled
// by direct global->LDS loads (global_load_lds_dwordx4), up to three steps ahead.
// LDS rows are 128 B; 16-byte chunk c of row r sits at slot c ^ (r & 7), so the eight
// rows read by one ds_read_b128 phase land on eight different bank groups.  A direct
// load writes 64 lanes x 16 B contiguously, so each lane fetches the global chunk that
// belongs at its slot.  Four waves in 2 x 2; each wave owns 64 rows x 128 B-rows as
// 2 x 4 MFMA 32x32 tiles (128 f32 accumulators per lane).
#include "moe_device.h"
#include "moe_launch.h"

namespace moe {

constexpr int kRowBytes = 128;
constexpr int kBM = kGemmBM;                  // 128
constexpr int kBRows = 256;
constexpr int kStageA = kBM * kRowBytes;      // 16 KB
constexpr int kStageB = kBRows * kRowBytes;   // 32 KB
constexpr int kStage = kStageA + kStageB;     // 48 KB
constexpr int kStages = 3;                    // 144 KB of the CU's 160 KB

__device__ __forceinline__ int swz(int row, int chunk) {
  return row * kRowBytes + ((chunk ^ (row & 7)) << 4);
}

typedef __attribute__((address_space(3))) void* lds_ptr_t;
typedef const __attribute__((address_space(1))) void* gbl_ptr_t;

// 16 bytes per lane from global memory straight into LDS at lds + 16 * lane.
__device__ __forceinline__ void load_lds16(const void* g, char* lds_wave_base) {
  __builtin_amdgcn_global_load_lds((gbl_ptr_t)(g),
                                   (lds_ptr_t)(lds_wave_base), 16, 0, 0);
}

template <typename TE>
struct Mfma;

// bf16: v_mfma_f32_32x32x16_bf16.  Operand lane l: row/col (l % 32), K elements
// [8 (l / 32), 8 (l / 32) + 8) of the 16-wide step, i.e. 16-byte chunk (l / 32) of the
// step's 32 bytes.
template <>
struct Mfma<uint16_t> {
  static constexpr int kSteps = 4;  // 16-wide K steps per 64-element LDS row
  typedef bf16x8 frag_t;
  __device__ static inline frag_t frag(const char* base, int row, int s, int lane) {
    const int chunk = 2 * s + (lane >> 5);
    return *reinterpret_cast<const bf16x8*>(base + swz(row, chunk));
  }
  __device__ static inline f32x16 mma(frag_t a, frag_t b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
};

// f32: v_mfma_f32_32x32x2_f32.  Operand lane l: row/col (l % 32), K element (l / 32) of
// the 2-wide step.
template <>
struct Mfma<float> {
  static constexpr int kSteps = 16;  // 2-wide K steps per 32-element LDS row
  typedef float frag_t;
  __device__ static inline frag_t frag(const char* base, int row, int s, int lane) {
    const int kk = 2 * s + (lane >> 5);
    return *reinterpret_cast<const float*>(base + swz(row, kk >> 2) + ((kk & 3) << 2));
  }
  __device__ static inline f32x16 mma(frag_t a, frag_t b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
  }
};

__device__ __forceinline__ float silu(float z) { return z / (1.0f + expf(-z)); }

__device__ __forceinline__ void store_h(uint16_t* p, float v) { *p = f32_to_bf16_rne(v); }
__device__ __forceinline__ void store_h(float* p, float v) { *p = v; }

// MODE 0: gate/up + SwiGLU -> h.  MODE 1: down -> y_rows.
template <typename TE, int MODE>
__global__ __launch_bounds__(256) void grouped_gemm_kernel(
    const TE* __restrict__ a_src,           // MODE 0: x [T, K]; MODE 1: h [R, K]
    const int32_t* __restrict__ row_token,  // MODE 0 only
    const TE* __restrict__ b0,              // MODE 0: w_gate [G, N, K]; MODE 1: w_down
    const TE* __restrict__ b1,              // MODE 0: w_up [G, N, K]
    const int32_t* __restrict__ offsets,    // [G + 1] group row offsets
    const PlanEntry* __restrict__ plan,     // plan[0].group = m-tile count
    void* __restrict__ c_out,               // MODE 0: h [R, N] (TE); MODE 1: y [R, N] f32
    int K, int N, int T, int NT) {
  constexpr int EPC = 16 / sizeof(TE);  // elements per 16-byte chunk
  constexpr int EPR = kRowBytes / sizeof(TE);
  __shared__ __attribute__((aligned(1024))) char smem[kStages * kStage];

  // ---- tile of this workgroup
  const uint32_t ntiles = static_cast<uint32_t>(plan[0].group) * NT;
  if (blockIdx.x >= ntiles) return;
  const uint32_t logical = xcd_remap(blockIdx.x, ntiles);
  const PlanEntry first = plan[1 + logical / NT];
  const int g = first.group, gmt0 = first.pad;
  const int mg = (offsets[g + 1] - offsets[g] + kBM - 1) / kBM;  // m-tiles of the group
  const uint32_t local = logical - static_cast<uint32_t>(gmt0) * NT;
  const int nt = local / mg;
  const PlanEntry pe = plan[1 + gmt0 + local % mg];
  const int row0 = pe.row0, nrows = pe.nrows;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int n0 = nt * (MODE == 0 ? kGateUpBN : kDownBN);

  // ---- per-lane global sources.  Wave w fills A blocks 4w..4w+3 and B blocks
  // 8w..8w+7 (a block = 1 KB = 8 rows); lane l of a block carries row 8 b + l / 8 and
  // logical chunk (l % 8) ^ (l / 8), which the swizzle places at physical slot l % 8.
  const int lrow = lane >> 3;
  const int lchunk = (lane & 7) ^ lrow;
  uint32_t a_off[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = 8 * (4 * wave + i) + lrow;
    const int rr = min(row, nrows - 1);
    uint32_t base;
    if (MODE == 0) {
      int tok = row_token[row0 + rr];
      tok = min(max(tok, 0), T - 1);
      base = static_cast<uint32_t>(tok) * K;
    } else {
      base = static_cast<uint32_t>(row0 + rr) * K;
    }
    a_off[i] = base + lchunk * EPC;
  }
  // gate/up: B-rows 0..127 (waves 0, 1) are gate rows n0.., B-rows 128..255 (waves 2,
  // 3) the up rows n0..;  down: B-rows 0..255 are w_down rows n0..
  const TE* bsrc;
  int brow0;
  if (MODE == 0) {
    bsrc = (wave < 2 ? b0 : b1) + ((size_t)g * N + n0) * K;
    brow0 = 64 * (wave & 1);
  } else {
    bsrc = b0 + ((size_t)g * N + n0) * K;
    brow0 = 64 * wave;
  }
  uint32_t b_off[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) b_off[i] = static_cast<uint32_t>(brow0 + 8 * i + lrow) * K +
                                         lchunk * EPC;

  const int wm = wave & 1, wn = wave >> 1;
  int brow[4];
#pragma unroll
  for (int ni = 0; ni < 4; ++ni) {
    if (MODE == 0)
      brow[ni] = (ni < 2 ? 0 : kGateUpBN) + wn * 64 + (ni & 1) * 32 + (lane & 31);
    else
      brow[ni] = wn * 128 + ni * 32 + (lane & 31);
  }
  int arow[2];
#pragma unroll
  for (int mi = 0; mi < 2; ++mi) arow[mi] = wm * 64 + mi * 32 + (lane & 31);

  f32x16 acc[2][4];
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int ni = 0; ni < 4; ++ni) acc[mi][ni] = f32x16{};

  // Issue the 12 direct loads of K step kt into ring slot kt % 3.
#define MOE_ISSUE(kt)                                                                   \
  do {                                                                                  \
    char* st_ = smem + ((kt) % kStages) * kStage;                                       \
    const int k0_ = (kt) * EPR;                                                         \
    _Pragma("unroll") for (int i = 0; i < 4; ++i)                                       \
        load_lds16(a_src + a_off[i] + k0_, st_ + (4 * wave + i) * 1024);                \
    _Pragma("unroll") for (int i = 0; i < 8; ++i)                                       \
        load_lds16(bsrc + b_off[i] + k0_, st_ + kStageA + (8 * wave + i) * 1024);       \
  } while (0)

  // Fragments of one 16-wide (bf16) / 2-wide (f32) K step, double-buffered so the LDS
  // reads of step s + 1 are in flight while the MFMAs of step s run.
  typedef typename Mfma<TE>::frag_t frag_t;
  constexpr int S = Mfma<TE>::kSteps;
  frag_t fa[2][2], fb[2][4];
#define MOE_LOADF(st, s, buf)                                                           \
  do {                                                                                  \
    fa[buf][0] = Mfma<TE>::frag((st), arow[0], (s), lane);                              \
    fa[buf][1] = Mfma<TE>::frag((st), arow[1], (s), lane);                              \
    _Pragma("unroll") for (int ni = 0; ni < 4; ++ni)                                    \
        fb[buf][ni] = Mfma<TE>::frag((st) + kStageA, brow[ni], (s), lane);              \
  } while (0)

  const int KT = K / EPR;
  MOE_ISSUE(0);
  if (KT > 1) MOE_ISSUE(1);
  if (KT > 2) MOE_ISSUE(2);
  if (KT > 2)
    asm volatile("s_waitcnt vmcnt(24)\n\ts_barrier" ::: "memory");
  else if (KT == 2)
    asm volatile("s_waitcnt vmcnt(12)\n\ts_barrier" ::: "memory");
  else
    asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
  MOE_LOADF(smem, 0, 0);
  for (int kt = 0; kt < KT; ++kt) {
    const char* st = smem + (kt % kStages) * kStage;
#pragma unroll
    for (int s = 0; s < S; ++s) {
      const int cur = s & 1, nxt = cur ^ 1;
      if (s + 1 < S) {
        MOE_LOADF(st, s + 1, nxt);
      } else if (kt + 1 < KT) {
        // Stage kt + 1 must have landed (only stage kt + 2 may still be in flight) and
        // every wave must be done reading stage kt before its slot is refilled.
        if (kt + 2 < KT)
          asm volatile("s_waitcnt vmcnt(12) lgkmcnt(0)\n\ts_barrier" ::: "memory");
        else
          asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
        if (kt + 3 < KT) MOE_ISSUE(kt + 3);
        MOE_LOADF(smem + ((kt + 1) % kStages) * kStage, 0, nxt);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int ni = 0; ni < 4; ++ni) {
        acc[0][ni] = Mfma<TE>::mma(fa[cur][0], fb[cur][ni], acc[0][ni]);
        acc[1][ni] = Mfma<TE>::mma(fa[cur][1], fb[cur][ni], acc[1][ni]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }
#undef MOE_LOADF
#undef MOE_ISSUE

  // Accumulator layout of a 32x32 tile: lane l, register r -> column (l % 32),
  // row 8 (r / 4) + 4 (l / 32) + (r % 4).
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int m = wm * 64 + mi * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
      if (m >= nrows) continue;
      const size_t orow = (size_t)(row0 + m) * N;
      if (MODE == 0) {
        TE* h = static_cast<TE*>(c_out);
#pragma unroll
        for (int nj = 0; nj < 2; ++nj) {
          const int n = n0 + wn * 64 + nj * 32 + (lane & 31);
          const float gv = acc[mi][nj][r], uv = acc[mi][nj + 2][r];
          store_h(h + orow + n, silu(gv) * uv);
        }
      } else {
        float* y = static_cast<float*>(c_out);
#pragma unroll
        for (int ni = 0; ni < 4; ++ni) {
          const int n = n0 + wn * 128 + ni * 32 + (lane & 31);
          y[orow + n] = acc[mi][ni][r];
        }
      }
    }
}

// m-tile plan: plan[0].group = number of m-tiles; plan[1 + i] = the i-th m-tile, groups in
// order, 128 rows each except a group's last; .pad holds the group's first m-tile.
__global__ __launch_bounds__(1024) void plan_kernel(const int32_t* __restrict__ offsets,
                                                    int G, PlanEntry* __restrict__ plan) {
  __shared__ int32_t scan[1024];
  const int g = threadIdx.x;
  int c = 0, m = 0;
  if (g < G) {
    c = offsets[g + 1] - offsets[g];
    m = (c + kBM - 1) / kBM;
  }
  scan[g] = m;
  __syncthreads();
  for (int o = 1; o < 1024; o <<= 1) {
    const int v = g >= o ? scan[g - o] : 0;
    __syncthreads();
    scan[g] += v;
    __syncthreads();
  }
  const int start = scan[g] - m;
  if (g == 1023) plan[0] = PlanEntry{scan[g], 0, 0, 0};
  if (g < G) {
    const int r0 = offsets[g];
    for (int i = 0; i < m; ++i)
      plan[1 + start + i] = PlanEntry{g, r0 + i * kBM, min(kBM, c - i * kBM), start};
  }
}

template <typename TE>
static hipError_t launch_typed(const TE* x, const int32_t* offsets, const int32_t* row_token,
                               const TE* wg, const TE* wu, const TE* wd, TE* h, float* y,
                               PlanEntry* plan, int T, int d, int I, int G, int R,
                               hipStream_t stream) {
  hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(1024), 0, stream, offsets, G, plan);
  const int64_t mtiles = max_mtiles(R, G);
  const int nt_gu = I / kGateUpBN;
  hipLaunchKernelGGL((grouped_gemm_kernel<TE, 0>), dim3(static_cast<uint32_t>(mtiles * nt_gu)),
                     dim3(256), 0, stream, x, row_token, wg, wu, offsets, plan,
                     static_cast<void*>(h), d, I, T, nt_gu);
  const int nt_dn = d / kDownBN;
  hipLaunchKernelGGL((grouped_gemm_kernel<TE, 1>), dim3(static_cast<uint32_t>(mtiles * nt_dn)),
                     dim3(256), 0, stream, static_cast<const TE*>(h), row_token, wd, wd,
                     offsets, plan, static_cast<void*>(y), I, d, T, nt_dn);
  return hipGetLastError();
}

hipError_t launch_grouped_swiglu(int dtype, const void* x, const int32_t* offsets,
                                 const int32_t* row_token, const void* w_gate,
                                 const void* w_up, const void* w_down, void* h,
                                 float* y_rows, PlanEntry* plan, int T, int d, int I, int G,
                                 int R, hipStream_t stream) {
  if (dtype == 1)
    return launch_typed<uint16_t>(
        static_cast<const uint16_t*>(x), offsets, row_token,
        static_cast<const uint16_t*>(w_gate), static_cast<const uint16_t*>(w_up),
        static_cast<const uint16_t*>(w_down), static_cast<uint16_t*>(h), y_rows, plan, T, d,
        I, G, R, stream);
  return launch_typed<float>(static_cast<const float*>(x), offsets, row_token,
                             static_cast<const float*>(w_gate),
                             static_cast<const float*>(w_up),
                             static_cast<const float*>(w_down), static_cast<float*>(h),
                             y_rows, plan, T, d, I, G, R, stream);
}

}  // namespace moe
