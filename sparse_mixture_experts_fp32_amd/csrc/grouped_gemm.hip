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
// Work decomposition: a device-built plan lists the m-tiles (128 rows of one group); the
// grid covers an upper bound of m-tiles x n-tiles and idle workgroups exit at once.
// Workgroup ids are remapped so that each XCD walks a contiguous range of tiles, n-tile
// fastest, so the gathered rows of one m-tile are reused from that XCD's L2.
//
// Tile: 128 rows x 256 B-rows (gate/up: 128 gate + 128 up; down: 256 outputs), K staged
// 128 bytes per row per step (64 bf16 / 32 f32) through double-buffered LDS (96 KB).
// LDS rows are 128 B; 16-byte chunk c of row r sits at slot c ^ (r & 7), so the eight
// lanes of a ds_read_b128 phase (eight rows, same chunk) hit eight different bank groups.
// Four waves in 2 x 2; each wave owns 64 rows x 128 B-rows = 2 x 4 MFMA 32x32 tiles.
#include "moe_device.h"
#include "moe_launch.h"

namespace moe {

constexpr int kRowBytes = 128;
constexpr int kBM = kGemmBM;            // 128
constexpr int kBRows = 256;
constexpr int kStageA = kBM * kRowBytes;      // 16 KB
constexpr int kStageB = kBRows * kRowBytes;   // 32 KB
constexpr int kStage = kStageA + kStageB;     // 48 KB

__device__ __forceinline__ int swz(int row, int chunk) {
  return row * kRowBytes + ((chunk ^ (row & 7)) << 4);
}

template <typename TE>
struct Mfma;

// bf16: v_mfma_f32_32x32x16_bf16.  Operand lane l: row/col (l % 32), K elements
// [8 (l / 32), 8 (l / 32) + 8) of the 16-wide step, i.e. 16-byte chunk (l / 32) of the
// step's 32 bytes.
template <>
struct Mfma<uint16_t> {
  static constexpr int kSteps = 4;  // 16-wide K steps per 64-element LDS row
  __device__ static inline bf16x8 frag(const char* base, int row, int s, int lane) {
    const int chunk = 2 * s + (lane >> 5);
    return *reinterpret_cast<const bf16x8*>(base + swz(row, chunk));
  }
  __device__ static inline f32x16 mma(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
};

// f32: v_mfma_f32_32x32x2_f32.  Operand lane l: row/col (l % 32), K element (l / 32) of
// the 2-wide step.
template <>
struct Mfma<float> {
  static constexpr int kSteps = 16;  // 2-wide K steps per 32-element LDS row
  __device__ static inline float frag(const char* base, int row, int s, int lane) {
    const int kk = 2 * s + (lane >> 5);
    return *reinterpret_cast<const float*>(base + swz(row, kk >> 2) + ((kk & 3) << 2));
  }
  __device__ static inline f32x16 mma(float a, float b, f32x16 c) {
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
    const PlanEntry* __restrict__ plan,     // plan[0].group = m-tile count
    void* __restrict__ c_out,               // MODE 0: h [R, N] (TE); MODE 1: y [R, N] f32
    int K, int N, int T, int NT) {
  constexpr int EPC = 16 / sizeof(TE);  // elements per 16-byte chunk
  constexpr int EPR = kRowBytes / sizeof(TE);
  __shared__ __attribute__((aligned(16))) char smem[2 * kStage];

  const uint32_t logical = xcd_remap(blockIdx.x, gridDim.x);
  const int mt = logical / NT, nt = logical % NT;
  if (mt >= plan[0].group) return;
  const PlanEntry pe = plan[1 + mt];
  const int g = pe.group, row0 = pe.row0, nrows = pe.nrows;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int n0 = nt * (MODE == 0 ? kGateUpBN : kDownBN);

  // Per-thread global sources: 4 A chunks and 8 B chunks of 16 bytes per K step.
  uint32_t a_off[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int cid = tid + 256 * i, row = cid >> 3, c = cid & 7;
    const int rr = min(row, nrows - 1);
    uint32_t base;
    if (MODE == 0) {
      int tok = row_token[row0 + rr];
      tok = min(max(tok, 0), T - 1);
      base = static_cast<uint32_t>(tok) * K;
    } else {
      base = static_cast<uint32_t>(row0 + rr) * K;
    }
    a_off[i] = base + c * EPC;
  }
  // gate/up: B-rows 0..127 are gate rows n0.., B-rows 128..255 the up rows n0..;
  // down: B-rows 0..255 are w_down rows n0..
  const TE* bg0 = b0 + ((size_t)g * N + n0) * K;
  const TE* bg1 = (MODE == 0) ? b1 + ((size_t)g * N + n0) * K : bg0;
  uint32_t b_off[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int cid = tid + 256 * i, row = cid >> 3, c = cid & 7;
    const int brow_src = (MODE == 0) ? (row & (kGateUpBN - 1)) : row;
    b_off[i] = static_cast<uint32_t>(brow_src) * K + c * EPC;
  }

  u32x4 ra[4], rb[8];
  // Global -> registers for K step k0 (issued early, consumed after the MFMAs).
#define MOE_LOAD(k0)                                                                   \
  do {                                                                                 \
    _Pragma("unroll") for (int i = 0; i < 4; ++i) ra[i] =                              \
        *reinterpret_cast<const u32x4*>(a_src + a_off[i] + (k0));                      \
    _Pragma("unroll") for (int i = 0; i < 8; ++i) rb[i] =                              \
        *reinterpret_cast<const u32x4*>((i < 4 ? bg0 : bg1) + b_off[i] + (k0));        \
  } while (0)
  // Registers -> one LDS stage (16-byte chunk cid -> row cid / 8, chunk cid % 8).
#define MOE_STORE(stage)                                                               \
  do {                                                                                 \
    char* sa_ = (stage);                                                               \
    char* sb_ = sa_ + kStageA;                                                         \
    _Pragma("unroll") for (int i = 0; i < 4; ++i) {                                    \
      const int cid = tid + 256 * i;                                                   \
      *reinterpret_cast<u32x4*>(sa_ + swz(cid >> 3, cid & 7)) = ra[i];                 \
    }                                                                                  \
    _Pragma("unroll") for (int i = 0; i < 8; ++i) {                                    \
      const int cid = tid + 256 * i;                                                   \
      *reinterpret_cast<u32x4*>(sb_ + swz(cid >> 3, cid & 7)) = rb[i];                 \
    }                                                                                  \
  } while (0)

  const int wm = wave & 1, wn = wave >> 1;
  // B-rows of this wave's four 32-wide n blocks.
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

  const int KT = K / EPR;
  char* const stage0 = smem;
  char* const stage1 = smem + kStage;
  MOE_LOAD(0);
  MOE_STORE(stage0);
  __syncthreads();
  for (int kt = 0; kt < KT; ++kt) {
    if (kt + 1 < KT) MOE_LOAD((kt + 1) * EPR);
    const char* sa = (kt & 1) ? stage1 : stage0;
    const char* sb = sa + kStageA;
#pragma unroll
    for (int s = 0; s < Mfma<TE>::kSteps; ++s) {
      auto a0 = Mfma<TE>::frag(sa, arow[0], s, lane);
      auto a1 = Mfma<TE>::frag(sa, arow[1], s, lane);
#pragma unroll
      for (int ni = 0; ni < 4; ++ni) {
        auto b = Mfma<TE>::frag(sb, brow[ni], s, lane);
        acc[0][ni] = Mfma<TE>::mma(a0, b, acc[0][ni]);
        acc[1][ni] = Mfma<TE>::mma(a1, b, acc[1][ni]);
      }
    }
    if (kt + 1 < KT) MOE_STORE((kt & 1) ? stage0 : stage1);
    __syncthreads();
  }

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

#undef MOE_LOAD
#undef MOE_STORE

// m-tile plan: plan[0].group = number of m-tiles; plan[1 + i] = the i-th m-tile, groups in
// order, 128 rows each except a group's last.
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
      plan[1 + start + i] = PlanEntry{g, r0 + i * kBM, min(kBM, c - i * kBM), 0};
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
                     dim3(256), 0, stream, x, row_token, wg, wu, plan,
                     static_cast<void*>(h), d, I, T, nt_gu);
  const int nt_dn = d / kDownBN;
  hipLaunchKernelGGL((grouped_gemm_kernel<TE, 1>), dim3(static_cast<uint32_t>(mtiles * nt_dn)),
                     dim3(256), 0, stream, static_cast<const TE*>(h), row_token, wd, wd, plan,
                     static_cast<void*>(y), I, d, T, nt_dn);
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
