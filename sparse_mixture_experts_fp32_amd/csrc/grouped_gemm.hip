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
// Three tilings share the grouped-row layout and the m-tile plan (below):
//   - 128 rows x 256 B-rows (grouped_gemm_kernel): f32 layers and bf16 layers whose
//     groups average fewer than 128 rows, with more than 32 tokens;
//   - 256 x 256 (grouped_gemm_wide_kernel): bf16 layers whose groups average 128 rows or
//     more;
//   - 32 x 128 with K split over four waves (grouped_gemm_skinny_kernel; 16 x 128 for
//     MXFP4 groups): bf16 layers of at most 32 tokens, where the step streams weights.
// Routed experts may hold MXFP4 weights (4-bit codes, one power-of-two scale per 32
// elements along K, the scales packed in records of 64 rows x 8 MX blocks); the 128-row
// and decode tilings expand them to bf16 on the way to the MFMAs.
//
// Work decomposition (128-row tiling).  A device-built plan lists the m-tiles (up to 128
// rows of one group).  Tiles are ordered group by group; inside a group in blocks of 4
// n-tiles, m-tile by m-tile, so the workgroups that run together on one XCD share a few
// weight slices (read from HBM once, then from L2) and a few sets of gathered rows.  The
// grid is persistent (one workgroup per CU); each XCD walks one contiguous range of tiles.
//
// Tile: 128 rows x 256 B-rows (gate/up: 128 gate + 128 up rows; down: 256 outputs).  K
// moves 128 bytes per row per step (64 bf16 / 32 f32).  Each step is fetched from global
// memory into registers two steps ahead (buffer_load_dwordx4), then written to one of two
// LDS buffers with ds_write_b128; on gfx950 this outruns direct buffer->LDS loads, whose
// LDS writes throttled the whole pipeline.  LDS rows are 128 B; 16-byte chunk c of row r
// sits at slot c ^ ((r / 2) % 8).  A wave writes each 1 KB block as 64 lanes x 16 B, so
// each lane fetches the global chunk that belongs at its slot.  Eight waves (two per
// SIMD, so one wave's MFMAs cover the other's waits) in 2 x 4; each owns 64 rows x 64
// B-rows as 2 x 2 MFMA 32x32 tiles.
#include "moe_device.h"
#include "moe_launch.h"

namespace moe {

constexpr int kBM = kGemmBM;                  // 128
constexpr int kBRows = 256;
constexpr int kStageA = kBM * kRowBytes;      // 16 KB
constexpr int kStageB = kBRows * kRowBytes;   // 32 KB
constexpr int kStage = kStageA + kStageB;     // 48 KB
constexpr int kStages = 2;                    // 96 KB of the CU's 160 KB
constexpr int kNB = 4;                        // n-tiles per scheduling block

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// A buffer offset that fails the range check of every A buffer the launchers build
// (each holds fewer than 2^31 bytes): such a lane's load returns zeros and makes no cache
// access.  Were a buffer larger, the offset would still lie inside it.
constexpr uint32_t kPastEnd = 0x80000000u;

// 16 bytes per lane from buffer offset voffset + soffset straight into LDS at
// lds_wave_base + 16 * lane (buffer_load_dwordx4 ... lds; counted by vmcnt).
template <int POLICY = kCached>
__device__ __forceinline__ void load_lds16(__amdgpu_buffer_rsrc_t rsrc, uint32_t voffset,
                                           uint32_t soffset, char* lds_wave_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_ptr_t)(lds_wave_base), 16, voffset,
                                           soffset, 0, POLICY);
}

// s_waitcnt immediate that waits for vmcnt <= n only (gfx9 encoding: vmcnt in bits 3:0
// and 15:14, expcnt 6:4, lgkmcnt 11:8).
constexpr int vmcnt_imm(int n) {
  return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8);
}

// MXFP4 (OCP Microscaling FP4) decode with gfx950's scaled conversion: one
// v_cvt_scalef32_pk_bf16_fp4 turns the two E2M1 codes of one byte (element 0 in the low
// nibble) into two bf16, multiplied by 2^(exponent field of the f32 scale operand - 127)
// and rounded to nearest even.  Only the scale's exponent field is read, so the E8M0 byte
// s is passed as the f32 bit pattern s << 23: s = 0 gives 2^-127 and s = 255 a NaN, as
// the E8M0 format defines.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ float mx_scale(uint32_t s) {
  return __uint_as_float((s & 0xffu) << 23);
}
// 8 codes (one 32-bit word, element i in bits 4i..4i+3) -> 8 bf16 (one 16-byte chunk,
// element i in halfword i).
__device__ __forceinline__ u32x4 mxfp4_chunk(uint32_t w, float sc) {
  u32x4 o;
  o[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 0));
  o[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 1));
  o[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 2));
  o[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 3));
  return o;
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

// The same from the hardware base-2 exponential and reciprocal (v_exp_f32, v_rcp_f32;
// each within about an ulp of f32): five instructions where expf and an IEEE division
// take about twenty-five.  The 256-row tiling evaluates 64 per lane per tile in an
// epilogue that stalls the whole workgroup, and rounds h to bf16 next (2^-8 relative),
// which a few f32 ulps change only when h lies at a rounding boundary (Inkling prefill
// grouped step 8.20 -> 8.13 ms; the 128-row tiling measured slower with it, 8.36 ->
// 8.45 ms at the Qwen3.8 shape, and keeps silu).  e^-z overflows to inf for z < -88
// (SiLU -> -0) and underflows to 0 for large z (SiLU -> z).
__device__ __forceinline__ float silu_hw(float z) {
  return z * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-z * 1.44269504088896341f));
}

__device__ __forceinline__ void store_h(uint16_t* p, float v) { *p = f32_to_bf16_rne(v); }
__device__ __forceinline__ void store_h(float* p, float v) { *p = v; }
// The same, non-temporal: the grouped GEMMs' outputs (h, Y_rows) are read once, by the
// next kernel, and stored with the default policy they take L2 lines from the weights and
// rows that the tiles running together share.
__device__ __forceinline__ void store_h_nt(uint16_t* p, float v) {
  __builtin_nontemporal_store(f32_to_bf16_rne(v), p);
}
__device__ __forceinline__ void store_h_nt(float* p, float v) {
  __builtin_nontemporal_store(v, p);
}

// MODE 0: gate/up + SwiGLU -> h.  MODE 1: down -> y_rows.
//
// Persistent: the grid has one workgroup per CU and workgroup p runs on XCD p % 8 (the
// dispatcher deals workgroups round-robin over the XCDs).  The tiles are split into 8
// contiguous ranges, one per XCD, and the XCD's 32 workgroups walk their range in
// phases of 32 consecutive tiles.  Tiles take equal time, so the tiles of a phase run in
// lockstep and the data they share (weight slices, gathered rows) is fetched into the
// XCD's L2 once.
template <typename TE, int MODE, bool FP4>
__global__ __launch_bounds__(512) void grouped_gemm_kernel(
    const TE* __restrict__ a_src,           // MODE 0: x [T, K]; MODE 1: h [R, K]
    const int32_t* __restrict__ row_token,  // MODE 0 only
    const TE* __restrict__ b0,              // MODE 0: w_gate [G, N, K]; MODE 1: w_down
    const TE* __restrict__ b1,              // MODE 0: w_up [G, N, K]
    const int32_t* __restrict__ offsets,    // [G + 1] group row offsets
    const PlanEntry* __restrict__ plan,     // plan[0].group = m-tile count
    void* __restrict__ c_out,               // MODE 0: h [R, N] (TE); MODE 1: y [R, N] f32
    uint32_t a_bytes,                       // bytes of a_src
    int K, int N, int T, int NT,
    int lda, int ldc,                       // row pitch (elements) of a_src and c_out
    // FP4: the E routed experts' B in MXFP4 (codes [E, N, K/2], packed scales;
    // MODE 0: q0/s0 gate, q1/s1 up; MODE 1: q0/s0 down); b0/b1 then hold only the shared
    // experts, expert g >= E at index g - E.
    const uint8_t* __restrict__ q0, const uint8_t* __restrict__ q1,
    const uint8_t* __restrict__ s0, const uint8_t* __restrict__ s1, int E) {
  constexpr int EPC = 16 / sizeof(TE);  // elements per 16-byte chunk
  __shared__ __attribute__((aligned(1024))) char smem[kStages * kStage];

  // Each XCD walks one contiguous range of the list.  (Dealing chunks of 32 tiles to the
  // XCDs in turn, as the 256-row tiling does, was slower here: 9.56 against 9.25 ms on
  // the Qwen3.8 shape, whose tiles cost about the same everywhere.)
  const uint32_t ntiles = static_cast<uint32_t>(plan[0].group) * NT;
  const uint32_t xcd = blockIdx.x % kXcds, per_xcd = gridDim.x / kXcds;
  const uint32_t q = ntiles / kXcds, r = ntiles % kXcds;
  const uint32_t lo = xcd * q + (xcd < r ? xcd : r);
  const uint32_t hi = lo + q + (xcd < r ? 1 : 0);

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  const int wm = wave & 1, wn = wave >> 1;   // 2 (rows) x 4 (columns) waves
  const int lrow = lane >> 3;
  // Lane l of LDS block b carries row 8 b + l / 8 and the logical chunk that the
  // swizzle places at physical slot l % 8 (depends on the parity of b).
  const int lchunk[2] = {(lane & 7) ^ ((lane >> 4) & 7),          // even blocks
                         (lane & 7) ^ ((4 + (lane >> 4)) & 7)};   // odd blocks
  // B-rows of this wave's two 32-wide n blocks: gate/up -> one gate block and the up
  // block of the same h columns; down -> two adjacent output blocks.
  int brow[2];
#pragma unroll
  for (int ni = 0; ni < 2; ++ni) {
    if (MODE == 0)
      brow[ni] = ni * kGateUpBN + wn * 32 + (lane & 31);
    else
      brow[ni] = wn * 64 + ni * 32 + (lane & 31);
  }
  int arow[2];
#pragma unroll
  for (int mi = 0; mi < 2; ++mi) arow[mi] = wm * 64 + mi * 32 + (lane & 31);
  const __amdgpu_buffer_rsrc_t a_rsrc = buffer_rsrc(a_src, a_bytes);
  const int KT = K * static_cast<int>(sizeof(TE)) / kRowBytes;

  for (uint32_t logical = lo + blockIdx.x / kXcds; logical < hi; logical += per_xcd) {
    // ---- the tile
    const PlanEntry first = plan[1 + logical / NT];
    const int g = first.group, gmt0 = first.pad;
    const int mg = (offsets[g + 1] - offsets[g] + kBM - 1) / kBM;  // m-tiles of the group
    // Inside a group: blocks of kNB n-tiles; within a block, m-tile by m-tile with the
    // n-tiles fastest, so one phase covers up to 8 m-tiles x 4 n-tiles.
    const uint32_t local = logical - static_cast<uint32_t>(gmt0) * NT;
    const int full = NT / kNB;
    int mloc, nt;
    if (local < static_cast<uint32_t>(full * mg * kNB)) {
      const int blk = local / (mg * kNB), rr = local % (mg * kNB);
      mloc = rr / kNB;
      nt = blk * kNB + rr % kNB;
    } else {
      const int rem = NT - full * kNB, rr = local - full * mg * kNB;
      mloc = rr / rem;
      nt = full * kNB + rr % rem;
    }
    const PlanEntry pe = plan[1 + gmt0 + mloc];
    const int row0 = pe.row0, nrows = pe.nrows;
    const int n0 = nt * (MODE == 0 ? kGateUpBN : kDownBN);

    // ---- per-lane sources (byte offsets).  Wave w fills A blocks 2w, 2w+1 and B blocks
    // 4w..4w+3 of each stage (a block = 1 KB = 8 rows).
    uint32_t a_off[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int row = 8 * (2 * wave + i) + lrow;
      const int rr = min(row, nrows - 1);
      uint32_t base;
      if (MODE == 0) {
        int tok = row_token[row0 + rr];
        tok = min(max(tok, 0), T - 1);
        base = static_cast<uint32_t>(tok) * lda;
      } else {
        base = static_cast<uint32_t>(row0 + rr) * lda;
      }
      // Rows past the m-tile: an offset past the buffer (zeros, no L1 lookup); their
      // output rows are not stored.
      a_off[i] = row < nrows ? (base + lchunk[i & 1] * EPC) * sizeof(TE) : kPastEnd;
    }
    // gate/up: B-rows 0..127 (waves 0..3) are gate rows n0.., B-rows 128..255 (waves
    // 4..7) the up rows n0..;  down: B-rows 0..255 are w_down rows n0..
    const bool quant = FP4 && g < E;          // tile-uniform
    const int gb = FP4 ? (quant ? 0 : g - E) : g;   // index into b0 / b1 (dense tiles)
    const TE* bsrc;
    int brow0;
    if (MODE == 0) {
      bsrc = (wv < 4 ? b0 : b1) + ((size_t)gb * N + n0) * K;
      brow0 = 32 * (wv & 3);
    } else {
      bsrc = b0 + ((size_t)gb * N + n0) * K;
      brow0 = 32 * wv;
    }
    const __amdgpu_buffer_rsrc_t b_rsrc =
        buffer_rsrc(bsrc, static_cast<uint32_t>((MODE == 0 ? kGateUpBN : kDownBN) * K *
                                                sizeof(TE)));
    uint32_t b_off[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      b_off[i] = (static_cast<uint32_t>(brow0 + 8 * i + lrow) * K + lchunk[i & 1] * EPC) *
                 sizeof(TE);

    f32x16 acc[2][2];
#pragma unroll
    for (int mi = 0; mi < 2; ++mi)
#pragma unroll
      for (int ni = 0; ni < 2; ++ni) acc[mi][ni] = f32x16{};

    // Global -> registers for K step kt into register set P (6 x 16 bytes per lane), and
    // registers -> LDS slot kt % 2.  Wave w owns 1 KB blocks of each stage; lane l writes
    // bytes [16 l, 16 l + 16) of a block, which the swizzle maps to row 8 b + l / 8.
    u32x4 ra[2][2], rb[2][4];
#define MOE_FETCH(kt, P)                                                                \
  do {                                                                                  \
    const uint32_t k0_ = (kt) * kRowBytes;                                              \
    _Pragma("unroll") for (int i = 0; i < 2; ++i)                                       \
        ra[P][i] = load16(a_rsrc, a_off[i], k0_);                                       \
    _Pragma("unroll") for (int i = 0; i < 4; ++i)                                       \
        rb[P][i] = load16<kStream>(b_rsrc, b_off[i], k0_);                              \
  } while (0)
#define MOE_STORE(kt, P)                                                                \
  do {                                                                                  \
    char* st_ = smem + ((kt) % kStages) * kStage + lane * 16;                           \
    _Pragma("unroll") for (int i = 0; i < 2; ++i)                                       \
        *reinterpret_cast<u32x4*>(st_ + (2 * wv + i) * 1024) = ra[P][i];                \
    _Pragma("unroll") for (int i = 0; i < 4; ++i)                                       \
        *reinterpret_cast<u32x4*>(st_ + kStageA + (4 * wv + i) * 1024) = rb[P][i];      \
  } while (0)

    // Fragments of one 16-wide (bf16) / 2-wide (f32) K step, double-buffered so the LDS
    // reads of step s + 1 are in flight while the MFMAs of step s run.
    typedef typename Mfma<TE>::frag_t frag_t;
    constexpr int S = Mfma<TE>::kSteps;
    frag_t fa[2][2], fb[2][2];
#define MOE_LOADF(st, s, buf)                                                           \
  do {                                                                                  \
    fa[buf][0] = Mfma<TE>::frag((st), arow[0], (s), lane);                              \
    fa[buf][1] = Mfma<TE>::frag((st), arow[1], (s), lane);                              \
    _Pragma("unroll") for (int ni = 0; ni < 2; ++ni)                                    \
        fb[buf][ni] = Mfma<TE>::frag((st) + kStageA, brow[ni], (s), lane);              \
  } while (0)

    // One K step kt (register set and LDS slot P = kt % 2): fetch step kt + 2 into the
    // registers step kt vacated, run the MFMAs of step kt from LDS, and before the last
    // MFMA group store step kt + 1 (fetched one step earlier) into the other slot.
    // The barrier makes step kt + 1 visible and retires every read of step kt.  The
    // fetch is unconditional (the last two steps re-fetch step KT - 1 and drop it) so
    // that the compiler's wait before each store counts exactly the younger fetch.
#define MOE_STEP(kt, P, NEXT)                                                           \
  do {                                                                                  \
    MOE_FETCH(min((kt) + 2, KT - 1), P);                                                \
    const char* st = smem + (P) * kStage;                                               \
    _Pragma("unroll") for (int s = 0; s < S; ++s) {                                     \
      const int cur = s & 1, nxt = cur ^ 1;                                             \
      if (s + 1 < S) {                                                                  \
        MOE_LOADF(st, s + 1, nxt);                                                      \
      } else if (NEXT) {                                                                \
        MOE_STORE((kt) + 1, (P) ^ 1);                                                   \
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");                 \
        MOE_LOADF(smem + ((P) ^ 1) * kStage, 0, nxt);                                   \
      }                                                                                 \
      __builtin_amdgcn_sched_barrier(0);                                                \
      _Pragma("unroll") for (int ni = 0; ni < 2; ++ni) {                                \
        acc[0][ni] = Mfma<TE>::mma(fa[cur][0], fb[cur][ni], acc[0][ni]);                \
        acc[1][ni] = Mfma<TE>::mma(fa[cur][1], fb[cur][ni], acc[1][ni]);                \
      }                                                                                 \
      __builtin_amdgcn_sched_barrier(0);                                                \
    }                                                                                   \
  } while (0)

    if (FP4 && quant) {
      // MXFP4 B: thread t stages B-row t / 2, elements 32 (t % 2) .. +32 of the 64-wide K
      // step = one MX block: 16 bytes of codes and its scale byte, dequantized to bf16
      // (exact in the normal range: 2 significant bits times a power of two) on the
      // way into LDS chunks 4 (t % 2) .. +3 of that row.
      const int qrow = tid >> 1, qhalf = tid & 1;
      const int qlocal = MODE == 0 ? (qrow & (kGateUpBN - 1)) : qrow;
      const uint8_t* qsrc = MODE == 0 ? (wv < 4 ? q0 : q1) : q0;
      const uint8_t* ssrc = MODE == 0 ? (wv < 4 ? s0 : s1) : s0;
      const int qrows = MODE == 0 ? kGateUpBN : kDownBN;
      const __amdgpu_buffer_rsrc_t q_rsrc = buffer_rsrc(
          qsrc + ((size_t)g * N + n0) * (K / 2), static_cast<uint32_t>(qrows * (K / 2)));
      // Packed scales (records of 64 rows x 8 MX blocks): MX block 2 kt + qhalf of tile
      // row qlocal is byte 2 (kt % 4) + qhalf of its row in record kt / 4.
      const int KR = static_cast<int>(mx_rec_k(K));
      const __amdgpu_buffer_rsrc_t s_rsrc = buffer_rsrc(
          ssrc + ((size_t)g * N + n0) / kMxRecRows * KR * kMxRecBytes,
          static_cast<uint32_t>(qrows / kMxRecRows * KR * kMxRecBytes));
      const uint32_t q_off = static_cast<uint32_t>(qlocal) * (K / 2) + qhalf * 16;
      const uint32_t s_off = static_cast<uint32_t>(qlocal / kMxRecRows) * KR * kMxRecBytes +
                             static_cast<uint32_t>(qlocal % kMxRecRows) * kMxRecBlocks + qhalf;
      u32x4 rq[2];
      uint32_t rs[2];
#define MOE_FETCHQ(kt, P)                                                               \
  do {                                                                                  \
    const uint32_t k0_ = (kt) * kRowBytes;                                              \
    _Pragma("unroll") for (int i = 0; i < 2; ++i)                                       \
        ra[P][i] = load16(a_rsrc, a_off[i], k0_);                                       \
    rq[P] = load16<kStream>(q_rsrc, q_off, (kt) * 32);                                  \
    rs[P] = __builtin_amdgcn_raw_buffer_load_b8(                                        \
        s_rsrc, s_off, ((kt) >> 2) * kMxRecBytes + 2 * ((kt) & 3), 0);                  \
  } while (0)
#define MOE_STOREQ(kt, P)                                                               \
  do {                                                                                  \
    char* st_ = smem + ((kt) % kStages) * kStage;                                       \
    _Pragma("unroll") for (int i = 0; i < 2; ++i)                                       \
        *reinterpret_cast<u32x4*>(st_ + lane * 16 + (2 * wv + i) * 1024) = ra[P][i];    \
    const float sc_ = mx_scale(rs[P]);                                                  \
    _Pragma("unroll") for (int j = 0; j < 4; ++j)                                       \
        *reinterpret_cast<u32x4*>(st_ + kStageA + swz(qrow, 4 * qhalf + j)) =           \
            mxfp4_chunk(rq[P][j], sc_);                                                 \
  } while (0)
#define MOE_STEPQ(kt, P, NEXT)                                                          \
  do {                                                                                  \
    MOE_FETCHQ(min((kt) + 2, KT - 1), P);                                               \
    const char* st = smem + (P) * kStage;                                               \
    _Pragma("unroll") for (int s = 0; s < S; ++s) {                                     \
      const int cur = s & 1, nxt = cur ^ 1;                                             \
      if (s + 1 < S) {                                                                  \
        MOE_LOADF(st, s + 1, nxt);                                                      \
      } else if (NEXT) {                                                                \
        MOE_STOREQ((kt) + 1, (P) ^ 1);                                                  \
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");                 \
        MOE_LOADF(smem + ((P) ^ 1) * kStage, 0, nxt);                                   \
      }                                                                                 \
      __builtin_amdgcn_sched_barrier(0);                                                \
      _Pragma("unroll") for (int ni = 0; ni < 2; ++ni) {                                \
        acc[0][ni] = Mfma<TE>::mma(fa[cur][0], fb[cur][ni], acc[0][ni]);                \
        acc[1][ni] = Mfma<TE>::mma(fa[cur][1], fb[cur][ni], acc[1][ni]);                \
      }                                                                                 \
      __builtin_amdgcn_sched_barrier(0);                                                \
    }                                                                                   \
  } while (0)
      MOE_FETCHQ(0, 0);
      MOE_FETCHQ(1, 1);
      MOE_STOREQ(0, 0);
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
      MOE_LOADF(smem, 0, 0);
      int kt = 0;
      for (; kt + 2 < KT; kt += 2) {
        MOE_STEPQ(kt, 0, 1);
        MOE_STEPQ(kt + 1, 1, 1);
      }
      MOE_STEPQ(kt, 0, 1);
      MOE_STEPQ(kt + 1, 1, 0);
#undef MOE_STEPQ
#undef MOE_STOREQ
#undef MOE_FETCHQ
    } else {
    // KT is even: d and I are multiples of 256 and 128 elements, i.e. of 2 K steps.  The
    // last step (NEXT = 0) is peeled off the loop so that no control-flow join sits
    // between a fragment load and the MFMAs that do not depend on it (the waitcnt pass
    // would wait for every outstanding load at a join).
    MOE_FETCH(0, 0);
    MOE_FETCH(1, 1);
    MOE_STORE(0, 0);
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    MOE_LOADF(smem, 0, 0);
    int kt = 0;
    for (; kt + 2 < KT; kt += 2) {
      MOE_STEP(kt, 0, 1);
      MOE_STEP(kt + 1, 1, 1);
    }
    MOE_STEP(kt, 0, 1);
    MOE_STEP(kt + 1, 1, 0);
    }
#undef MOE_STEP
#undef MOE_LOADF
#undef MOE_STORE
#undef MOE_FETCH
    // Every wave has finished reading the ring before the next tile refills it.
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");

    // Accumulator layout of a 32x32 tile: lane l, register r -> column (l % 32),
    // row 8 (r / 4) + 4 (l / 32) + (r % 4).
#pragma unroll
    for (int mi = 0; mi < 2; ++mi)
#pragma unroll
      for (int rg = 0; rg < 16; ++rg) {
        const int m = wm * 64 + mi * 32 + 8 * (rg >> 2) + 4 * (lane >> 5) + (rg & 3);
        if (m >= nrows) continue;
        const size_t orow = (size_t)(row0 + m) * ldc;
        if (MODE == 0) {
          TE* h = static_cast<TE*>(c_out);
          const int n = n0 + wn * 32 + (lane & 31);
          store_h_nt(h + orow + n, silu(acc[mi][0][rg]) * acc[mi][1][rg]);
        } else {
          float* y = static_cast<float*>(c_out);
#pragma unroll
          for (int ni = 0; ni < 2; ++ni) {
            const int n = n0 + wn * 64 + ni * 32 + (lane & 31);
            store_h_nt(y + orow + n, acc[mi][ni][rg]);
          }
        }
      }
  }
}

// ---- Decode-shaped tiles (bf16 layers with at most 32 tokens)
//
// Every group then has at most 32 rows, so one 32-row m-tile per bf16 group (MXFP4 groups
// take 16-row m-tiles, below), and the step is bound by streaming the experts' weights.
// A tile is 32 (16) rows x 128 B-rows (gate/up: 64
// gate + 64 up rows of the same h columns; down: 128 output columns); the 4 waves of a
// workgroup split its K range into interleaved chunks, double-buffered in registers one
// chunk ahead, and the K loop's only barrier is at its last chunk (below).  Weights are
// loaded coalesced (8 lanes x 16 bytes cover a 128-byte line of one B-row, so the L1
// sends whole-line requests and does one tag lookup per 64 bytes) and pass through the
// wave's own 16 KB of LDS to the MFMA operand layout; A goes straight into registers in
// the operand layout.  The K order inside a chunk is permuted (the product sums over K,
// so any order shared by A and B is exact) so that an A load is 16 contiguous bytes and
// an MXFP4 operand is one MX block (16 bytes of codes, one scale byte).  MXFP4 codes are
// converted to bf16 in registers.  Rows past the group's end load a copy of its last row
// (their outputs are not stored).  The 4 waves' partial sums are added in LDS in wave
// order (of 32-row tiles only the row quads that hold rows of the group), then the SwiGLU
// (gate/up) or the f32 row store (down) runs.  Tiles are taken last plan m-tile first, so
// the shared experts' bf16 tiles (about 4x the bytes of an MXFP4 tile) start before the
// routed ones: a workgroup's first tile is its index, later ones come from a counter.  A
// workgroup takes its next tile from the counter during its current tile's last chunks
// and fetches the next tile's first chunk (pair), and the row index of its A rows, while
// the last MFMAs and the epilogue run.
constexpr int kSkBM = 32;                 // rows per m-tile (bf16 groups)
constexpr int kSkBM16 = 16;               // rows per m-tile of MXFP4 groups
constexpr int kSkWaves = 4;               // waves per workgroup (K split)
constexpr int kSkBlocks = 4;              // 32-wide B-row blocks per tile (128 B-rows)

// One m-tile of the decode tiling: group, first grouped row, rows, and the first B-row of
// each source (gate/up: 64 gate + 64 up rows; down: 128 rows).
struct SkTile {
  int g, row0, nrows, n0;
};

template <int MODE>
__device__ __forceinline__ SkTile sk_tile(const PlanEntry* __restrict__ plan, uint32_t logical,
                                          int NT) {
  const PlanEntry pe = plan[1 + logical / NT];
  return SkTile{pe.group, pe.row0, pe.nrows,
                static_cast<int>(logical % NT) * (MODE == 0 ? 64 : 128)};
}

// The A row of lane ln (MODE 0: its token, MODE 1: its grouped row); lanes past the
// group's rows read its last row (an MFMA output row depends only on its own A row, and
// those rows are not stored).
template <int MODE>
__device__ __forceinline__ int sk_a_src(const int32_t* __restrict__ row_token,
                                        const SkTile& tl, int ln) {
  const int lr = min(ln, tl.nrows - 1);
  return MODE == 0 ? row_token[tl.row0 + lr] : tl.row0 + lr;
}

// Byte offset of that row.
template <int MODE>
__device__ __forceinline__ uint32_t sk_a_off(int src, int T, int lda) {
  if (MODE == 0) src = min(max(src, 0), T - 1);
  return static_cast<uint32_t>(src) * lda * 2;
}

struct SkQSrc {   // MXFP4 codes and packed scales of a tile (gate/up: gate, up)
  __amdgpu_buffer_rsrc_t q0, q1, s0, s1;
};
struct SkBSrc {   // bf16 weights of a tile (gate/up: gate, up)
  __amdgpu_buffer_rsrc_t b0, b1;
};

template <int MODE, bool FP4>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2)))
void grouped_gemm_skinny_kernel(
    const uint16_t* __restrict__ a_src,      // MODE 0: x [T, K]; MODE 1: h [R, K]
    const int32_t* __restrict__ row_token,   // MODE 0 only
    const uint16_t* __restrict__ b0,         // bf16 B: MODE 0 gate, MODE 1 down [., N, K]
    const uint16_t* __restrict__ b1,         // bf16 B: MODE 0 up
    const uint8_t* __restrict__ q0, const uint8_t* __restrict__ q1,   // MXFP4 codes
    const uint8_t* __restrict__ s0, const uint8_t* __restrict__ s1,   // packed E8M0 scales
    const PlanEntry* __restrict__ plan, uint32_t* __restrict__ next_tile,
    void* __restrict__ c_out, uint32_t a_bytes, int K, int N, int T, int NT, int lda,
    int ldc, int E) {
  // FP4: groups g < E are MXFP4 (codes [E, N, K/2], packed scales) and groups
  // g >= E bf16 at index g - E of b0 / b1; otherwise every group is bf16 at index g.
  __shared__ float red[kSkWaves * kSkBlocks * 16 * 64];   // 64 KB of partial sums
  __shared__ uint32_t s_tile[2];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ln = lane & 31, lh = lane >> 5;
  const uint32_t ntiles = static_cast<uint32_t>(plan[0].group) * NT;
  const __amdgpu_buffer_rsrc_t a_rsrc = buffer_rsrc(a_src, a_bytes);
  constexpr int kRowsPerSrc = MODE == 0 ? 64 : 128;   // B-rows of one source per tile

  // MXFP4 B: chunks of 128 K elements (64 code bytes and 4 scale bytes per B-row).  Wave
  // w takes the chunk pairs 8 p + 2 w, 8 p + 2 w + 1 (one 128-byte line of codes and 8
  // scale bytes per B-row); iteration i of a wave is chunk 8 (i / 2) + 2 w + i % 2.  The
  // MXFP4 tiles hold 16 rows and run on v_mfma_f32_16x16x32_bf16 (below); their operand
  // layout gives lane 16 g + r MX block g of the chunk (16 code bytes) of B-row r of each
  // 16-row column block.  The record of 64 B-rows x 8 MX blocks that holds the scales of
  // chunk pair p of the tile's 64-row block s sits at (s * KR + p) * 512 from the tile's
  // scale base.
  const int nchq = K / 128;
  const int KR = static_cast<int>(mx_rec_k(K));
  const uint32_t qbytes = static_cast<uint32_t>(kRowsPerSrc * (K / 2));
  const uint32_t sbytes = static_cast<uint32_t>(kRowsPerSrc / kMxRecRows * KR * kMxRecBytes);
  // bf16 B: chunks of 64 K elements (128 bytes per B-row), wave w: chunks w, w + 4, ...
  // MFMA step u, operand half hh covers K elements 32 hh + 8 u .. +8 of the chunk
  // (16-byte slot 4 hh + u of the row) for A and B alike.
  const int nchb = K / 64;
  const uint32_t bbytes = static_cast<uint32_t>(kRowsPerSrc * K * 2);
  // Weights are loaded coalesced: load q brings tile rows 8 q + lane / 8 (gate/up: rows
  // 0..63 of the gate source for q < 8, of the up source for q >= 8), 16 bytes
  // (lane % 8) of the chunk's (bf16) or chunk pair's (MXFP4) 128, and goes through this
  // wave's 16 KB of LDS (its partial-sum area) to the MFMA layout, the 16-byte slot
  // swizzled by (row / 2) % 8.
  const uint32_t cq_voff = static_cast<uint32_t>(lane >> 3) * (K / 2) + 16 * (lane & 7);
  const uint32_t cb_voff = static_cast<uint32_t>(lane >> 3) * K * 2 + 16 * (lane & 7);
  // Scales: one 8-byte load per 64 B-rows, lane l taking B-row l of the record; a lane
  // swap then gives every lane the bytes of its B-rows ln and ln + 32.
  const uint32_t s_voff = static_cast<uint32_t>(lane) * kMxRecBlocks;
  char* stg = reinterpret_cast<char*>(red) + wv * (kSkBlocks * 16 * 64 * 4);
  uint32_t w_off[2];
#pragma unroll
  for (int e = 0; e < 2; ++e)
    w_off[e] = 128 * (lane >> 3) + 16 * ((lane & 7) ^ ((4 * e + (lane >> 4)) & 7));

  auto q_src = [&](const SkTile& tl) {
    const size_t qbase = ((size_t)tl.g * N + tl.n0) * (K / 2);
    const size_t sbase = ((size_t)tl.g * N + tl.n0) / kMxRecRows * KR * kMxRecBytes;
    return SkQSrc{buffer_rsrc(q0 + qbase, qbytes),
                  buffer_rsrc((MODE == 0 ? q1 : q0) + qbase, qbytes),
                  buffer_rsrc(s0 + sbase, sbytes),
                  buffer_rsrc((MODE == 0 ? s1 : s0) + sbase, sbytes)};
  };
  auto b_src = [&](const SkTile& tl) {
    const size_t bbase = ((size_t)(FP4 ? tl.g - E : tl.g) * N + tl.n0) * K;
    return SkBSrc{buffer_rsrc(b0 + bbase, bbytes),
                  buffer_rsrc((MODE == 0 ? b1 : b0) + bbase, bbytes)};
  };

  // Operand registers, double-buffered by chunk.  A tile's first chunk (pair) is fetched
  // during the previous tile's last one (below), so the registers of its buffer 0 carry
  // over from one tile to the next.
  u32x4 qa[2][4], qc[16];      // MXFP4: A of a chunk (16 rows), codes of a chunk pair
  u32x2 qs[kSkBlocks / 2];     // MXFP4: scale bytes of a chunk pair, B-row lane of a record
  u32x4 ba[2][4], bc[2][16];   // bf16: A and B of a chunk

  // B-row of this lane in block b, relative to its source's tile base: ln + bro(b).
  // Gate/up blocks 0, 1 are gate rows and 2, 3 the up rows of the same columns.
#define MOE_SK_BRO(b) (MODE == 0 ? 32 * ((b) & 1) : 32 * (b))
#define MOE_SKQ_CHUNK(i) (8 * ((i) >> 1) + 2 * wv + ((i) & 1))
  // Codes and scales of the chunk pair that starts at iteration i (even), from SRC.
#define MOE_SKQ_CODES(i, SRC)                                                           \
  do {                                                                                  \
    const uint32_t c_ = static_cast<uint32_t>(min(MOE_SKQ_CHUNK(i), nchq - 1));         \
    _Pragma("unroll") for (int q = 0; q < 16; ++q)                                      \
        qc[q] = load16<kStream>((MODE == 0 && q >= 8) ? (SRC).q1 : (SRC).q0, cq_voff,   \
                                8 * (MODE == 0 ? (q & 7) : q) * (K / 2) + c_ * 64);     \
    _Pragma("unroll") for (int r = 0; r < kSkBlocks / 2; ++r)                           \
        qs[r] = __builtin_amdgcn_raw_buffer_load_b64(                                   \
            (MODE == 0 && r == 1) ? (SRC).s1 : (SRC).s0, s_voff,                        \
            ((MOE_SK_BRO(2 * r) >> 6) * KR + (c_ >> 1)) * kMxRecBytes, 0);              \
  } while (0)
  // MXFP4 tiles hold 16 rows (the plan cuts MXFP4 groups into 16-row m-tiles: a decode
  // group holds a few rows, so 32-row tiles spent half their A loads and MFMAs on
  // padding) and run on v_mfma_f32_16x16x32_bf16.  Lane l = 16 g + r takes A row r, B-row
  // r of each 16-row column block cb (tile B-row 16 cb + r) and MX block g of the chunk:
  // MFMA step u covers K elements 32 g + 8 u .. +8 of the chunk for A and B alike (exact:
  // the product sums over K).  The output of block cb in lane l is column 16 cb + r, rows
  // 4 g .. +4.
  // A of iteration i into qa[P], rows at AV.
#define MOE_SKQ16_ROWS(i, P, AV)                                                        \
  do {                                                                                  \
    const uint32_t c_ = static_cast<uint32_t>(min(MOE_SKQ_CHUNK(i), nchq - 1));         \
    _Pragma("unroll") for (int u = 0; u < 4; ++u)                                       \
        qa[P][u] = load16(a_rsrc, (AV), c_ * 256 + 16 * u);                             \
  } while (0)
  // The scale byte of column block cb's B-row in MX block 4 P + g comes from the lane of
  // its record that loaded that B-row (ds_bpermute); chunk 1's bytes are kept packed in
  // rsp past the next pair's fetch.  Column blocks 0..3 / 4..7 are records 0 / 1.
#define MOE_SKQ16_MMA(i, P)                                                             \
  do {                                                                                  \
    if (MOE_SKQ_CHUNK(i) < nchq) {                                                      \
      uint32_t sb_[8];                                                                  \
      if ((P) == 0) {                                                                   \
        _Pragma("unroll") for (int q = 0; q < 16; ++q)                                  \
            *reinterpret_cast<u32x4*>(stg + 1024 * q + w_off[q & 1]) = qc[q];           \
        rsp[0] = 0u;                                                                    \
        rsp[1] = 0u;                                                                    \
        _Pragma("unroll") for (int cb = 0; cb < 8; ++cb) {                              \
          const int src_ = (16 * (cb & 3) + r16) << 2;                                  \
          const uint32_t w0_ = static_cast<uint32_t>(__builtin_amdgcn_ds_bpermute(      \
              src_, static_cast<int>(qs[cb >> 2][0])));                                 \
          const uint32_t w1_ = static_cast<uint32_t>(__builtin_amdgcn_ds_bpermute(      \
              src_, static_cast<int>(qs[cb >> 2][1])));                                 \
          sb_[cb] = (w0_ >> (8 * g16)) & 0xffu;                                         \
          rsp[cb >> 2] |= ((w1_ >> (8 * g16)) & 0xffu) << (8 * (cb & 3));               \
        }                                                                               \
      } else {                                                                          \
        _Pragma("unroll") for (int cb = 0; cb < 8; ++cb)                                \
            sb_[cb] = (rsp[cb >> 2] >> (8 * (cb & 3))) & 0xffu;                         \
      }                                                                                 \
      _Pragma("unroll") for (int h_ = 0; h_ < 2; ++h_) {                                \
        u32x4 cq_[4];                                                                   \
        float sc_[4];                                                                   \
        _Pragma("unroll") for (int c = 0; c < 4; ++c) {                                 \
          cq_[c] = *reinterpret_cast<const u32x4*>(stg + lq16[P] + 2048 * (4 * h_ + c));\
          sc_[c] = mx_scale(sb_[4 * h_ + c]);                                           \
        }                                                                               \
        _Pragma("unroll") for (int u = 0; u < 4; ++u) {                                 \
          __builtin_amdgcn_sched_barrier(0);                                            \
          _Pragma("unroll") for (int c = 0; c < 4; ++c) {                               \
            const bf16x8 fb_ =                                                          \
                __builtin_bit_cast(bf16x8, mxfp4_chunk(cq_[c][u], sc_[c]));             \
            acc16[4 * h_ + c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(                \
                __builtin_bit_cast(bf16x8, qa[P][u]), fb_, acc16[4 * h_ + c], 0, 0, 0); \
          }                                                                             \
        }                                                                               \
        __builtin_amdgcn_sched_barrier(0);                                              \
      }                                                                                 \
    }                                                                                   \
  } while (0)
  // B of chunk wv + 4 i into bc[P], from SRC; A of that chunk into ba[P], rows at AV.
#define MOE_SKB_CODES(i, P, SRC)                                                        \
  do {                                                                                  \
    const uint32_t c_ = static_cast<uint32_t>(min(wv + kSkWaves * (i), nchb - 1));      \
    _Pragma("unroll") for (int q = 0; q < 16; ++q)                                      \
        bc[P][q] = load16<kStream>((MODE == 0 && q >= 8) ? (SRC).b1 : (SRC).b0,         \
                                   cb_voff,                                             \
                                   8 * (MODE == 0 ? (q & 7) : q) * K * 2 + c_ * 128);   \
  } while (0)
#define MOE_SKB_ROWS(i, P, AV)                                                          \
  do {                                                                                  \
    const uint32_t c_ = static_cast<uint32_t>(min(wv + kSkWaves * (i), nchb - 1));      \
    _Pragma("unroll") for (int u = 0; u < 4; ++u)                                       \
        ba[P][u] = load16(a_rsrc, (AV), c_ * 128 + 16 * u);                             \
  } while (0)
#define MOE_SKB_MMA(i, P)                                                               \
  do {                                                                                  \
    if (wv + kSkWaves * (i) < nchb) {                                                   \
      _Pragma("unroll") for (int q = 0; q < 16; ++q)                                    \
          *reinterpret_cast<u32x4*>(stg + 1024 * q + w_off[q & 1]) = bc[P][q];          \
      _Pragma("unroll") for (int u = 0; u < 4; ++u) {                                   \
        const bf16x8 fa_ = __builtin_bit_cast(bf16x8, ba[P][u]);                        \
        _Pragma("unroll") for (int b = 0; b < kSkBlocks; ++b)                           \
            acc[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(                           \
                fa_,                                                                    \
                *reinterpret_cast<const bf16x8*>(                                       \
                    stg + 4096 * b + 128 * ln + 16 * ((4 * lh + u) ^ ((ln >> 1) & 7))), \
                acc[b], 0, 0, 0);                                                       \
      }                                                                                 \
    }                                                                                   \
  } while (0)
  // The next tile: lane 0 of wave 0 takes it from the counter one chunk pair (MXFP4) or
  // chunk (bf16) before this tile's last, and publishes it at the last one, so the wait
  // for the counter and the first loads of the next tile overlap this tile's last MFMAs
  // and its epilogue.  The slot alternates between tiles: the one written here was last
  // read two tiles ago, before several barriers.
#define MOE_SK_PUBLISH()                                                                \
  do {                                                                                  \
    if (tid == 0) s_tile[par ^ 1] = nxt;                                                \
    __syncthreads();                                                                    \
    tn = __builtin_amdgcn_readfirstlane(s_tile[par ^ 1]);                               \
  } while (0)

  // Sums of the four waves' partials and the tile's output, plus the next tile's first A
  // rows (ROWS) at n_aoff, from the row index n_src loaded before that tile's first
  // weights: a wave's loads complete in issue order, so waiting here for that index does
  // not wait for the weights, as a row_token lookup issued here would.  Partial sums ->
  // LDS in quads of accumulator registers ([wave][block][quad][lane], 16 bytes per lane),
  // then each wave adds the four waves' partials of its share in wave order.  Accumulator
  // layout: lane l, register 4 q + j -> B-row (l % 32), row 8 q + 4 (l / 32) + j, so only
  // the quads q < ceil(rows / 8) hold rows of the group (one quad for up to 8 rows, the
  // usual decode group): the others are neither exchanged nor stored.  Everything derived
  // from the lane and the tile is computed here from opaque copies, so the compiler
  // neither hoists it out of the tile loop nor keeps it (spilled) through the K loop: a
  // reload from scratch behind the weight stream costs a full memory round trip per use.
#define MOE_SK_EPILOGUE(ROWS)                                                           \
  do {                                                                                  \
    int lane_e = lane;                                                                  \
    uint32_t lg_ = logical;                                                             \
    asm volatile("" : "+v"(lane_e), "+s"(lg_));                                         \
    const int lne = lane_e & 31, lhe = lane_e >> 5;                                     \
    const SkTile te = sk_tile<MODE>(plan, lg_, NT);                                     \
    const int nq = (te.nrows + 7) >> 3;                                                 \
    f32x4* red4 = reinterpret_cast<f32x4*>(red);                                        \
    f32x4* mine = red4 + wv * (kSkBlocks * 4 * 64);                                     \
    _Pragma("unroll") for (int b = 0; b < kSkBlocks; ++b)                               \
        _Pragma("unroll") for (int q = 0; q < 4; ++q)                                   \
            if (q < nq)                                                                 \
              mine[(b * 4 + q) * 64 + lane_e] =                                         \
                  f32x4{acc[b][4 * q], acc[b][4 * q + 1], acc[b][4 * q + 2],            \
                        acc[b][4 * q + 3]};                                             \
    __syncthreads();                                                                    \
    if (pre_n) {                                                                        \
      n_aoff = sk_a_off<MODE>(n_src, T, lda) + 64 * lh;                                 \
      ROWS(0, 0, n_aoff);                                                               \
    }                                                                                   \
    if (MODE == 0) {                                                                    \
      /* Wave w: h columns of block w % 2 (gate block w % 2, up block w % 2 + 2), */    \
      /* quads 2 (w / 2) and 2 (w / 2) + 1. */                                          \
      uint16_t* h = static_cast<uint16_t*>(c_out);                                      \
      const int qb = wv & 1;                                                            \
      _Pragma("unroll") for (int qq = 0; qq < 2; ++qq) {                                \
        const int q = 2 * (wv >> 1) + qq;                                               \
        if (q < nq) {                                                                   \
          f32x4 gs = {0.0f, 0.0f, 0.0f, 0.0f}, us = gs;                                 \
          _Pragma("unroll") for (int w2 = 0; w2 < kSkWaves; ++w2) {                     \
            gs += red4[((w2 * kSkBlocks + qb) * 4 + q) * 64 + lane_e];                  \
            us += red4[((w2 * kSkBlocks + qb + 2) * 4 + q) * 64 + lane_e];              \
          }                                                                             \
          _Pragma("unroll") for (int j = 0; j < 4; ++j) {                               \
            const int m = 8 * q + 4 * lhe + j;                                          \
            if (m < te.nrows)                                                           \
              store_h(h + (size_t)(te.row0 + m) * ldc + te.n0 + 32 * qb + lne,          \
                      silu(gs[j]) * us[j]);                                             \
          }                                                                             \
        }                                                                               \
      }                                                                                 \
    } else {                                                                            \
      float* y = static_cast<float*>(c_out);                                            \
      _Pragma("unroll") for (int q = 0; q < 4; ++q) {                                   \
        if (q < nq) {                                                                   \
          f32x4 ys = {0.0f, 0.0f, 0.0f, 0.0f};                                          \
          _Pragma("unroll") for (int w2 = 0; w2 < kSkWaves; ++w2)                       \
              ys += red4[((w2 * kSkBlocks + wv) * 4 + q) * 64 + lane_e];                \
          _Pragma("unroll") for (int j = 0; j < 4; ++j) {                               \
            const int m = 8 * q + 4 * lhe + j;                                          \
            if (m < te.nrows)                                                           \
              y[(size_t)(te.row0 + m) * ldc + te.n0 + 32 * wv + lne] = ys[j];           \
          }                                                                             \
        }                                                                               \
      }                                                                                 \
    }                                                                                   \
    __syncthreads();                                                                    \
  } while (0)

  // The epilogue of the 16-row MXFP4 tiles: partial sums -> LDS as the accumulator
  // quads ([wave][column block][lane], in the wave's own 16 KB, which only it read in the
  // K loop: no wave writes where another may still be reading codes); then gate/up wave
  // w forms h columns 16 w .. +16 (gate block w, up block w + 4) and down wave w outputs
  // column blocks 2 w and 2 w + 1, adding the four waves' partials in wave order; plus
  // the next tile's first A rows at n_aoff.
#define MOE_SK16_EPILOGUE()                                                             \
  do {                                                                                  \
    int lane_e = lane;                                                                  \
    uint32_t lg_ = logical;                                                             \
    asm volatile("" : "+v"(lane_e), "+s"(lg_));                                         \
    const int re = lane_e & 15, ge = lane_e >> 4;                                       \
    const SkTile te = sk_tile<MODE>(plan, lg_, NT);                                     \
    f32x4* red4 = reinterpret_cast<f32x4*>(red);                                        \
    f32x4* mine = red4 + wv * (16 * 64);   /* this wave's own 16 KB */                  \
    _Pragma("unroll") for (int cb = 0; cb < 8; ++cb) mine[cb * 64 + lane_e] = acc16[cb];\
    __syncthreads();                                                                    \
    if (pre_n) {                                                                        \
      n_aoff = sk_a_off<MODE>(n_src, T, lda) + 64 * (lane_e >> 4);                      \
      MOE_SKQ16_ROWS(0, 0, n_aoff);                                                     \
    }                                                                                   \
    if (MODE == 0) {                                                                    \
      uint16_t* h = static_cast<uint16_t*>(c_out);                                      \
      f32x4 gs = {0.0f, 0.0f, 0.0f, 0.0f}, us = gs;                                     \
      _Pragma("unroll") for (int w2 = 0; w2 < kSkWaves; ++w2) {                         \
        gs += red4[(w2 * 16 + wv) * 64 + lane_e];                                        \
        us += red4[(w2 * 16 + wv + 4) * 64 + lane_e];                                    \
      }                                                                                 \
      _Pragma("unroll") for (int j = 0; j < 4; ++j) {                                   \
        const int m = 4 * ge + j;                                                       \
        if (m < te.nrows)                                                               \
          store_h(h + (size_t)(te.row0 + m) * ldc + te.n0 + 16 * wv + re,               \
                  silu(gs[j]) * us[j]);                                                 \
      }                                                                                 \
    } else {                                                                            \
      float* y = static_cast<float*>(c_out);                                            \
      _Pragma("unroll") for (int cc = 0; cc < 2; ++cc) {                                \
        const int cb = 2 * wv + cc;                                                     \
        f32x4 ys = {0.0f, 0.0f, 0.0f, 0.0f};                                            \
        _Pragma("unroll") for (int w2 = 0; w2 < kSkWaves; ++w2)                         \
            ys += red4[(w2 * 16 + cb) * 64 + lane_e];                                    \
        _Pragma("unroll") for (int j = 0; j < 4; ++j) {                                 \
          const int m = 4 * ge + j;                                                     \
          if (m < te.nrows)                                                             \
            y[(size_t)(te.row0 + m) * ldc + te.n0 + 16 * cb + re] = ys[j];              \
        }                                                                               \
      }                                                                                 \
    }                                                                                   \
    __syncthreads();                                                                    \
  } while (0)

  // A workgroup's first tile is its own index, later ones come from the counter offset by
  // the grid: every tile is taken once, without the grid's atomics on one address at the
  // start.
  uint32_t t = blockIdx.x;
  int par = 0;
  bool pre = false;   // this tile's first chunk (pair) was fetched during the previous one
  int n_src = 0;          // A row of the next tile (loaded with its first weights)
  uint32_t n_aoff = 0;    // its byte offset, computed in the epilogue

  // bf16 tiles: every tile of a bf16 layer; in an MXFP4 layer the shared experts' tiles,
  // which the counter hands out before all routed (MXFP4) ones.  Each phase carries only
  // its own operand registers from tile to tile.
  while (t < ntiles) {
    const uint32_t logical = ntiles - 1 - t;
    const SkTile tl = sk_tile<MODE>(plan, logical, NT);
    if (FP4 && tl.g < E) break;
    const uint32_t a_voff =
        pre ? n_aoff : sk_a_off<MODE>(sk_a_src<MODE>(row_token, tl, ln), T, lda) + 64 * lh;
    uint32_t nxt = 0, tn = 0;   // next tile (nxt: lane 0 of wave 0 only)
    bool pre_n = false;         // its first chunk is fetched below
    SkTile ntl{0, 0, 1, 0};
    f32x16 acc[kSkBlocks];
#pragma unroll
    for (int b = 0; b < kSkBlocks; ++b) acc[b] = f32x16{};
    const int nw = max(2, ((nchb + kSkWaves - 1) / kSkWaves + 1) & ~1);
    const SkBSrc src = b_src(tl);
    if (!pre) {
      MOE_SKB_CODES(0, 0, src);
      MOE_SKB_ROWS(0, 0, a_voff);
    }
    int i = 0;
    for (; i + 2 < nw; i += 2) {
      if (i + 4 >= nw && tid == 0) nxt = gridDim.x + atomicAdd(next_tile, 1u);
      MOE_SKB_CODES(i + 1, 1, src);
      MOE_SKB_ROWS(i + 1, 1, a_voff);
      MOE_SKB_MMA(i, 0);
      MOE_SKB_CODES(i + 2, 0, src);
      MOE_SKB_ROWS(i + 2, 0, a_voff);
      MOE_SKB_MMA(i + 1, 1);
    }
    if (nw == 2 && tid == 0) nxt = gridDim.x + atomicAdd(next_tile, 1u);
    MOE_SK_PUBLISH();
    MOE_SKB_CODES(i + 1, 1, src);
    MOE_SKB_ROWS(i + 1, 1, a_voff);
    MOE_SKB_MMA(i, 0);
    if (tn < ntiles) {   // bc[0] is free once chunk i is in LDS
      ntl = sk_tile<MODE>(plan, ntiles - 1 - tn, NT);
      if (!FP4 || ntl.g >= E) {
        n_src = sk_a_src<MODE>(row_token, ntl, ln);
        MOE_SKB_CODES(0, 0, b_src(ntl));
        pre_n = true;
      }
    }
    MOE_SKB_MMA(i + 1, 1);
    MOE_SK_EPILOGUE(MOE_SKB_ROWS);
    t = tn;
    par ^= 1;
    pre = pre_n;
  }

  // MXFP4 tiles (every tile after them is one as well), on 16-row MFMA blocks.
  if (FP4) {
    const int r16 = lane & 15, g16 = lane >> 4;
    // LDS offset of this lane's 16 code bytes in column block 0, per chunk of a pair
    // (B-row r16, MX block g16, slot swizzled by (row / 2) % 8; block cb adds 2048 cb).
    uint32_t lq16[2];
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      lq16[c] = 128 * r16 + 16 * ((4 * c + g16) ^ ((r16 >> 1) & 7));
      asm volatile("" : "+v"(lq16[c]));
    }
    pre = false;
    while (t < ntiles) {
      const uint32_t logical = ntiles - 1 - t;
      const SkTile tl = sk_tile<MODE>(plan, logical, NT);
      const uint32_t a_voff =
          pre ? n_aoff : sk_a_off<MODE>(sk_a_src<MODE>(row_token, tl, r16), T, lda) + 64 * g16;
      uint32_t nxt = 0, tn = 0;
      bool pre_n = false;
      SkTile ntl{0, 0, 1, 0};
      f32x4 acc16[8];
#pragma unroll
      for (int cb = 0; cb < 8; ++cb) acc16[cb] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
      const int nw = 2 * ((nchq + 2 * kSkWaves - 1) / (2 * kSkWaves));
      const SkQSrc src = q_src(tl);
      uint32_t rsp[2];   // chunk 1's scale bytes of a pair, kept past the next fetch
      if (!pre) {
        MOE_SKQ_CODES(0, src);
        MOE_SKQ16_ROWS(0, 0, a_voff);
      }
      int i = 0;
      for (; i + 2 < nw; i += 2) {
        if (i + 4 >= nw && tid == 0) nxt = gridDim.x + atomicAdd(next_tile, 1u);
        MOE_SKQ16_ROWS(i + 1, 1, a_voff);
        MOE_SKQ16_MMA(i, 0);
        MOE_SKQ_CODES(i + 2, src);
        MOE_SKQ16_ROWS(i + 2, 0, a_voff);
        MOE_SKQ16_MMA(i + 1, 1);
      }
      if (nw == 2 && tid == 0) nxt = gridDim.x + atomicAdd(next_tile, 1u);
      MOE_SK_PUBLISH();
      MOE_SKQ16_ROWS(i + 1, 1, a_voff);
      MOE_SKQ16_MMA(i, 0);
      if (tn < ntiles) {   // qc and qs are free once chunk pair i is in LDS
        ntl = sk_tile<MODE>(plan, ntiles - 1 - tn, NT);
        n_src = sk_a_src<MODE>(row_token, ntl, r16);
        MOE_SKQ_CODES(0, q_src(ntl));
        pre_n = true;
      }
      MOE_SKQ16_MMA(i + 1, 1);
      MOE_SK16_EPILOGUE();
      t = tn;
      par ^= 1;
      pre = pre_n;
    }
  }
#undef MOE_SK_EPILOGUE
#undef MOE_SK16_EPILOGUE
#undef MOE_SKQ16_MMA
#undef MOE_SKQ16_ROWS
#undef MOE_SK_PUBLISH
#undef MOE_SKB_MMA
#undef MOE_SKB_ROWS
#undef MOE_SKB_CODES
#undef MOE_SKQ_CODES
#undef MOE_SKQ_CHUNK
#undef MOE_SK_BRO
}

// ---- 256 x 256 tiles (bf16 layers whose groups average at least 128 rows)
//
// The plan (plan_wide_kernel) lists 256-row m-tiles with the groups in descending order
// of rows and a group's cheap last m-tile (at most 128 rows) split into a run of its own
// after its full ones; within a run the tile order is the one above (blocks of 4 n-tiles,
// the run's m-tiles consecutive).  The list is dealt to the XCDs in chunks of 32 tiles,
// one chunk per phase (below), so most chunks hold m-tiles of one size.  A 256 x 256 tile moves
// 64 KB per 64-wide K step for 2 x 256 x 256 x 64 flops, two thirds of the bytes per
// flop of the 128 x 256 tile, so the CU's vector-memory path and the L2 keep up with
// the MFMAs.  The K step is split into two halves, the 256 B-rows (32 KB) and the 256
// A rows (32 KB), streamed by direct buffer->LDS loads through a ring of 5 half slots
// (160 KB): half h (even: B of step h / 2, odd: A of step h / 2) goes to slot h % 5.
// While step kt runs, halves 2kt + 2 .. 2kt + 4 are in flight; the barrier that ends
// step kt frees the slots of halves 2kt and 2kt + 1, which take halves 2kt + 5 and
// 2kt + 6.  The weight halves are issued two steps before use, the row halves one.
// Eight waves in 2 (rows) x 4 (B-rows); each owns 128 rows x 64 B-rows as 4 x 2 MFMA
// 32x32 tiles.  Waves 0..3 hold rows 0..127 and waves 4..7 rows 128..255, one of each
// per SIMD, so a group's last m-tile with at most 128 rows costs each SIMD half a tile:
// waves 4..7 then only take part in the loads and barriers.
constexpr int kWBM = 256;
constexpr int kWHalf = 256 * kRowBytes;   // 32 KB
constexpr int kWSlots = 5;                // 160 KB, the whole LDS of a CU
constexpr bool kPhaseSync = true;
constexpr int kWLoadWaves = 4;            // waves that issue the loads (4 or 8)
constexpr int kWNB = 32 / kWLoadWaves;    // 1 KB blocks per loader wave per half
constexpr uint32_t kSpinTicks = 20000;    // a phase wait ends after 200 us (100 MHz clock)
constexpr int kSpinLimit = 100000;        // and after this many polls in any case


template <int MODE>
__global__ __launch_bounds__(512) void grouped_gemm_wide_kernel(
    const uint16_t* __restrict__ a_src,      // MODE 0: x [T, K]; MODE 1: h [R, K]
    const int32_t* __restrict__ row_token,   // MODE 0 only
    const uint16_t* __restrict__ b0,         // MODE 0: w_gate [G, N, K]; MODE 1: w_down
    const uint16_t* __restrict__ b1,         // MODE 0: w_up [G, N, K]
    const int32_t* __restrict__ offsets,     // [G + 1] group row offsets
    const PlanEntry* __restrict__ plan,      // 256-row m-tiles; plan[0].group = count
    uint32_t* __restrict__ sync,             // [8] phase counters, zero at launch
    void* __restrict__ c_out,                // MODE 0: h [R, N] bf16; MODE 1: y [R, N] f32
    uint32_t a_bytes, int K, int N, int T, int NT,
    int lda, int ldc) {                      // row pitch (elements) of a_src and c_out
  typedef uint16_t TE;
  constexpr int EPC = 8;  // bf16 elements per 16-byte chunk
  __shared__ __attribute__((aligned(1024))) char smem[kWSlots * kWHalf];

  // Chunks of per_xcd consecutive tiles dealt to the XCDs in turn (chunk c on XCD c % 8),
  // one chunk per phase.  Contiguous per-XCD ranges left the XCD that held the shared
  // experts' full tiles ~10% more work than those holding routed groups, whose smaller
  // tail m-tiles cost less (Inkling prefill: 8.92 -> 8.32 ms for both GEMMs).
  const uint32_t ntiles = static_cast<uint32_t>(plan[0].group) * NT;
  const uint32_t xcd = blockIdx.x % kXcds, per_xcd = gridDim.x / kXcds;

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  const int wm = wv >> 2, wn = wv & 3;
  const int lrow = lane >> 3;
  const int lchunk[2] = {(lane & 7) ^ ((lane >> 4) & 7),
                         (lane & 7) ^ ((4 + (lane >> 4)) & 7)};
  int brow[2];
#pragma unroll
  for (int ni = 0; ni < 2; ++ni) {
    if (MODE == 0)
      brow[ni] = ni * kGateUpBN + wn * 32 + (lane & 31);
    else
      brow[ni] = wn * 64 + ni * 32 + (lane & 31);
  }
  int arow[4];
#pragma unroll
  for (int mi = 0; mi < 4; ++mi) arow[mi] = wm * 128 + mi * 32 + (lane & 31);
  const __amdgpu_buffer_rsrc_t a_rsrc = buffer_rsrc(a_src, a_bytes);
  const int KT = K * static_cast<int>(sizeof(TE)) / kRowBytes;

  uint32_t phase = 0;
  for (uint32_t logical = xcd * per_xcd + blockIdx.x / kXcds; logical < ntiles;
       logical += kXcds * per_xcd, ++phase) {
    if (kPhaseSync && MODE == 0) {
      // The XCD's workgroups start each phase together, so the tiles of a phase stay
      // within a few K steps of each other and share their weight and row halves
      // through the L2.  Phases 0..p hold 32 p tiles plus those of chunk 8 p + xcd (all
      // 32 but in the list's last chunk).  The wait is bounded in time: a workgroup that
      // has waited kSpinTicks of the 100 MHz real-time clock (a legitimate wait is the
      // gap between the tiles of one phase, ~10 us on average, tens of us at most) goes
      // on alone, so a workgroup that is not yet resident (another kernel holds its CU)
      // costs each phase at most 200 us; a bound in polls (each an agent-scope load of
      // ~1-2 us) allowed several ms.  (Measured on the Inkling prefill shape: faster for
      // gate/up, slower for the shorter down tiles, which run unsynchronized.)
      if (tid == 0) {
        __hip_atomic_fetch_add(sync + xcd, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const uint32_t target =
            phase * per_xcd + min(per_xcd, ntiles - (phase * kXcds + xcd) * per_xcd);
        const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
        for (int it = 0; it < kSpinLimit; ++it) {
          if (__hip_atomic_load(sync + xcd, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >=
                  target ||
              __builtin_amdgcn_s_memrealtime() - t0 >= kSpinTicks)
            break;
          __builtin_amdgcn_s_sleep(4);
        }
      }
      asm volatile("s_barrier" ::: "memory");
    }
    // The tile's run of m-tiles (a group's full m-tiles, or its split-off tail): first
    // m-tile and length, from the plan entry.
    const PlanEntry first = plan[1 + logical / NT];
    const int g = first.group, gmt0 = first.pad & 0xffff, mg = first.pad >> 16;
    const uint32_t local = logical - static_cast<uint32_t>(gmt0) * NT;
    const int full = NT / kNB;
    int mloc, nt;
    if (local < static_cast<uint32_t>(full * mg * kNB)) {
      const int blk = local / (mg * kNB), rr = local % (mg * kNB);
      mloc = rr / kNB;
      nt = blk * kNB + rr % kNB;
    } else {
      const int rem = NT - full * kNB, rr = local - full * mg * kNB;
      mloc = rr / rem;
      nt = full * kNB + rr % rem;
    }
    const PlanEntry pe = plan[1 + gmt0 + mloc];
    const int row0 = pe.row0, nrows = pe.nrows;
    const int n0 = nt * (MODE == 0 ? kGateUpBN : kDownBN);
    const bool active = wm * 128 < nrows;   // wave-uniform

    // The kWLoadWaves waves wv >= 8 - kWLoadWaves issue every load: loader lw fills 1 KB
    // blocks kWNB lw .. kWNB lw + kWNB - 1 (rows / B-rows 8 kWNB lw ..) of every half.
    const bool loader = wv >= 8 - kWLoadWaves;   // wave-uniform
    const int lw = loader ? wv - (8 - kWLoadWaves) : 0;
    uint32_t a_off[kWNB];
#pragma unroll
    for (int i = 0; i < kWNB; ++i) {
      const int row = 8 * kWNB * lw + 8 * i + lrow;
      const int rr = min(row, nrows - 1);
      uint32_t base;
      if (MODE == 0) {
        int tok = row_token[row0 + rr];
        tok = min(max(tok, 0), T - 1);
        base = static_cast<uint32_t>(tok) * lda;
      } else {
        base = static_cast<uint32_t>(row0 + rr) * lda;
      }
      // Rows past the m-tile get an offset beyond any buffer: the range check turns
      // their loads into zeros without an L1 lookup (their output rows are not stored).
      a_off[i] = row < nrows ? (base + lchunk[i & 1] * EPC) * sizeof(TE) : kPastEnd;
    }
    // gate/up: B-rows 0..127 are gate rows n0.., 128..255 the up rows n0..;  down: B-rows
    // 0..255 are w_down rows n0..  Block i of a loader is B-row brow0 + 8 i + lane / 8.
    const TE* bsrc;
    int brow0;
    if (MODE == 0) {
      bsrc = (lw < kWLoadWaves / 2 ? b0 : b1) + ((size_t)g * N + n0) * K;
      brow0 = 8 * kWNB * (lw % (kWLoadWaves / 2));
    } else {
      bsrc = b0 + ((size_t)g * N + n0) * K;
      brow0 = 8 * kWNB * lw;
    }
    const __amdgpu_buffer_rsrc_t b_rsrc =
        buffer_rsrc(bsrc, static_cast<uint32_t>((MODE == 0 ? kGateUpBN : kDownBN) * K *
                                                sizeof(TE)));
    // Blocks 2j + p sit 16 j rows below blocks p: a per-lane base per parity plus a
    // uniform offset.
    uint32_t b_base[2];
#pragma unroll
    for (int p = 0; p < 2; ++p)
      b_base[p] = (static_cast<uint32_t>(brow0 + 8 * p + lrow) * K + lchunk[p] * EPC) *
                  sizeof(TE);
    const uint32_t b_pair = 16u * K * sizeof(TE);

    f32x16 acc[4][2];
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
      for (int ni = 0; ni < 2; ++ni) acc[mi][ni] = f32x16{};

    // Loads i0 .. i0 + kWNB / 2 - 1 of this wave's kWNB blocks of the A half of step k
    // (slot (2k + 1) % 5) or of the B half of step k (slot 2k % 5); loader waves only.
#define MOE_WLOAD_A(k, i0)                                                              \
  do {                                                                                  \
    if (loader) {                                                                       \
      char* st_ = smem + ((2 * (k) + 1) % kWSlots) * kWHalf + lw * (kWNB * 1024);       \
      _Pragma("unroll") for (int i = (i0); i < (i0) + kWNB / 2; ++i)                    \
          load_lds16(a_rsrc, a_off[i], (k) * kRowBytes, st_ + i * 1024);                \
    }                                                                                   \
  } while (0)
#define MOE_WLOAD_B(k, i0)                                                              \
  do {                                                                                  \
    if (loader) {                                                                       \
      char* st_ = smem + ((2 * (k)) % kWSlots) * kWHalf + lw * (kWNB * 1024);           \
      _Pragma("unroll") for (int i = (i0); i < (i0) + kWNB / 2; ++i)                    \
          load_lds16<MODE == 0 ? kStream : kCached>(                                    \
              b_rsrc, b_base[i & 1], (k) * kRowBytes + (i >> 1) * b_pair, st_ + i * 1024); \
    }                                                                                   \
  } while (0)

    bf16x8 fa[2][4], fb[2][2];
  // In the order the MFMAs use them (row block 0 with both B-row blocks first), so the
  // first MFMAs of a substep wait for three of the six reads, not five.
#define MOE_WLOADF(sa, sb, s, buf)                                                      \
  do {                                                                                  \
    fa[buf][0] = Mfma<TE>::frag((sa), arow[0], (s), lane);                              \
    fb[buf][0] = Mfma<TE>::frag((sb), brow[0], (s), lane);                              \
    fb[buf][1] = Mfma<TE>::frag((sb), brow[1], (s), lane);                              \
    _Pragma("unroll") for (int mi = 1; mi < 4; ++mi)                                    \
        fa[buf][mi] = Mfma<TE>::frag((sa), arow[mi], (s), lane);                        \
  } while (0)

    // Halves 0, 1, 2 (B and A of step 0, B of step 1); wait for halves 0 and 1.  During
    // step kt a loader wave issues halves 2kt + 3 (A of step kt + 1, kWNB / 2 loads in
    // each of substeps 0 and 1) and 2kt + 4 (B of step kt + 2, substeps 2 and 3), into the slots
    // that the barrier ending step kt - 1 freed; spreading them over the step keeps the
    // L1's miss queue busy without stalling a wave's MFMA issue on a burst of loads.
    MOE_WLOAD_B(0, 0);
    MOE_WLOAD_B(0, kWNB / 2);
    MOE_WLOAD_A(0, 0);
    MOE_WLOAD_A(0, kWNB / 2);
    MOE_WLOAD_B(1, 0);
    MOE_WLOAD_B(1, kWNB / 2);
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(kWNB));
    asm volatile("s_barrier" ::: "memory");

    if (active) {
      // MFMAs of substep s from fragment buffer s % 2; substeps 0..2 first load the
      // fragments of substep s + 1 into the other buffer.  The last two K steps are
      // peeled off the loop so that no control-flow join sits between a fragment load
      // and the MFMAs that do not depend on it (the waitcnt pass would wait for every
      // load at a join).
#define MOE_WMMA(cur)                                                                   \
  do {                                                                                  \
    __builtin_amdgcn_sched_barrier(0);                                                  \
    _Pragma("unroll") for (int mi = 0; mi < 4; ++mi)                                    \
        _Pragma("unroll") for (int ni = 0; ni < 2; ++ni)                                \
            acc[mi][ni] = Mfma<TE>::mma(fa[cur][mi], fb[cur][ni], acc[mi][ni]);         \
    __builtin_amdgcn_sched_barrier(0);                                                  \
  } while (0)
      // Step kt; ISSA / ISSB: issue A of step kt + 1 / B of step kt + 2; NEXT: a step
      // follows (wait, barrier, first fragments of step kt + 1).
#define MOE_WSTEP(kt, ISSA, ISSB, NEXT)                                                 \
  do {                                                                                  \
    const char* sa_ = smem + ((2 * (kt) + 1) % kWSlots) * kWHalf;                       \
    const char* sb_ = smem + ((2 * (kt)) % kWSlots) * kWHalf;                           \
    if (ISSA) MOE_WLOAD_A((kt) + 1, 0);                                                 \
    MOE_WLOADF(sa_, sb_, 1, 1);                                                         \
    MOE_WMMA(0);                                                                        \
    if (ISSA) MOE_WLOAD_A((kt) + 1, kWNB / 2);                                          \
    MOE_WLOADF(sa_, sb_, 2, 0);                                                         \
    MOE_WMMA(1);                                                                        \
    if (ISSB) MOE_WLOAD_B((kt) + 2, 0);                                                 \
    MOE_WLOADF(sa_, sb_, 3, 1);                                                         \
    MOE_WMMA(0);                                                                        \
    if (ISSB) MOE_WLOAD_B((kt) + 2, kWNB / 2);                                          \
    if (NEXT) {                                                                         \
      /* Halves 2kt + 2 and 2kt + 3 (step kt + 1) must have landed; only half 2kt + 4 \
         may still be in flight. */                                                     \
      __builtin_amdgcn_s_waitcnt(vmcnt_imm((ISSB) ? kWNB : 0));                         \
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");                   \
      MOE_WLOADF(smem + ((2 * (kt) + 3) % kWSlots) * kWHalf,                            \
                 smem + ((2 * (kt) + 2) % kWSlots) * kWHalf, 0, 0);                     \
    }                                                                                   \
    MOE_WMMA(1);                                                                        \
  } while (0)
      MOE_WLOADF(smem + kWHalf, smem, 0, 0);
      int kt = 0;
      for (; kt + 2 < KT; ++kt) MOE_WSTEP(kt, 1, 1, 1);
      MOE_WSTEP(kt, 1, 0, 1);
      MOE_WSTEP(kt + 1, 0, 0, 0);
#undef MOE_WSTEP
#undef MOE_WMMA
    } else {
      // No rows for this wave in this tile: the same loads, waits and barriers.
      for (int kt = 0; kt + 1 < KT; ++kt) {
        MOE_WLOAD_A(kt + 1, 0);
        MOE_WLOAD_A(kt + 1, kWNB / 2);
        if (kt + 2 < KT) {
          MOE_WLOAD_B(kt + 2, 0);
          MOE_WLOAD_B(kt + 2, kWNB / 2);
          __builtin_amdgcn_s_waitcnt(vmcnt_imm(kWNB));
        } else {
          __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
        }
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
      }
    }
#undef MOE_WLOADF
#undef MOE_WLOAD_B
#undef MOE_WLOAD_A
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");

    if (active) {
#pragma unroll
      for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int rg = 0; rg < 16; ++rg) {
          const int m = wm * 128 + mi * 32 + 8 * (rg >> 2) + 4 * (lane >> 5) + (rg & 3);
          if (m >= nrows) continue;
          const size_t orow = (size_t)(row0 + m) * ldc;
          if (MODE == 0) {
            // Non-temporal outputs: Inkling prefill 8.17 -> 8.08 ms.
            TE* h = static_cast<TE*>(c_out);
            const int n = n0 + wn * 32 + (lane & 31);
            store_h_nt(h + orow + n, silu_hw(acc[mi][0][rg]) * acc[mi][1][rg]);
          } else {
            float* y = static_cast<float*>(c_out);
#pragma unroll
            for (int ni = 0; ni < 2; ++ni) {
              const int n = n0 + wn * 64 + ni * 32 + (lane & 31);
              store_h_nt(y + orow + n, acc[mi][ni][rg]);
            }
          }
        }
    }
  }
}

// m-tile plan: plan[0].group = number of m-tiles; plan[1 + i] = the i-th m-tile, groups in
// order, BM rows each (16 for groups g < E16: the MXFP4 decode tiles) except a group's
// last; .pad holds the group's first m-tile.
template <int BM>
__global__ __launch_bounds__(1024) void plan_kernel(const int32_t* __restrict__ offsets,
                                                    int G, PlanEntry* __restrict__ plan,
                                                    uint32_t* __restrict__ sync, int E16) {
  __shared__ int32_t scan[1024];
  const int g = threadIdx.x;
  if (g < 4 * kSyncEntries) sync[g] = 0;
  const int bm = g < E16 ? kSkBM16 : BM;   // groups g < E16: 16-row m-tiles
  int c = 0, m = 0;
  if (g < G) {
    c = offsets[g + 1] - offsets[g];
    m = (c + bm - 1) / bm;
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
      plan[1 + start + i] = PlanEntry{g, r0 + i * bm, min(bm, c - i * bm), start};
  }
}

// m-tile plan of the 256-row tilings.  plan[0].group = number of m-tiles; plan[1 + i]
// = the i-th m-tile: group, first row, rows, and in .pad its run of m-tiles (first m-tile
// in the low 16 bits, length in the high 16): the tiles of a run are consecutive in the
// kernels' tile list.  SORT: groups in descending order of rows (ties: lower index
// first), and a group's last m-tile with at most 128 rows, when it has full ones before
// it, forms a run of its own right after them, so the 32-tile chunks that an XCD's
// workgroups run together mostly hold m-tiles of one size.  Without SORT: groups in
// index order, one run per group (the order of plan_kernel).
template <bool SORT>
__global__ __launch_bounds__(1024) void plan_wide_kernel(const int32_t* __restrict__ offsets,
                                                         int G, PlanEntry* __restrict__ plan,
                                                         uint32_t* __restrict__ sync) {
  __shared__ int32_t cnt_s[1024];
  __shared__ int32_t by_rank[1024];
  __shared__ int32_t scan[1024];
  const int t = threadIdx.x;
  if (t < 4 * kSyncEntries) sync[t] = 0;
  const int c = t < G ? offsets[t + 1] - offsets[t] : 0;
  cnt_s[t] = c;
  __syncthreads();
  if (t < G) {
    int rank = t;
    if (SORT) {
      rank = 0;
      for (int j = 0; j < G; ++j) {
        const int cj = cnt_s[j];
        rank += (cj > c) || (cj == c && j < t);
      }
    }
    by_rank[rank] = t;
  }
  __syncthreads();
  const int g = t < G ? by_rank[t] : -1;   // the group at rank t
  const int cg = t < G ? cnt_s[g] : 0;
  const int m = (cg + kWBM - 1) / kWBM;
  scan[t] = m;
  __syncthreads();
  for (int o = 1; o < 1024; o <<= 1) {
    const int v = t >= o ? scan[t - o] : 0;
    __syncthreads();
    scan[t] += v;
    __syncthreads();
  }
  const int start = scan[t] - m;
  if (t == 1023) plan[0] = PlanEntry{scan[t], 0, 0, 0};
  if (t < G && m > 0) {
    const int r0 = offsets[g];
    const int split = (SORT && m >= 2 && cg - (m - 1) * kWBM <= kWBM / 2) ? 1 : 0;
    const int mf = m - split;
    for (int i = 0; i < m; ++i) {
      const int run0 = i < mf ? start : start + mf, runlen = i < mf ? mf : 1;
      plan[1 + start + i] =
          PlanEntry{g, r0 + i * kWBM, min(kWBM, cg - i * kWBM), run0 | (runlen << 16)};
    }
  }
}

// Decode-shaped tiling: plan of 32-row m-tiles (16-row for MXFP4 groups), then the gate/up
// and down kernels, each taking tiles from its own counter (zeroed by the plan kernel).
// Two workgroups per CU.
template <bool FP4>
static hipError_t launch_skinny(const uint16_t* x, const int32_t* offsets,
                                const int32_t* row_token, const uint16_t* wg,
                                const uint16_t* wu, const uint16_t* wd, const MxWeights& q,
                                uint16_t* h, float* y, PlanEntry* plan, int T, int d, int I,
                                int E, int G, int R, hipStream_t stream) {
  int dev = 0, cus = 256;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    cus = 256;
  const uint32_t grid = static_cast<uint32_t>(2 * (cus > 0 ? cus : 256));
  uint32_t* sync = reinterpret_cast<uint32_t*>(plan + 1 + max_mtiles(R, G));
  const int hp = static_cast<int>(h_pitch(I));
  hipLaunchKernelGGL(plan_kernel<kSkBM>, dim3(1), dim3(1024), 0, stream, offsets, G, plan,
                     sync, FP4 ? E : 0);
  hipLaunchKernelGGL((grouped_gemm_skinny_kernel<0, FP4>), dim3(grid), dim3(256), 0, stream,
                     x, row_token, wg, wu, q.codes_gate, q.codes_up, q.scales_gate,
                     q.scales_up, plan, sync, static_cast<void*>(h),
                     static_cast<uint32_t>((size_t)T * d * 2), d, I, T, I / 64, d, hp, E);
  hipLaunchKernelGGL((grouped_gemm_skinny_kernel<1, FP4>), dim3(grid), dim3(256), 0, stream,
                     static_cast<const uint16_t*>(h), row_token, wd, wd, q.codes_down,
                     q.codes_down, q.scales_down, q.scales_down, plan, sync + 1,
                     static_cast<void*>(y), static_cast<uint32_t>((size_t)R * hp * 2), I, d,
                     T, d / 128, hp, d, E);
  return hipGetLastError();
}

template <typename TE>
static hipError_t launch_typed(const TE* x, const int32_t* offsets, const int32_t* row_token,
                               const TE* wg, const TE* wu, const TE* wd, TE* h, float* y,
                               PlanEntry* plan, int T, int d, int I, int G, int R,
                               hipStream_t stream) {
  // One workgroup per CU (the LDS ring allows one), a multiple of the 8 XCDs.
  int dev = 0, cus = 256;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    cus = 256;
  const uint32_t grid = static_cast<uint32_t>(cus / kXcds > 0 ? cus / kXcds * kXcds : kXcds);
  if constexpr (sizeof(TE) == 2) {
    if (T <= kDecodeMaxTokens)
      return launch_skinny<false>(x, offsets, row_token, wg, wu, wd, MxWeights{}, h, y, plan,
                                  T, d, I, G, G, R, stream);
  }
  const int nt_gu = I / kGateUpBN;
  const int nt_dn = d / kDownBN;
  uint32_t* sync = reinterpret_cast<uint32_t*>(plan + 1 + max_mtiles(R, G));
  const int hp = static_cast<int>(h_pitch(I));
  if (sizeof(TE) == 2 && use_wide_tiles(1, R, G)) {
    // Groups average at least 128 rows: 256-row tiles.
    const uint16_t* xb = reinterpret_cast<const uint16_t*>(x);
    hipLaunchKernelGGL(plan_wide_kernel<true>, dim3(1), dim3(1024), 0, stream,
                       offsets, G, plan, sync);
    hipLaunchKernelGGL((grouped_gemm_wide_kernel<0>), dim3(grid), dim3(512), 0, stream, xb,
                       row_token, reinterpret_cast<const uint16_t*>(wg),
                       reinterpret_cast<const uint16_t*>(wu), offsets, plan, sync,
                       static_cast<void*>(h), static_cast<uint32_t>((size_t)T * d * 2), d, I,
                       T, nt_gu, d, hp);
    hipLaunchKernelGGL((grouped_gemm_wide_kernel<1>), dim3(grid), dim3(512), 0, stream,
                       reinterpret_cast<const uint16_t*>(h), row_token,
                       reinterpret_cast<const uint16_t*>(wd),
                       reinterpret_cast<const uint16_t*>(wd), offsets, plan, sync + kXcds,
                       static_cast<void*>(y), static_cast<uint32_t>((size_t)R * hp * 2), I, d,
                       T, nt_dn, hp, d);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(plan_kernel<kBM>, dim3(1), dim3(1024), 0, stream, offsets, G, plan,
                     sync, 0);
  hipLaunchKernelGGL((grouped_gemm_kernel<TE, 0, false>), dim3(grid),
                     dim3(512), 0, stream, x, row_token, wg, wu, offsets, plan,
                     static_cast<void*>(h), static_cast<uint32_t>((size_t)T * d * sizeof(TE)),
                     d, I, T, nt_gu, d, hp, nullptr, nullptr, nullptr, nullptr, 0);
  hipLaunchKernelGGL((grouped_gemm_kernel<TE, 1, false>), dim3(grid),
                     dim3(512), 0, stream, static_cast<const TE*>(h), row_token, wd, wd,
                     offsets, plan, static_cast<void*>(y),
                     static_cast<uint32_t>((size_t)R * hp * sizeof(TE)), I, d, T, nt_dn, hp,
                     d, nullptr, nullptr, nullptr, nullptr, 0);
  return hipGetLastError();
}

// bf16 layer whose E routed experts are MXFP4 (the S shared experts bf16 [S, ...]):
// 128-row tiles for every workload.
hipError_t launch_grouped_swiglu_mxfp4(const uint16_t* x, const int32_t* offsets,
                                       const int32_t* row_token, const MxWeights& q,
                                       const uint16_t* wg_shared, const uint16_t* wu_shared,
                                       const uint16_t* wd_shared, uint16_t* h, float* y,
                                       PlanEntry* plan, int T, int d, int I, int E, int G,
                                       int R, hipStream_t stream) {
  if (T <= kDecodeMaxTokens)
    return launch_skinny<true>(x, offsets, row_token, wg_shared, wu_shared, wd_shared, q, h, y,
                               plan, T, d, I, E, G, R, stream);
  int dev = 0, cus = 256;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    cus = 256;
  const uint32_t grid = static_cast<uint32_t>(cus / kXcds > 0 ? cus / kXcds * kXcds : kXcds);
  uint32_t* sync = reinterpret_cast<uint32_t*>(plan + 1 + max_mtiles(R, G));
  const int hp = static_cast<int>(h_pitch(I));
  hipLaunchKernelGGL(plan_kernel<kBM>, dim3(1), dim3(1024), 0, stream, offsets, G, plan,
                     sync, 0);
  hipLaunchKernelGGL((grouped_gemm_kernel<uint16_t, 0, true>), dim3(grid), dim3(512), 0,
                     stream, x, row_token, wg_shared, wu_shared, offsets, plan,
                     static_cast<void*>(h), static_cast<uint32_t>((size_t)T * d * 2), d, I, T,
                     I / kGateUpBN, d, hp, q.codes_gate, q.codes_up, q.scales_gate,
                     q.scales_up, E);
  hipLaunchKernelGGL((grouped_gemm_kernel<uint16_t, 1, true>), dim3(grid), dim3(512), 0,
                     stream, static_cast<const uint16_t*>(h), row_token, wd_shared, wd_shared,
                     offsets, plan, static_cast<void*>(y),
                     static_cast<uint32_t>((size_t)R * hp * 2), I, d, T, d / kDownBN, hp, d,
                     q.codes_down, q.codes_down, q.scales_down, q.scales_down, E);
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
