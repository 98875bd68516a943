// Host stand-ins for the kernel launchers and the two HIP runtime calls of moe_api.cpp, for
// a CPU build of the C ABI under AddressSanitizer and UndefinedBehaviorSanitizer.
//
// Each launcher reads every byte of every buffer the real kernels read and writes every
// byte they write, over the extents the launch arguments give.  The test driver hands the
// C ABI host buffers of exactly the sizes the header states (and a workspace of exactly
// moe_workspace_size bytes), so a wrong extent or workspace offset in the C ABI layer
// becomes a heap overflow that the sanitizer reports.  The permute stand-in writes a valid
// grouping of its (valid) input, so that the later stages see consistent offsets.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "moe.h"
#include "moe_launch.h"

namespace {

volatile uint8_t g_sink;
int g_launches = 0;

void touch_read(const void* p, size_t bytes) {
  if (bytes == 0) return;
  if (p == nullptr) {
    std::fprintf(stderr, "stub: NULL read of %zu bytes\n", bytes);
    std::abort();
  }
  const uint8_t* b = static_cast<const uint8_t*>(p);
  uint8_t acc = 0;
  for (size_t i = 0; i < bytes; ++i) acc ^= b[i];
  g_sink = acc;
}

// The byte ranges written since the last moe_stub_reset(), by buffer role: within one
// entry-point call, buffers of different roles (e.g. the intermediate h and the per-row
// expert outputs, both carved out of the workspace) must not overlap.
struct Written {
  uintptr_t lo, hi;
  const char* role;
};
std::vector<Written> g_written;

void touch_write(void* p, size_t bytes, const char* role) {
  if (bytes == 0) return;
  if (p == nullptr) {
    std::fprintf(stderr, "stub: NULL write of %zu bytes (%s)\n", bytes, role);
    std::abort();
  }
  const uintptr_t lo = reinterpret_cast<uintptr_t>(p), hi = lo + bytes;
  for (const Written& w : g_written)
    if (std::strcmp(w.role, role) != 0 && lo < w.hi && w.lo < hi) {
      std::fprintf(stderr, "stub: %s [%#lx, %#lx) overlaps %s [%#lx, %#lx)\n", role,
                   (unsigned long)lo, (unsigned long)hi, w.role, (unsigned long)w.lo,
                   (unsigned long)w.hi);
      std::abort();
    }
  g_written.push_back({lo, hi, role});
  std::memset(p, 0, bytes);
}

void expect(bool ok, const char* what) {
  if (!ok) {
    std::fprintf(stderr, "stub: launch argument check failed: %s\n", what);
    std::abort();
  }
}

size_t es(int dtype) { return dtype == MOE_BF16 ? 2 : 4; }

}  // namespace

extern "C" int moe_stub_launches() { return g_launches; }
extern "C" void moe_stub_reset() { g_written.clear(); }

extern "C" hipError_t hipGetLastError(void) { return hipSuccess; }
extern "C" hipError_t hipStreamSynchronize(hipStream_t) { return hipSuccess; }

namespace moe {

hipError_t launch_rmsnorm(int dtype, const void* x, const void* gain, void* y, int T, int d,
                          float eps, float gain_offset, hipStream_t) {
  ++g_launches;
  expect(T > 0 && d > 0 && eps > 0 && (gain_offset == 0.0f || gain_offset == 1.0f),
         "rmsnorm dims");
  touch_read(x, es(dtype) * T * d);
  touch_read(gain, es(dtype) * d);
  touch_write(y, es(dtype) * T * d, "rmsnorm y");
  return hipSuccess;
}

hipError_t launch_router_logits(int dtype, const void* x, const void* w_router, float* part,
                                int T, int d, int NE, int nsplit, int kchunk, hipStream_t) {
  ++g_launches;
  expect(nsplit >= 1 && kchunk % 64 == 0 && int64_t{nsplit} * kchunk >= d &&
             int64_t{nsplit - 1} * kchunk < d,
         "router K split covers d exactly once");
  touch_read(x, es(dtype) * T * d);
  touch_read(w_router, es(dtype) * NE * d);
  touch_write(part, sizeof(float) * nsplit * T * NE, "router partial logits");
  return hipSuccess;
}

hipError_t launch_topk(const float* part, int nsplit, int T, int E, int S, int k, int router,
                       int, float route_scale, const float* sel_bias,
                       const float* logit_offset, int32_t* topk_idx, float* weights,
                       hipStream_t) {
  ++g_launches;
  expect(k >= 1 && k <= E && route_scale > 0, "topk dims");
  const int NE = router == MOE_ROUTER_SIGMOID_SHARED ? E + S : E;
  touch_read(part, sizeof(float) * nsplit * T * NE);
  if (sel_bias != nullptr) touch_read(sel_bias, sizeof(float) * E);
  if (logit_offset != nullptr) touch_read(logit_offset, sizeof(float) * E);
  // A valid selection: token t takes experts (t + j) mod E, j < k (distinct).
  touch_write(topk_idx, sizeof(int32_t) * T * k, "topk_idx");
  for (int t = 0; t < T; ++t)
    for (int j = 0; j < k; ++j) topk_idx[int64_t{t} * k + j] = (t + j) % E;
  touch_write(weights, sizeof(float) * T * (k + S), "weights");
  return hipSuccess;
}

hipError_t launch_permute(const int32_t* topk_idx, int T, int E, int S, int k,
                          int32_t* block_hist, int32_t* counts, int32_t* offsets,
                          int32_t* row_token, int32_t* slot_row, hipStream_t) {
  ++g_launches;
  touch_read(topk_idx, sizeof(int32_t) * T * k);
  const int64_t nb = (T + kPermBlock - 1) / kPermBlock;
  touch_write(block_hist, sizeof(int32_t) * nb * E, "block histogram");
  // The grouping the kernels produce: routed groups by expert (tokens ascending), then
  // the shared groups in token order.
  const int A = k + S;
  touch_write(counts, sizeof(int32_t) * (E + S), "counts");
  touch_write(offsets, sizeof(int32_t) * (E + S + 1), "offsets");
  touch_write(row_token, sizeof(int32_t) * T * A, "row_token");
  touch_write(slot_row, sizeof(int32_t) * T * A, "slot_row");
  std::vector<int32_t> cnt(E + S, 0);
  for (int64_t i = 0; i < int64_t{T} * k; ++i) {
    expect(topk_idx[i] >= 0 && topk_idx[i] < E, "permute input in range");
    ++cnt[topk_idx[i]];
  }
  for (int s = 0; s < S; ++s) cnt[E + s] = T;
  offsets[0] = 0;
  for (int g = 0; g < E + S; ++g) {
    counts[g] = cnt[g];
    offsets[g + 1] = offsets[g] + cnt[g];
  }
  expect(offsets[E + S] == T * A, "permute rows");
  std::vector<int32_t> fill(offsets, offsets + E + S);
  for (int t = 0; t < T; ++t)
    for (int j = 0; j < k; ++j) {
      const int g = topk_idx[int64_t{t} * k + j];
      const int32_t r = fill[g]++;
      row_token[r] = t;
      slot_row[int64_t{t} * A + j] = r;
    }
  for (int s = 0; s < S; ++s)
    for (int t = 0; t < T; ++t) {
      const int32_t r = fill[E + s]++;
      row_token[r] = t;
      slot_row[int64_t{t} * A + k + s] = r;
    }
  return hipSuccess;
}

hipError_t launch_grouped_swiglu(int dtype, const void* x, const int32_t* offsets,
                                 const int32_t* row_token, const void* w_gate,
                                 const void* w_up, const void* w_down, void* h, float* y_rows,
                                 PlanEntry* plan, int T, int d, int I, int G, int R,
                                 hipStream_t) {
  ++g_launches;
  touch_read(x, es(dtype) * T * d);
  touch_read(offsets, sizeof(int32_t) * (G + 1));
  expect(offsets[0] == 0 && offsets[G] == R, "grouped offsets span R rows");
  touch_read(row_token, sizeof(int32_t) * R);
  for (int r = 0; r < R; ++r) expect(row_token[r] >= 0 && row_token[r] < T, "row_token");
  touch_read(w_gate, es(dtype) * G * I * d);
  touch_read(w_up, es(dtype) * G * I * d);
  touch_read(w_down, es(dtype) * G * d * I);
  touch_write(plan, sizeof(PlanEntry) * plan_entries(R, G), "m-tile plan");
  touch_write(h, es(dtype) * R * h_pitch(I), "h");
  touch_write(y_rows, sizeof(float) * R * d, "y_rows");
  return hipSuccess;
}

hipError_t launch_grouped_swiglu_mxfp4(const uint16_t* x, const int32_t* offsets,
                                       const int32_t* row_token, const MxWeights& q,
                                       const uint16_t* wg_shared, const uint16_t* wu_shared,
                                       const uint16_t* wd_shared, uint16_t* h, float* y,
                                       PlanEntry* plan, int T, int d, int I, int E, int G,
                                       int R, hipStream_t) {
  ++g_launches;
  const int S = G - E;
  touch_read(x, 2 * int64_t{T} * d);
  touch_read(offsets, sizeof(int32_t) * (G + 1));
  touch_read(row_token, sizeof(int32_t) * R);
  touch_read(q.codes_gate, int64_t{E} * I * d / 2);
  touch_read(q.codes_up, int64_t{E} * I * d / 2);
  touch_read(q.codes_down, int64_t{E} * d * I / 2);
  touch_read(q.scales_gate, mx_scales_bytes(E, I, d));
  touch_read(q.scales_up, mx_scales_bytes(E, I, d));
  touch_read(q.scales_down, mx_scales_bytes(E, d, I));
  if (S > 0) {
    touch_read(wg_shared, 2 * int64_t{S} * I * d);
    touch_read(wu_shared, 2 * int64_t{S} * I * d);
    touch_read(wd_shared, 2 * int64_t{S} * d * I);
  }
  touch_write(plan, sizeof(PlanEntry) * plan_entries(R, G), "m-tile plan");
  touch_write(h, 2 * R * h_pitch(I), "h");
  touch_write(y, sizeof(float) * R * d, "y_rows");
  return hipSuccess;
}

hipError_t launch_combine(const float* y_rows, const int32_t* slot_row, const float* weights,
                          const float* residual, float* out, int T, int d, int A, int R,
                          hipStream_t) {
  ++g_launches;
  expect(R == T * A, "combine rows");
  touch_read(y_rows, sizeof(float) * R * d);
  touch_read(slot_row, sizeof(int32_t) * R);
  for (int r = 0; r < R; ++r) expect(slot_row[r] >= 0 && slot_row[r] < R, "slot_row");
  touch_read(weights, sizeof(float) * T * A);
  if (residual != nullptr) touch_read(residual, sizeof(float) * T * d);
  touch_write(out, sizeof(float) * T * d, "out");
  return hipSuccess;
}

hipError_t launch_pack_mx_scales(const uint8_t* src, uint8_t* dst, int64_t E, int64_t N,
                                 int64_t K, hipStream_t) {
  ++g_launches;
  touch_read(src, E * N * (K / 32));
  touch_write(dst, mx_scales_bytes(E, N, K), "packed scales");
  return hipSuccess;
}

}  // namespace moe
