// C ABI of the MoE layer: argument validation, workspace layout and the launch sequence.
// Nothing here allocates, frees or synchronizes (except the opt-in MOE_DEBUG_SYNC=1
// mode, which synchronizes the stream after every launch to localize failures).
#include <cmath>
#include <cstdint>
#include <cstdlib>

#include "moe.h"
#include "moe_launch.h"

namespace {

using moe::PlanEntry;

constexpr size_t kAlign = 256;
constexpr int kMaxNormWidth = 16384;   // rmsnorm_kernel: 256 threads x 8 runs of 8

size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

struct Layout {
  int nsplit = 1, kchunk = 0;
  size_t part = 0, idx = 0, wts = 0, counts = 0, offsets = 0, row_token = 0, slot_row = 0,
         hist = 0, plan = 0, h = 0, y = 0, xn = 0, total = 0;
};

struct Dims {
  int64_t T, d, E, S, I, k, A, G, R;
  int64_t NR;  // router rows: E + S (sigmoid) or E (softmax: ungated shared experts)
  int dtype;
};

Dims dims_of(const moe_config_t& c, int64_t T) {
  Dims m;
  m.T = T;
  m.d = c.d_model;
  m.E = c.n_experts;
  m.S = c.n_shared;
  m.I = c.d_ff;
  m.k = c.top_k;
  m.A = m.k + m.S;
  m.G = m.E + m.S;
  m.dtype = c.dtype;
  m.R = T * m.A;
  m.NR = c.router == MOE_ROUTER_SIGMOID_SHARED ? m.G : m.E;
  return m;
}

// Router K split: enough workgroups to cover the chip at small T, chunks of >= 256.
void router_split(const Dims& m, int* nsplit, int* kchunk) {
  const int64_t tile = moe::router_tile(m.dtype, m.T);
  const int64_t tiles = ((m.T + tile - 1) / tile) * ((m.NR + tile - 1) / tile);
  int64_t maxsplit = m.d / 256 > 0 ? m.d / 256 : 1;
  int64_t want = tiles > 0 ? (512 + tiles - 1) / tiles : 1;
  int64_t ns = want < maxsplit ? want : maxsplit;
  if (ns < 1) ns = 1;
  int64_t kc = (m.d + ns - 1) / ns;
  kc = (kc + 63) / 64 * 64;
  ns = (m.d + kc - 1) / kc;
  *nsplit = static_cast<int>(ns);
  *kchunk = static_cast<int>(kc);
}

Layout layout_of(const moe_config_t& c, int64_t T) {
  const Dims m = dims_of(c, T);
  Layout L;
  router_split(m, &L.nsplit, &L.kchunk);
  const size_t esize = c.dtype == MOE_BF16 ? 2 : 4;
  const int64_t nb = (T + moe::kPermBlock - 1) / moe::kPermBlock;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off += align_up(bytes);
    return at;
  };
  L.part = take(sizeof(float) * L.nsplit * m.T * m.NR);
  L.idx = take(sizeof(int32_t) * m.T * m.k);
  L.wts = take(sizeof(float) * m.T * m.A);
  L.counts = take(sizeof(int32_t) * m.G);
  L.offsets = take(sizeof(int32_t) * (m.G + 1));
  L.row_token = take(sizeof(int32_t) * m.R);
  L.slot_row = take(sizeof(int32_t) * m.R);
  L.hist = take(sizeof(int32_t) * nb * m.E);
  L.plan = take(sizeof(PlanEntry) * moe::plan_entries(m.R, m.G));
  L.h = take(esize * m.R * moe::h_pitch(m.I));
  L.y = take(sizeof(float) * m.R * m.d);
  L.xn = take(esize * m.T * m.d);   // normalized input of moe_forward_rmsnorm
  L.total = off;
  return L;
}

moe_status_t check_cfg(const moe_config_t* c) {
  if (c == nullptr) return MOE_ERR_ARG;
  if (c->d_model <= 0 || c->n_experts <= 0 || c->d_ff <= 0 || c->top_k <= 0 ||
      c->n_shared < 0)
    return MOE_ERR_ARG;
  if (c->router != MOE_ROUTER_SOFTMAX_TOPK && c->router != MOE_ROUTER_SIGMOID_SHARED)
    return MOE_ERR_ARG;
  if (c->dtype != MOE_F32 && c->dtype != MOE_BF16) return MOE_ERR_ARG;
  if (c->bias_on_logits != 0 && c->bias_on_logits != 1) return MOE_ERR_ARG;
  if (c->top_k > c->n_experts) return MOE_ERR_ARG;
  if (!std::isfinite(c->route_scale) || !(c->route_scale > 0.0f)) return MOE_ERR_ARG;
  if (c->router == MOE_ROUTER_SOFTMAX_TOPK &&
      (c->route_scale != 1.0f || c->bias_on_logits != 0))
    return MOE_ERR_ARG;
  if (c->top_k > 32 || c->n_shared > 8 || c->n_experts + c->n_shared > 1024)
    return MOE_ERR_UNSUPPORTED;
  if (c->d_model % moe::kDownBN != 0 || c->d_ff % moe::kGateUpBN != 0)
    return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

moe_status_t check_tokens(const moe_config_t& c, int64_t T) {
  if (T < 0) return MOE_ERR_ARG;
  const Dims m = dims_of(c, T);
  const int64_t lim = int64_t{1} << 31;
  const int64_t widest = m.d > m.I ? m.d : m.I;
  // 32-bit element offsets into the grouped rows inside the kernels.
  if (m.R > lim / widest) return MOE_ERR_UNSUPPORTED;
  // The GEMMs and the router read x [T, d] and the intermediate h [R, I + pad] through
  // buffer resources with 32-bit sizes and byte offsets: both stay below 2^31 bytes.
  const int64_t es = m.dtype == MOE_BF16 ? 2 : 4;
  if (m.T > (lim - 1) / (m.d * es) || m.R > (lim - 1) / (moe::h_pitch(m.I) * es))
    return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

moe_status_t check_ws(const moe_config_t& c, int64_t T, const void* ws, size_t ws_bytes) {
  if (ws == nullptr || (reinterpret_cast<uintptr_t>(ws) & (kAlign - 1)) != 0)
    return MOE_ERR_ARG;
  if (ws_bytes < layout_of(c, T).total) return MOE_ERR_WORKSPACE;
  return MOE_OK;
}

template <typename P>
P* at(void* ws, size_t off) {
  return reinterpret_cast<P*>(static_cast<char*>(ws) + off);
}

bool debug_sync() {
  const char* v = std::getenv("MOE_DEBUG_SYNC");
  return v != nullptr && v[0] == '1';
}

moe_status_t finish(hipError_t e, hipStream_t stream) {
  if (e != hipSuccess) return MOE_ERR_HIP;
  if (debug_sync()) {
    if (hipStreamSynchronize(stream) != hipSuccess) return MOE_ERR_HIP;
    if (hipGetLastError() != hipSuccess) return MOE_ERR_HIP;
  }
  return MOE_OK;
}

#define MOE_TRY(expr)                     \
  do {                                    \
    const moe_status_t st_ = (expr);      \
    if (st_ != MOE_OK) return st_;        \
  } while (0)

moe_status_t do_route(const moe_config_t& c, int64_t T, const void* x, const void* w_router,
                      const float* sel_bias, const float* logit_offset, int32_t* topk_idx,
                      float* weights, void* ws, hipStream_t stream) {
  const Layout L = layout_of(c, T);
  const Dims m = dims_of(c, T);
  float* part = at<float>(ws, L.part);
  MOE_TRY(finish(moe::launch_router_logits(c.dtype, x, w_router, part, (int)m.T, (int)m.d,
                                           (int)m.NR, L.nsplit, L.kchunk, stream),
                 stream));
  return finish(moe::launch_topk(part, L.nsplit, (int)m.T, (int)m.E, (int)m.S, (int)m.k,
                                 c.router, c.bias_on_logits, c.route_scale, sel_bias,
                                 logit_offset, topk_idx, weights, stream),
                stream);
}

moe_status_t do_permute(const moe_config_t& c, int64_t T, const int32_t* topk_idx,
                        int32_t* counts, int32_t* offsets, int32_t* row_token,
                        int32_t* slot_row, void* ws, hipStream_t stream) {
  const Layout L = layout_of(c, T);
  const Dims m = dims_of(c, T);
  return finish(moe::launch_permute(topk_idx, (int)m.T, (int)m.E, (int)m.S, (int)m.k,
                                    at<int32_t>(ws, L.hist), counts, offsets, row_token,
                                    slot_row, stream),
                stream);
}

moe_status_t do_grouped(const moe_config_t& c, int64_t T, const void* x,
                        const int32_t* offsets, const int32_t* row_token, const void* w_gate,
                        const void* w_up, const void* w_down, float* y_rows, void* ws,
                        hipStream_t stream) {
  const Layout L = layout_of(c, T);
  const Dims m = dims_of(c, T);
  return finish(moe::launch_grouped_swiglu(c.dtype, x, offsets, row_token, w_gate, w_up,
                                           w_down, at<void>(ws, L.h), y_rows,
                                           at<PlanEntry>(ws, L.plan), (int)m.T, (int)m.d,
                                           (int)m.I, (int)m.G, (int)m.R, stream),
                stream);
}

moe_status_t do_grouped_mxfp4(const moe_config_t& c, int64_t T, const void* x,
                              const int32_t* offsets, const int32_t* row_token,
                              const moe::MxWeights& q, const void* wg_shared,
                              const void* wu_shared, const void* wd_shared, float* y_rows,
                              void* ws, hipStream_t stream) {
  const Layout L = layout_of(c, T);
  const Dims m = dims_of(c, T);
  return finish(moe::launch_grouped_swiglu_mxfp4(
                    static_cast<const uint16_t*>(x), offsets, row_token, q,
                    static_cast<const uint16_t*>(wg_shared),
                    static_cast<const uint16_t*>(wu_shared),
                    static_cast<const uint16_t*>(wd_shared), at<uint16_t>(ws, L.h), y_rows,
                    at<PlanEntry>(ws, L.plan), (int)m.T, (int)m.d, (int)m.I, (int)m.E,
                    (int)m.G, (int)m.R, stream),
                stream);
}

// MXFP4 pointers: codes and packed scales 16-byte aligned; shared experts' bf16 weights
// present iff S > 0.
moe_status_t check_mxfp4(const moe_config_t& c, const uint8_t* const* q, const void* wg_s,
                         const void* wu_s, const void* wd_s) {
  if (c.dtype != MOE_BF16) return MOE_ERR_UNSUPPORTED;
  for (int i = 0; i < 6; ++i)
    if (q[i] == nullptr || !aligned16(q[i])) return MOE_ERR_ARG;
  if (c.n_shared > 0) {
    if (wg_s == nullptr || wu_s == nullptr || wd_s == nullptr) return MOE_ERR_ARG;
    if (!aligned16(wg_s) || !aligned16(wu_s) || !aligned16(wd_s)) return MOE_ERR_ARG;
  }
  return MOE_OK;
}

// Shape of a scale tensor to pack: whole MX blocks along K, whole 64-row records along N.
moe_status_t check_mx_dims(int64_t E, int64_t N, int64_t K) {
  if (E <= 0 || N <= 0 || K <= 0) return MOE_ERR_ARG;
  if (N % moe::kMxRecRows != 0 || K % 32 != 0) return MOE_ERR_UNSUPPORTED;
  // 32-bit byte offsets inside the GEMM kernels (one expert's scales).
  if ((N / moe::kMxRecRows) * moe::mx_rec_k(K) * moe::kMxRecBytes >= (int64_t{1} << 31))
    return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

moe_status_t do_combine(const moe_config_t& c, int64_t T, const float* y_rows,
                        const int32_t* slot_row, const float* weights, const float* residual,
                        float* out, hipStream_t stream) {
  const Dims m = dims_of(c, T);
  return finish(moe::launch_combine(y_rows, slot_row, weights, residual, out, (int)m.T,
                                    (int)m.d, (int)m.A, (int)m.R, stream),
                stream);
}

}  // namespace

namespace moe {

moe_status_t check_forward_args(const moe_config_t* cfg, int64_t T, const void* x,
                                const void* w_router, const float* sel_bias,
                                const void* w_gate, const void* w_up, const void* w_down,
                                const float* residual, const float* out,
                                size_t* ws_bytes_needed) {
  MOE_TRY(check_cfg(cfg));
  MOE_TRY(check_tokens(*cfg, T));
  if (ws_bytes_needed != nullptr) *ws_bytes_needed = layout_of(*cfg, T).total;
  if (T == 0) return MOE_OK;
  if (x == nullptr || w_router == nullptr || w_gate == nullptr || w_up == nullptr ||
      w_down == nullptr || out == nullptr)
    return MOE_ERR_ARG;
  if (!aligned16(x) || !aligned16(w_router) || !aligned16(w_gate) || !aligned16(w_up) ||
      !aligned16(w_down) || !aligned16(out) || (residual != nullptr && !aligned16(residual)))
    return MOE_ERR_ARG;
  if (sel_bias != nullptr && cfg->router != MOE_ROUTER_SIGMOID_SHARED) return MOE_ERR_ARG;
  return MOE_OK;
}

}  // namespace moe

extern "C" {

const char* moe_status_str(moe_status_t s) {
  switch (s) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_ARG: return "MOE_ERR_ARG: invalid argument";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED: shape not supported by this build";
    case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE: workspace too small";
    case MOE_ERR_HIP: return "MOE_ERR_HIP: HIP launch or runtime error";
  }
  return "MOE_ERR_UNKNOWN";
}

moe_status_t moe_workspace_size(const moe_config_t* cfg, int64_t T, size_t* bytes) {
  MOE_TRY(check_cfg(cfg));
  if (bytes == nullptr) return MOE_ERR_ARG;
  MOE_TRY(check_tokens(*cfg, T));
  *bytes = layout_of(*cfg, T).total;
  return MOE_OK;
}

moe_status_t moe_route(const moe_config_t* cfg, int64_t T, const void* x,
                       const void* w_router, const float* sel_bias, const float* logit_offset,
                       int32_t* topk_idx, float* weights, void* ws, size_t ws_bytes,
                       hipStream_t stream) {
  MOE_TRY(check_cfg(cfg));
  MOE_TRY(check_tokens(*cfg, T));
  if (T == 0) return MOE_OK;
  if (x == nullptr || w_router == nullptr || topk_idx == nullptr || weights == nullptr)
    return MOE_ERR_ARG;
  if (!aligned16(x) || !aligned16(w_router)) return MOE_ERR_ARG;
  if (sel_bias != nullptr && cfg->router != MOE_ROUTER_SIGMOID_SHARED) return MOE_ERR_ARG;
  MOE_TRY(check_ws(*cfg, T, ws, ws_bytes));
  (void)hipGetLastError();
  return do_route(*cfg, T, x, w_router, sel_bias, logit_offset, topk_idx, weights, ws, stream);
}

moe_status_t moe_permute(const moe_config_t* cfg, int64_t T, const int32_t* topk_idx,
                         int32_t* counts, int32_t* offsets, int32_t* row_token,
                         int32_t* slot_row, void* ws, size_t ws_bytes, hipStream_t stream) {
  MOE_TRY(check_cfg(cfg));
  MOE_TRY(check_tokens(*cfg, T));
  if (T == 0) return MOE_OK;
  if (topk_idx == nullptr || counts == nullptr || offsets == nullptr || row_token == nullptr ||
      slot_row == nullptr)
    return MOE_ERR_ARG;
  MOE_TRY(check_ws(*cfg, T, ws, ws_bytes));
  (void)hipGetLastError();
  return do_permute(*cfg, T, topk_idx, counts, offsets, row_token, slot_row, ws, stream);
}

moe_status_t moe_grouped_swiglu(const moe_config_t* cfg, int64_t T, const void* x,
                                const int32_t* offsets, const int32_t* row_token,
                                const void* w_gate, const void* w_up, const void* w_down,
                                float* y_rows, void* ws, size_t ws_bytes, hipStream_t stream) {
  MOE_TRY(check_cfg(cfg));
  MOE_TRY(check_tokens(*cfg, T));
  if (T == 0) return MOE_OK;
  if (x == nullptr || offsets == nullptr || row_token == nullptr || w_gate == nullptr ||
      w_up == nullptr || w_down == nullptr || y_rows == nullptr)
    return MOE_ERR_ARG;
  if (!aligned16(x) || !aligned16(w_gate) || !aligned16(w_up) || !aligned16(w_down) ||
      !aligned16(y_rows))
    return MOE_ERR_ARG;
  MOE_TRY(check_ws(*cfg, T, ws, ws_bytes));
  (void)hipGetLastError();
  return do_grouped(*cfg, T, x, offsets, row_token, w_gate, w_up, w_down, y_rows, ws, stream);
}

moe_status_t moe_combine(const moe_config_t* cfg, int64_t T, const float* y_rows,
                         const int32_t* slot_row, const float* weights, const float* residual,
                         float* out, hipStream_t stream) {
  MOE_TRY(check_cfg(cfg));
  MOE_TRY(check_tokens(*cfg, T));
  if (T == 0) return MOE_OK;
  if (y_rows == nullptr || slot_row == nullptr || weights == nullptr || out == nullptr)
    return MOE_ERR_ARG;
  if (!aligned16(y_rows) || !aligned16(out) || (residual != nullptr && !aligned16(residual)))
    return MOE_ERR_ARG;
  (void)hipGetLastError();
  return do_combine(*cfg, T, y_rows, slot_row, weights, residual, out, stream);
}

moe_status_t moe_forward(const moe_config_t* cfg, int64_t T, const void* x,
                         const void* w_router, const float* sel_bias,
                         const float* logit_offset, const void* w_gate, const void* w_up,
                         const void* w_down, const float* residual, float* out,
                         int32_t* topk_idx_out, int32_t* counts_out, void* ws,
                         size_t ws_bytes, hipStream_t stream) {
  MOE_TRY(moe::check_forward_args(cfg, T, x, w_router, sel_bias, w_gate, w_up, w_down,
                                  residual, out, nullptr));
  if (T == 0) return MOE_OK;
  MOE_TRY(check_ws(*cfg, T, ws, ws_bytes));
  (void)hipGetLastError();
  const Layout L = layout_of(*cfg, T);
  int32_t* idx = topk_idx_out != nullptr ? topk_idx_out : at<int32_t>(ws, L.idx);
  int32_t* counts = counts_out != nullptr ? counts_out : at<int32_t>(ws, L.counts);
  float* wts = at<float>(ws, L.wts);
  int32_t* offsets = at<int32_t>(ws, L.offsets);
  int32_t* row_token = at<int32_t>(ws, L.row_token);
  int32_t* slot_row = at<int32_t>(ws, L.slot_row);
  float* y = at<float>(ws, L.y);
  MOE_TRY(do_route(*cfg, T, x, w_router, sel_bias, logit_offset, idx, wts, ws, stream));
  MOE_TRY(do_permute(*cfg, T, idx, counts, offsets, row_token, slot_row, ws, stream));
  MOE_TRY(do_grouped(*cfg, T, x, offsets, row_token, w_gate, w_up, w_down, y, ws, stream));
  return do_combine(*cfg, T, y, slot_row, wts, residual, out, stream);
}

moe_status_t moe_grouped_swiglu_mxfp4(const moe_config_t* cfg, int64_t T, const void* x,
                                      const int32_t* offsets, const int32_t* row_token,
                                      const uint8_t* wq_gate, const uint8_t* ws_gate,
                                      const uint8_t* wq_up, const uint8_t* ws_up,
                                      const uint8_t* wq_down, const uint8_t* ws_down,
                                      const void* w_gate_shared, const void* w_up_shared,
                                      const void* w_down_shared, float* y_rows, void* ws,
                                      size_t ws_bytes, hipStream_t stream) {
  MOE_TRY(check_cfg(cfg));
  MOE_TRY(check_tokens(*cfg, T));
  const uint8_t* q[6] = {wq_gate, ws_gate, wq_up, ws_up, wq_down, ws_down};
  if (cfg->dtype != MOE_BF16) return MOE_ERR_UNSUPPORTED;
  if (T == 0) return MOE_OK;
  MOE_TRY(check_mxfp4(*cfg, q, w_gate_shared, w_up_shared, w_down_shared));
  if (x == nullptr || offsets == nullptr || row_token == nullptr || y_rows == nullptr)
    return MOE_ERR_ARG;
  if (!aligned16(x) || !aligned16(y_rows)) return MOE_ERR_ARG;
  MOE_TRY(check_ws(*cfg, T, ws, ws_bytes));
  (void)hipGetLastError();
  const moe::MxWeights mx{wq_gate, ws_gate, wq_up, ws_up, wq_down, ws_down};
  return do_grouped_mxfp4(*cfg, T, x, offsets, row_token, mx, w_gate_shared, w_up_shared,
                          w_down_shared, y_rows, ws, stream);
}

moe_status_t moe_forward_mxfp4(const moe_config_t* cfg, int64_t T, const void* x,
                               const void* w_router, const float* sel_bias,
                               const float* logit_offset, const uint8_t* wq_gate,
                               const uint8_t* ws_gate, const uint8_t* wq_up,
                               const uint8_t* ws_up, const uint8_t* wq_down,
                               const uint8_t* ws_down, const void* w_gate_shared,
                               const void* w_up_shared, const void* w_down_shared,
                               const float* residual, float* out, int32_t* topk_idx_out,
                               int32_t* counts_out, void* ws, size_t ws_bytes,
                               hipStream_t stream) {
  MOE_TRY(check_cfg(cfg));
  MOE_TRY(check_tokens(*cfg, T));
  const uint8_t* q[6] = {wq_gate, ws_gate, wq_up, ws_up, wq_down, ws_down};
  if (cfg->dtype != MOE_BF16) return MOE_ERR_UNSUPPORTED;
  if (T == 0) return MOE_OK;
  MOE_TRY(check_mxfp4(*cfg, q, w_gate_shared, w_up_shared, w_down_shared));
  if (x == nullptr || w_router == nullptr || out == nullptr) return MOE_ERR_ARG;
  if (!aligned16(x) || !aligned16(w_router) || !aligned16(out) ||
      (residual != nullptr && !aligned16(residual)))
    return MOE_ERR_ARG;
  if (sel_bias != nullptr && cfg->router != MOE_ROUTER_SIGMOID_SHARED) return MOE_ERR_ARG;
  MOE_TRY(check_ws(*cfg, T, ws, ws_bytes));
  (void)hipGetLastError();
  const Layout L = layout_of(*cfg, T);
  int32_t* idx = topk_idx_out != nullptr ? topk_idx_out : at<int32_t>(ws, L.idx);
  int32_t* counts = counts_out != nullptr ? counts_out : at<int32_t>(ws, L.counts);
  float* wts = at<float>(ws, L.wts);
  int32_t* offsets = at<int32_t>(ws, L.offsets);
  int32_t* row_token = at<int32_t>(ws, L.row_token);
  int32_t* slot_row = at<int32_t>(ws, L.slot_row);
  float* y = at<float>(ws, L.y);
  const moe::MxWeights mx{wq_gate, ws_gate, wq_up, ws_up, wq_down, ws_down};
  MOE_TRY(do_route(*cfg, T, x, w_router, sel_bias, logit_offset, idx, wts, ws, stream));
  MOE_TRY(do_permute(*cfg, T, idx, counts, offsets, row_token, slot_row, ws, stream));
  MOE_TRY(do_grouped_mxfp4(*cfg, T, x, offsets, row_token, mx, w_gate_shared, w_up_shared,
                           w_down_shared, y, ws, stream));
  return do_combine(*cfg, T, y, slot_row, wts, residual, out, stream);
}

moe_status_t moe_mxfp4_scales_bytes(int64_t E, int64_t N, int64_t K, size_t* bytes) {
  if (bytes == nullptr) return MOE_ERR_ARG;
  MOE_TRY(check_mx_dims(E, N, K));
  *bytes = static_cast<size_t>(moe::mx_scales_bytes(E, N, K));
  return MOE_OK;
}

moe_status_t moe_mxfp4_pack_scales(int64_t E, int64_t N, int64_t K, const uint8_t* scales,
                                   uint8_t* packed, hipStream_t stream) {
  MOE_TRY(check_mx_dims(E, N, K));
  if (scales == nullptr || packed == nullptr || !aligned16(packed)) return MOE_ERR_ARG;
  (void)hipGetLastError();
  return finish(moe::launch_pack_mx_scales(scales, packed, E, N, K, stream), stream);
}

moe_status_t moe_rmsnorm(const moe_config_t* cfg, int64_t T, const void* x,
                         const void* gain, float eps, int32_t zero_centred, void* y,
                         hipStream_t stream) {
  MOE_TRY(check_cfg(cfg));
  MOE_TRY(check_tokens(*cfg, T));
  if (!std::isfinite(eps) || !(eps > 0.0f) || (zero_centred != 0 && zero_centred != 1))
    return MOE_ERR_ARG;
  if (cfg->d_model > kMaxNormWidth) return MOE_ERR_UNSUPPORTED;
  if (T == 0) return MOE_OK;
  if (x == nullptr || gain == nullptr || y == nullptr) return MOE_ERR_ARG;
  if (!aligned16(x) || !aligned16(gain) || !aligned16(y)) return MOE_ERR_ARG;
  (void)hipGetLastError();
  return finish(moe::launch_rmsnorm(cfg->dtype, x, gain, y, (int)T, cfg->d_model, eps,
                                    zero_centred ? 1.0f : 0.0f, stream),
                stream);
}

moe_status_t moe_forward_rmsnorm(const moe_config_t* cfg, int64_t T, const void* x,
                                 const void* norm_gain, float eps, int32_t zero_centred,
                                 const void* w_router, const float* sel_bias,
                                 const float* logit_offset, const void* w_gate,
                                 const void* w_up, const void* w_down, const float* residual,
                                 float* out, int32_t* topk_idx_out, int32_t* counts_out,
                                 void* ws, size_t ws_bytes, hipStream_t stream) {
  MOE_TRY(check_cfg(cfg));
  MOE_TRY(check_tokens(*cfg, T));
  if (!std::isfinite(eps) || !(eps > 0.0f) || (zero_centred != 0 && zero_centred != 1))
    return MOE_ERR_ARG;
  if (cfg->d_model > kMaxNormWidth) return MOE_ERR_UNSUPPORTED;
  if (T == 0) return MOE_OK;
  if (x == nullptr || norm_gain == nullptr || !aligned16(x) || !aligned16(norm_gain))
    return MOE_ERR_ARG;
  MOE_TRY(check_ws(*cfg, T, ws, ws_bytes));
  (void)hipGetLastError();
  const Layout L = layout_of(*cfg, T);
  void* xn = at<void>(ws, L.xn);
  MOE_TRY(finish(moe::launch_rmsnorm(cfg->dtype, x, norm_gain, xn, (int)T, cfg->d_model, eps,
                                     zero_centred ? 1.0f : 0.0f, stream),
                 stream));
  return moe_forward(cfg, T, xn, w_router, sel_bias, logit_offset, w_gate, w_up, w_down,
                     residual, out, topk_idx_out, counts_out, ws, ws_bytes, stream);
}

}  // extern "C"
