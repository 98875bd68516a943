// Driver of the host sanitizer build of the C ABI (moe_api.cpp + abi_stubs.cpp, no GPU).
// Each checked call starts a fresh record of written ranges, so the stand-ins can check
// that the buffers one entry point writes do not overlap.
//
// For several layer shapes it calls every entry point of include/moe.h (except
// moe_forward_static, whose scratch lives in device memory) with host buffers of exactly
// the sizes the header states, a workspace of exactly moe_workspace_size bytes, and the
// stand-in launchers, which touch every byte the kernels would.  It then drives the
// argument checks (NULL and misaligned pointers, bad configs, a short workspace, the
// 32-bit token limits, T = 0) and checks each status.  Exit status 0 means every call
// returned what it should and the sanitizers reported nothing.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "moe.h"

extern "C" int moe_stub_launches();
extern "C" void moe_stub_reset();

namespace {

int g_fail = 0;

#define CHECK_STATUS(call, want)                                                       \
  do {                                                                                 \
    moe_stub_reset();                                                                  \
    const moe_status_t got_ = (call);                                                  \
    if (got_ != (want)) {                                                              \
      std::fprintf(stderr, "%s:%d: %s returned %d, expected %d\n", __FILE__, __LINE__, \
                   #call, (int)got_, (int)(want));                                     \
      ++g_fail;                                                                        \
    }                                                                                  \
  } while (0)

// A heap buffer of exactly `bytes` bytes, 256-byte aligned, filled with a pattern.
struct Buf {
  void* p = nullptr;
  size_t n = 0;
  explicit Buf(size_t bytes) : n(bytes) {
    if (bytes == 0) return;
    if (posix_memalign(&p, 256, bytes) != 0) std::abort();
    std::memset(p, 0x5A, bytes);
  }
  ~Buf() { std::free(p); }
  Buf(const Buf&) = delete;
  Buf& operator=(const Buf&) = delete;
  template <typename P>
  P* as() const { return static_cast<P*>(p); }
};

struct Shape {
  const char* name;
  int64_t T;
  int d, E, S, I, k;
  int router, dtype;
  bool mxfp4;
};

size_t es(int dtype) { return dtype == MOE_BF16 ? 2 : 4; }

moe_config_t config_of(const Shape& s) {
  moe_config_t c{};
  c.d_model = s.d;
  c.n_experts = s.E;
  c.d_ff = s.I;
  c.top_k = s.k;
  c.n_shared = s.S;
  c.router = s.router;
  c.dtype = s.dtype;
  c.bias_on_logits = 0;
  c.route_scale = s.router == MOE_ROUTER_SIGMOID_SHARED ? float(s.k + s.S) : 1.0f;
  return c;
}

size_t packed_scales(int64_t E, int64_t N, int64_t K) {
  size_t b = 0;
  if (moe_mxfp4_scales_bytes(E, N, K, &b) != MOE_OK) std::abort();
  return b;
}

void run_shape(const Shape& s) {
  const moe_config_t cfg = config_of(s);
  const int64_t T = s.T, d = s.d, E = s.E, S = s.S, I = s.I, k = s.k;
  const int64_t A = k + S, G = E + S, R = T * A;
  const int64_t NR = s.router == MOE_ROUTER_SIGMOID_SHARED ? G : E;
  const size_t e = es(s.dtype);
  size_t ws_bytes = 0;
  CHECK_STATUS(moe_workspace_size(&cfg, T, &ws_bytes), MOE_OK);
  Buf ws(ws_bytes), x(e * T * d), wr(e * NR * d), bias(4 * E), off(4 * E), gain(e * d);
  Buf wg(e * G * I * d), wu(e * G * I * d), wd(e * G * d * I);
  Buf resid(4 * T * d), out(4 * T * d), idx(4 * T * k), counts(4 * G), offsets(4 * (G + 1));
  Buf row_token(4 * R), slot_row(4 * R), wts(4 * T * A), y_rows(4 * R * d), xn(e * T * d);
  const float* sb = s.router == MOE_ROUTER_SIGMOID_SHARED ? bias.as<float>() : nullptr;
  hipStream_t st = nullptr;

  const int before = moe_stub_launches();
  // The staged entry points, in the order of a layer.
  CHECK_STATUS(moe_route(&cfg, T, x.p, wr.p, sb, off.as<float>(), idx.as<int32_t>(),
                         wts.as<float>(), ws.p, ws_bytes, st),
               MOE_OK);
  CHECK_STATUS(moe_permute(&cfg, T, idx.as<int32_t>(), counts.as<int32_t>(),
                           offsets.as<int32_t>(), row_token.as<int32_t>(),
                           slot_row.as<int32_t>(), ws.p, ws_bytes, st),
               MOE_OK);
  CHECK_STATUS(moe_grouped_swiglu(&cfg, T, x.p, offsets.as<int32_t>(),
                                  row_token.as<int32_t>(), wg.p, wu.p, wd.p,
                                  y_rows.as<float>(), ws.p, ws_bytes, st),
               MOE_OK);
  CHECK_STATUS(moe_combine(&cfg, T, y_rows.as<float>(), slot_row.as<int32_t>(),
                           wts.as<float>(), resid.as<float>(), out.as<float>(), st),
               MOE_OK);
  // The fused layer, with and without the optional outputs and the residual.
  CHECK_STATUS(moe_forward(&cfg, T, x.p, wr.p, sb, nullptr, wg.p, wu.p, wd.p, nullptr,
                           out.as<float>(), nullptr, nullptr, ws.p, ws_bytes, st),
               MOE_OK);
  CHECK_STATUS(moe_forward(&cfg, T, x.p, wr.p, sb, off.as<float>(), wg.p, wu.p, wd.p,
                           resid.as<float>(), out.as<float>(), idx.as<int32_t>(),
                           counts.as<int32_t>(), ws.p, ws_bytes, st),
               MOE_OK);
  // Pre-norm.
  CHECK_STATUS(moe_rmsnorm(&cfg, T, x.p, gain.p, 1e-6f, 1, xn.p, st), MOE_OK);
  CHECK_STATUS(moe_forward_rmsnorm(&cfg, T, x.p, gain.p, 1e-6f, 0, wr.p, sb, nullptr, wg.p,
                                   wu.p, wd.p, nullptr, out.as<float>(), idx.as<int32_t>(),
                                   counts.as<int32_t>(), ws.p, ws_bytes, st),
               MOE_OK);
  if (s.mxfp4) {
    const size_t sgu = packed_scales(E, I, d), sdn = packed_scales(E, d, I);
    Buf qg(E * I * d / 2), qu(E * I * d / 2), qd(E * d * I / 2);
    Buf sg(sgu), su(sgu), sd(sdn), rows_g(E * I * (d / 32)), rows_d(E * d * (I / 32));
    Buf sh_g(2 * S * I * d), sh_u(2 * S * I * d), sh_d(2 * S * d * I);
    void* shg = S ? sh_g.p : nullptr;
    void* shu = S ? sh_u.p : nullptr;
    void* shd = S ? sh_d.p : nullptr;
    CHECK_STATUS(moe_mxfp4_pack_scales(E, I, d, rows_g.as<uint8_t>(), sg.as<uint8_t>(), st),
                 MOE_OK);
    CHECK_STATUS(moe_mxfp4_pack_scales(E, d, I, rows_d.as<uint8_t>(), sd.as<uint8_t>(), st),
                 MOE_OK);
    CHECK_STATUS(moe_grouped_swiglu_mxfp4(&cfg, T, x.p, offsets.as<int32_t>(),
                                          row_token.as<int32_t>(), qg.as<uint8_t>(),
                                          sg.as<uint8_t>(), qu.as<uint8_t>(), su.as<uint8_t>(),
                                          qd.as<uint8_t>(), sd.as<uint8_t>(), shg, shu, shd,
                                          y_rows.as<float>(), ws.p, ws_bytes, st),
                 MOE_OK);
    CHECK_STATUS(moe_forward_mxfp4(&cfg, T, x.p, wr.p, sb, nullptr, qg.as<uint8_t>(),
                                   sg.as<uint8_t>(), qu.as<uint8_t>(), su.as<uint8_t>(),
                                   qd.as<uint8_t>(), sd.as<uint8_t>(), shg, shu, shd,
                                   resid.as<float>(), out.as<float>(), idx.as<int32_t>(),
                                   counts.as<int32_t>(), ws.p, ws_bytes, st),
                 MOE_OK);
  }
  if (moe_stub_launches() == before) {
    std::fprintf(stderr, "%s: no launch reached the stand-ins\n", s.name);
    ++g_fail;
  }

  // Argument checks: each returns before any launch.
  const int pre = moe_stub_launches();
  CHECK_STATUS(moe_forward(&cfg, T, x.p, wr.p, sb, nullptr, wg.p, wu.p, wd.p, nullptr,
                           out.as<float>(), nullptr, nullptr, ws.p, ws_bytes - 1, st),
               MOE_ERR_WORKSPACE);
  CHECK_STATUS(moe_forward(&cfg, T, nullptr, wr.p, sb, nullptr, wg.p, wu.p, wd.p, nullptr,
                           out.as<float>(), nullptr, nullptr, ws.p, ws_bytes, st),
               MOE_ERR_ARG);
  CHECK_STATUS(moe_forward(&cfg, T, x.as<char>() + 8, wr.p, sb, nullptr, wg.p, wu.p, wd.p,
                           nullptr, out.as<float>(), nullptr, nullptr, ws.p, ws_bytes, st),
               MOE_ERR_ARG);
  CHECK_STATUS(moe_route(&cfg, T, x.p, wr.p, sb, nullptr, idx.as<int32_t>(), wts.as<float>(),
                         ws.as<char>() + 16, ws_bytes, st),
               MOE_ERR_ARG);
  CHECK_STATUS(moe_grouped_swiglu(&cfg, T, x.p, offsets.as<int32_t>(),
                                  row_token.as<int32_t>(), wg.p, wu.p, wd.p,
                                  y_rows.as<float>(), ws.p, 0, st),
               MOE_ERR_WORKSPACE);
  CHECK_STATUS(moe_combine(&cfg, T, y_rows.as<float>(), nullptr, wts.as<float>(), nullptr,
                           out.as<float>(), st),
               MOE_ERR_ARG);
  CHECK_STATUS(moe_rmsnorm(&cfg, T, x.p, gain.p, 0.0f, 0, xn.p, st), MOE_ERR_ARG);
  // T = 0 is a no-op before any pointer is looked at.
  CHECK_STATUS(moe_forward(&cfg, 0, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                           nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, 0, st),
               MOE_OK);
  // Token counts past the 32-bit offsets of the kernels.
  size_t big = 0;
  CHECK_STATUS(moe_workspace_size(&cfg, int64_t{1} << 40, &big), MOE_ERR_UNSUPPORTED);
  CHECK_STATUS(moe_workspace_size(&cfg, -1, &big), MOE_ERR_ARG);
  if (moe_stub_launches() != pre) {
    std::fprintf(stderr, "%s: a rejected call launched\n", s.name);
    ++g_fail;
  }
  std::printf("%s: ok (workspace %zu bytes)\n", s.name, ws_bytes);
}

void config_checks() {
  moe_config_t c = config_of({"cfg", 8, 256, 16, 2, 128, 4, MOE_ROUTER_SIGMOID_SHARED,
                              MOE_BF16, false});
  size_t b = 0;
  moe_config_t bad = c;
  bad.top_k = 17;  // k > E
  CHECK_STATUS(moe_workspace_size(&bad, 8, &b), MOE_ERR_ARG);
  bad = c;
  bad.d_model = 200;  // not a multiple of 256
  CHECK_STATUS(moe_workspace_size(&bad, 8, &b), MOE_ERR_UNSUPPORTED);
  bad = c;
  bad.router = 7;
  CHECK_STATUS(moe_workspace_size(&bad, 8, &b), MOE_ERR_ARG);
  bad = c;
  bad.n_shared = 9;
  CHECK_STATUS(moe_workspace_size(&bad, 8, &b), MOE_ERR_UNSUPPORTED);
  bad = c;
  bad.route_scale = -1.0f;
  CHECK_STATUS(moe_workspace_size(&bad, 8, &b), MOE_ERR_ARG);
  CHECK_STATUS(moe_workspace_size(nullptr, 8, &b), MOE_ERR_ARG);
  CHECK_STATUS(moe_workspace_size(&c, 8, nullptr), MOE_ERR_ARG);
  CHECK_STATUS(moe_mxfp4_scales_bytes(4, 100, 256, &b), MOE_ERR_UNSUPPORTED);
  if (moe_status_str(static_cast<moe_status_t>(99)) == nullptr) ++g_fail;
}

}  // namespace

int main() {
  const Shape shapes[] = {
      {"sigmoid_bf16", 300, 512, 40, 2, 256, 6, MOE_ROUTER_SIGMOID_SHARED, MOE_BF16, true},
      {"softmax_bf16", 257, 768, 64, 0, 384, 8, MOE_ROUTER_SOFTMAX_TOPK, MOE_BF16, true},
      {"softmax_bf16_ungated_shared", 100, 512, 32, 1, 256, 4, MOE_ROUTER_SOFTMAX_TOPK,
       MOE_BF16, true},
      {"sigmoid_f32", 100, 256, 20, 3, 128, 4, MOE_ROUTER_SIGMOID_SHARED, MOE_F32, false},
      {"softmax_f32_one_token", 1, 256, 16, 0, 128, 2, MOE_ROUTER_SOFTMAX_TOPK, MOE_F32,
       false},
      {"max_experts", 64, 256, 1016, 8, 128, 32, MOE_ROUTER_SIGMOID_SHARED, MOE_BF16, false},
      // the Inkling widths (d 6,144, I 3,072) at the decode batch, with few experts: the
      // router's 24-way K split and the widest rows
      {"inkling_widths_decode", 32, 6144, 2, 2, 3072, 2, MOE_ROUTER_SIGMOID_SHARED, MOE_BF16,
       true},
  };
  config_checks();
  for (const Shape& s : shapes) run_shape(s);
  if (g_fail != 0) {
    std::fprintf(stderr, "%d check(s) failed\n", g_fail);
    return 1;
  }
  std::printf("all shapes ok, %d stand-in launches\n", moe_stub_launches());
  return 0;
}
