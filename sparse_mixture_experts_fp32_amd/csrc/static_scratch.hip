// moe_forward_static: the whole layer with its scratch space in a static device array of
// the library instead of a caller workspace, for callers that cannot allocate device
// memory (code under graph capture, tight serving loops, harnesses that forbid it).
//
// The array `scratch` below is the workspace moe_forward would take: router partial
// logits, the routing and grouping buffers, the m-tile plan with its counters, the SwiGLU
// intermediate and the per-row expert outputs.  Each GPU the library runs on holds its own
// copy until the process ends.  Its device address is looked up once per device, with that
// device current, by hipGetSymbolAddress; host code never passes the array's own name to a
// kernel or a copy (in host code that name is a host-side stand-in, not a device address).
//
// The kernels rebuild every counter and plan they read within the call (the plan kernel
// clears the counters), so the contents a previous call left behind change nothing.
#include <atomic>
#include <mutex>

#include "moe.h"
#include "moe_launch.h"

namespace {

constexpr size_t kScratchBytes = MOE_STATIC_SCRATCH_BYTES;
static_assert(kScratchBytes % 256 == 0, "scratch size must keep 256-byte alignment");

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];   // device address of `scratch` per device
std::mutex g_init;

// Device address of the current device's copy of `scratch`, looked up on the first call
// on that device.  MOE_ERR_HIP if the device or the symbol cannot be resolved.
moe_status_t scratch_of_current_device(void** ptr) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return MOE_ERR_HIP;
  if (dev >= kMaxDevices) return MOE_ERR_UNSUPPORTED;
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    std::lock_guard<std::mutex> lock(g_init);
    p = g_scratch[dev].load(std::memory_order_relaxed);
    if (p == nullptr) {
      void* addr = nullptr;
      if (hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch)) != hipSuccess || addr == nullptr) {
        (void)hipGetLastError();
        return MOE_ERR_HIP;
      }
      if ((reinterpret_cast<uintptr_t>(addr) & 255u) != 0) return MOE_ERR_HIP;
      p = addr;
      g_scratch[dev].store(p, std::memory_order_release);
    }
  }
  *ptr = p;
  return MOE_OK;
}

}  // namespace

extern "C" moe_status_t moe_forward_static(const moe_config_t* cfg, int64_t T, const void* x,
                                           const void* w_router, const float* sel_bias,
                                           const float* logit_offset, const void* w_gate,
                                           const void* w_up, const void* w_down,
                                           const float* residual, float* out,
                                           int32_t* topk_idx_out, int32_t* counts_out,
                                           hipStream_t stream) {
  size_t need = 0;
  const moe_status_t st = moe::check_forward_args(cfg, T, x, w_router, sel_bias, w_gate,
                                                  w_up, w_down, residual, out, &need);
  if (st != MOE_OK) return st;
  if (T == 0) return MOE_OK;
  if (need > kScratchBytes) return MOE_ERR_WORKSPACE;
  void* ws = nullptr;
  const moe_status_t sp = scratch_of_current_device(&ws);
  if (sp != MOE_OK) return sp;
  return moe_forward(cfg, T, x, w_router, sel_bias, logit_offset, w_gate, w_up, w_down,
                     residual, out, topk_idx_out, counts_out, ws, kScratchBytes, stream);
}
