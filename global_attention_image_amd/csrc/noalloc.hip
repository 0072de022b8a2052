// uhla_forward_noalloc: the forward for callers that cannot allocate device memory (code
// under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).  Its
// scratch memory is a fixed array in the library's device code instead of a caller
// workspace; it calls no allocating routine.
#include <stdio.h>

#include <atomic>
#include <mutex>

#include "uhla_internal.h"

namespace uhla {

// One array per GPU, held for the life of the process and shared by every call on that
// GPU (calls that overlap on one GPU race; each call rewrites every byte it reads).  In host
// code the array's name is not a device address: the address comes from
// hipGetSymbolAddress, once per device with that device current, and only that address is
// ever handed to a kernel.
constexpr size_t kScratchBytes = size_t(64) << 20;
constexpr int kMaxDevices = 64;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

static std::atomic<void*> g_scratch_ptr[kMaxDevices];
static std::mutex g_scratch_mu;

// Device address of the current device's scratch array (looked up on the first call on
// that device).
static int scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return (set_hip_detail("hipGetDevice", e), UHLA_ERR_HIP);
  if (dev < 0 || dev >= kMaxDevices) return fail_unsupported("device index above 63");
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (!p) {
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e == hipSuccess && !p) e = hipErrorInvalidSymbol;
      if (e != hipSuccess) return (set_hip_detail("hipGetSymbolAddress(scratch)", e), UHLA_ERR_HIP);
      g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return UHLA_OK;
}

}  // namespace uhla

extern "C" int uhla_forward_noalloc(const void* q, const void* k, const void* v, void* o, int B,
                                    int H, int W, int w, int H_lr, int W_lr, int rho, int heads,
                                    int head_dim, float scale, float theta, void* stream) {
  using namespace uhla;
  // argument errors first, with no device call
  int st = validate_forward(q, k, v, o, B, 0, H, W, w, H_lr, W_lr, rho, heads, head_dim, 1, 0);
  if (st) return st;
  const size_t need = workspace_bytes(B, 0, H, W, w, H_lr, W_lr, rho, heads, head_dim, 1, 0);
  if (need > kScratchBytes) {
    char msg[192];
    snprintf(msg, sizeof(msg),
             "needs %zu bytes of scratch, above the %zu-byte static scratch of uhla_forward_noalloc",
             need, kScratchBytes);
    set_detail(msg);
    return UHLA_ERR_WORKSPACE;
  }
  void* ws = nullptr;
  st = scratch_address(&ws);
  if (st) return st;
  return forward_impl(q, k, v, o, B, 0, H, W, w, H_lr, W_lr, rho, heads, head_dim, scale, theta,
                      1, 0, ws, kScratchBytes, stream, nullptr);
}
