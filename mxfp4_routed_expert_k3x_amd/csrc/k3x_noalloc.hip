// The expert forward for callers that cannot allocate device memory: k3x_moe_forward with its
// workspace in a scratch array built into the library instead of a caller's buffer.
//
// The array is a file-scope device variable, so every GPU the library runs on holds its own
// copy from module load until the process ends.  Host code never passes the array's name to
// a kernel (on the host it only stands for the symbol): the first call on each device looks
// up that device's copy with hipGetSymbolAddress, with the device current, and every later
// call uses the recorded address.
#include <mutex>

#include "k3x_internal.h"

namespace {

__device__ __align__(256) uint8_t scratch[K3X_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
uint8_t* g_scratch[kMaxDevices] = {};

// The current device's copy of the scratch array (looked up once per device).
hipError_t scratch_of_current_device(uint8_t** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch[dev] = static_cast<uint8_t*>(p);
  }
  *out = g_scratch[dev];
  return hipSuccess;
}

}  // namespace

extern "C" k3x_status k3x_moe_forward_noalloc(const k3x_pool* p, const void* x_bf16, int32_t T,
                                              const int32_t* idx, const float* gates,
                                              int32_t topk, float* y, int64_t* drops_out,
                                              void* stream) {
  if (!p) return k3x::fail_status(K3X_E_INVALID_ARG, "moe_forward_noalloc: NULL pool");
  if (T < 0 || topk < 1 || topk > 64)
    return k3x::fail_status(K3X_E_INVALID_ARG, "moe_forward_noalloc: T %d or topk %d out of range",
                            T, topk);
  const size_t need = k3x_moe_workspace_size(p, T, topk);
  if (need == 0)
    return k3x::fail_status(K3X_E_UNSUPPORTED, "moe_forward_noalloc: T %d x topk %d not supported",
                            T, topk);
  if (need > K3X_NOALLOC_SCRATCH_BYTES)
    return k3x::fail_status(K3X_E_UNSUPPORTED,
                            "moe_forward_noalloc: T %d x topk %d needs %zu bytes of scratch; the "
                            "built-in scratch holds %zu (use k3x_moe_forward with a workspace)",
                            T, topk, need, (size_t)K3X_NOALLOC_SCRATCH_BYTES);
  if (drops_out && reinterpret_cast<uintptr_t>(drops_out) % 8)
    return k3x::fail_status(K3X_E_INVALID_ARG, "moe_forward_noalloc: drops_out not 8-byte aligned");
  uint8_t* ws = nullptr;
  hipError_t e = scratch_of_current_device(&ws);
  if (e != hipSuccess) return k3x::hip_status(e, "moe_forward_noalloc: scratch address");
  const k3x_status st = k3x_moe_forward(p, x_bf16, T, idx, gates, topk, y, ws,
                                        K3X_NOALLOC_SCRATCH_BYTES, stream);
  if (st != K3X_OK || !drops_out) return st;
  // the drop counter is the first 8 bytes of the workspace on every path
  e = hipMemcpyAsync(drops_out, ws, sizeof(int64_t), hipMemcpyDeviceToDevice, (hipStream_t)stream);
  if (e != hipSuccess) return k3x::hip_status(e, "moe_forward_noalloc: drop count copy");
  return K3X_OK;
}
