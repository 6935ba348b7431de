// The layer forward for callers that cannot allocate device memory (code under
// HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
// the same kernels as moe_expert_forward, with the workspace taken from a
// fixed-size array that the library's code object holds on each device.
//
// In host code the array's name is only a host-side stand-in, so its device
// address is looked up once per device (with that device current) through
// hipGetSymbolAddress and kept; every use below goes through that pointer.
// All calls on one device share the array, which keeps the last call's
// contents: nothing in the forward relies on it starting at zero (the decode
// exchange tags its values per launch), and calls that overlap in time on
// one device race on it.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <mutex>

#include "../../include/nf4moe.h"
#include "launch.h"

namespace {

static __device__ __align__(256) unsigned char scratch[NF4MOE_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The device address of `scratch` on the current device (looked up once).
int scratch_for_current_device(void** out) {
  int dev = 0;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess)
    return nf4moe::report_error(NF4MOE_EHIP, "hipGetDevice: %s", hipGetErrorString(err));
  if (dev < 0 || dev >= kMaxDevices)
    return nf4moe::report_error(NF4MOE_EINVAL, "device %d outside the %d the scratch table covers",
                                dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (err != hipSuccess || p == nullptr)
      return nf4moe::report_error(NF4MOE_EHIP, "hipGetSymbolAddress(scratch) on device %d: %s",
                                  dev, hipGetErrorString(err));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return NF4MOE_OK;
}

}  // namespace

extern "C" int moe_expert_forward_noalloc(
    const void* x, int x_dtype, const float* router_logits, int64_t T, int H, int I, int E,
    int k, int renormalize, const uint8_t* gu_packed, const float* gu_absmax,
    const uint8_t* dn_packed, const float* dn_absmax, const nf4moe_lora* gu_lora,
    const nf4moe_lora* dn_lora, void* y, int y_dtype, void* stream) {
  // argument errors first, exactly as the forward reports them: given no
  // workspace it validates everything, launches nothing and, when the
  // arguments are good, answers EWORKSPACE
  int st = moe_expert_forward(x, x_dtype, router_logits, T, H, I, E, k, renormalize,
                              gu_packed, gu_absmax, dn_packed, dn_absmax, gu_lora, dn_lora, y,
                              y_dtype, nullptr, 0, stream);
  if (st != NF4MOE_EWORKSPACE) return st;
  const int r = std::max(gu_lora ? gu_lora->r : 0, dn_lora ? dn_lora->r : 0);
  const size_t need = moe_expert_forward_workspace(T, H, I, E, k, r);
  if (need > (size_t)NF4MOE_NOALLOC_SCRATCH_BYTES)
    return nf4moe::report_error(
        NF4MOE_EWORKSPACE,
        "the allocation-free forward holds %zu bytes of scratch per device; T=%lld, H=%d, "
        "I=%d, E=%d, k=%d, adapter rank %d need %zu (use moe_expert_forward with a workspace)",
        (size_t)NF4MOE_NOALLOC_SCRATCH_BYTES, (long long)T, H, I, E, k, r, need);
  void* ws = nullptr;
  st = scratch_for_current_device(&ws);
  if (st != NF4MOE_OK) return st;
  return moe_expert_forward(x, x_dtype, router_logits, T, H, I, E, k, renormalize, gu_packed,
                            gu_absmax, dn_packed, dn_absmax, gu_lora, dn_lora, y, y_dtype, ws,
                            (size_t)NF4MOE_NOALLOC_SCRATCH_BYTES, stream);
}
