// switch_moe_forward without a caller workspace, for callers that cannot
// allocate device memory (code under HIP graph capture, tight serving loops,
// harnesses that forbid hipMalloc).  The forward's workspace (router
// partials, slot lists, the hidden matrix, the expert outputs) lives in one
// file-scope device array of kNoAllocScratchBytes, which every GPU the
// library runs on holds from the first use of this code object until the
// process ends.  The array's device address is looked up once per device,
// with that device current, and only that address reaches the kernels: in
// host code the array's name is a host-side stand-in, not a device pointer.
//
// Nothing in that workspace has to start at zero (every kernel of the
// forward writes what it later reads), so no clearing is enqueued.  All
// calls on one GPU share its array: calls that overlap on one GPU (two
// streams, two threads) race on it and must be serialised by the caller.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <mutex>

#include "kernels.hpp"
#include "switch_moe.h"

namespace {

constexpr size_t kNoAllocScratchBytes = (size_t)64 << 20;  // 64 MiB
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

std::mutex g_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// device address of `scratch` on the current device (looked up once per device)
switch_status scratch_on_current_device(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    char msg[160];
    snprintf(msg, sizeof(msg), "switch_moe_forward_noalloc: hipGetDevice: %s", hipGetErrorString(e));
    return swm::abi_fail(SWITCH_E_HIP, msg);
  }
  if (dev < 0 || dev >= kMaxDevices) return swm::abi_fail(SWITCH_E_UNSUPPORTED, "device index beyond 63");
  std::lock_guard<std::mutex> lock(g_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr) {
      char msg[160];
      snprintf(msg, sizeof(msg), "switch_moe_forward_noalloc: hipGetSymbolAddress: %s", hipGetErrorString(e));
      return swm::abi_fail(SWITCH_E_HIP, msg);
    }
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return SWITCH_OK;
}

}  // namespace

extern "C" {

size_t switch_moe_noalloc_max_bytes(void) { return kNoAllocScratchBytes; }

switch_status switch_moe_forward_noalloc(const switch_moe_desc* desc, const switch_moe_inputs* in,
                                         const switch_moe_outputs* out, void* stream) {
  size_t need = 0;
  switch_status s = swm::abi_forward_bytes(desc, &need);
  if (s != SWITCH_OK) return s;
  if (need > kNoAllocScratchBytes) {
    char msg[200];
    snprintf(msg, sizeof(msg),
             "switch_moe_forward_noalloc: the layer needs %zu bytes of workspace, beyond the %zu-byte scratch array "
             "(use switch_moe_forward with a workspace)",
             need, kNoAllocScratchBytes);
    return swm::abi_fail(SWITCH_E_WORKSPACE, msg);
  }
  void* ws = nullptr;
  s = scratch_on_current_device(&ws);
  if (s != SWITCH_OK) return s;
  return swm::abi_forward(desc, in, out, ws, kNoAllocScratchBytes, stream);
}

}  // extern "C"
