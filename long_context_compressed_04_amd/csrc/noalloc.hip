// csa_decode_noalloc: the fused decode step with its workspace in a device-resident
// array of the library, for callers that cannot allocate device memory (declared and
// documented in include/csa.h).
//
// `scratch` lives in the library's code object: every GPU the library runs on gets
// its own copy, at its own address, from the first use on that device until the
// process ends.  In host code the array's name is only a host-side stand-in, so its
// device address is looked up once per device (hipGetSymbolAddress, with that device
// current) and only that address is ever handed to kernels.
#include <hip/hip_runtime.h>

#include <mutex>

#include "csa.h"
#include "csa_kernels.hpp"
#include "validate.hpp"

namespace {

constexpr size_t kScratchBytes = CSA_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The device address of this device's scratch array (looked up on first use).
csa_status scratch_ptr(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return csa::fail(CSA_ERR_HIP, "csa_decode_noalloc: hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return csa::fail(CSA_ERR_UNSUPPORTED, "csa_decode_noalloc: device %d beyond the %d the library tracks", dev,
                         kMaxDevices);
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return csa::fail(CSA_ERR_HIP, "csa_decode_noalloc: hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return CSA_OK;
}

}  // namespace

extern "C" csa_status csa_decode_noalloc(const csa_decode_args* a, void* stream) {
  if (!a) return csa::fail(CSA_ERR_NULL, "csa_decode_noalloc: args is NULL");
  const size_t need = csa_decode_workspace_size(a);
  if (need > kScratchBytes)
    return csa::fail(CSA_ERR_WORKSPACE,
                         "csa_decode_noalloc: this step needs %zu bytes of workspace; the scratch array holds %zu "
                         "(use csa_decode with a workspace of your own)",
                         need, kScratchBytes);
  void* ws = nullptr;
  csa_status st = scratch_ptr(&ws);
  if (st != CSA_OK) return st;
  // The array keeps the previous call's contents.  No part of it needs clearing: the
  // decode step's kernels write every workspace byte they read (score rows, top-k
  // candidate lists, split partials) before reading it, and keep no counters there.
  return csa_decode(a, ws, kScratchBytes, stream);
}
