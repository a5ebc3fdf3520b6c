// ra_noalloc.hip -- the device-resident workspace behind ra_attn_fwd_noalloc.
//
// For callers that cannot allocate (code under HIP graph capture, tight
// serving loops): the workspace the forward pass needs (Q/K/V codes, scales,
// per-channel V maxima) lives in one file-scope device array of a fixed
// size.  Every GPU the library runs on holds its own copy, at its own
// address, until the process ends.  Host code must never pass the array's
// name to a kernel (in host code it is only a stand-in): its device address
// is looked up once per device with hipGetSymbolAddress and kept here.
#include <map>
#include <mutex>

#include "ra_attn.h"
#include "ra_kernels.h"

static __device__ __align__(256) uint8_t scratch[RA_NOALLOC_WORKSPACE_BYTES];

static std::mutex g_mu;
static std::map<int, void*> g_ptr;   // device -> address of that device's scratch

namespace ra {

// Device address of the current device's scratch array (looked up on the
// first call per device, with that device current).  hipSuccess or the
// error of hipGetDevice / hipGetSymbolAddress.
hipError_t noalloc_scratch(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> g(g_mu);
  auto it = g_ptr.find(dev);
  if (it != g_ptr.end()) {
    *ptr = it->second;
    return hipSuccess;
  }
  void* p = nullptr;
  e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
  if (e != hipSuccess) return e;
  g_ptr[dev] = p;
  *ptr = p;
  return hipSuccess;
}

}  // namespace ra
