// Static device scratch for the chunk-rule entry point that allocates nothing
// (gdn_chunk_rule_fwd_noalloc): the per-(chunk, value head) records and the
// chunk offsets of packed sequences live in a file-scope device array of
// GDN_NOALLOC_SCRATCH_BYTES instead of a caller workspace.
//
// In host code `scratch` names a host-side stand-in, not device memory, so it
// is never passed to a kernel or a copy: its device address is looked up once
// per device (with that device current) by hipGetSymbolAddress and kept per
// device. Each device holds its own copy of the array, at its own address,
// from the module's load until the process ends. Every call on one device
// shares that device's array; calls that overlap on one device race.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/gdn.h"
#include "gdn_internal.h"

namespace gdn {
namespace {

static __device__ __align__(256) unsigned char scratch[GDN_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void *g_ptr[kMaxDevices];

}  // namespace

hipError_t static_scratch(void **out) {
  *out = nullptr;
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_ptr[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p || (uintptr_t)p % 256) return hipErrorInvalidSymbol;
    g_ptr[dev] = p;
  }
  *out = g_ptr[dev];
  return hipSuccess;
}

}  // namespace gdn
