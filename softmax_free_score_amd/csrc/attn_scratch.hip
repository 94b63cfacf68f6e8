// attn_scratch.hip -- the device scratch of attn_fwd_noalloc.
//
// One file-scope device array per GPU the library runs on, of a fixed size
// (ATTN_NOALLOC_SCRATCH_BYTES), held until the process ends.  In host code
// the array's name is only a host-side stand-in for the symbol; its device
// address comes from hipGetSymbolAddress, taken once per device with that
// device current, and that address is what the launches use.
#include <hip/hip_runtime.h>

#include <mutex>

#include "attn_launch.h"
#include "sfs_attn.h"

namespace sfs {
namespace {

static __device__ __align__(256) unsigned char scratch[ATTN_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

}  // namespace

hipError_t scratch_address(void** ptr) {
  *ptr = nullptr;
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace sfs
