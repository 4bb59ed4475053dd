// Device scratch of the entry point that allocates nothing
// (psw_append_attention_noalloc): a file-scope device array, one copy per
// GPU, held for the life of the process.  It stands in for the caller's
// workspace (plan ints, split-KV records and outputs) for callers that
// cannot allocate device memory.
//
// On the host the array's name is only a stand-in for its symbol, not a
// device address: the address of each GPU's copy is looked up once per
// device, with that device current, and every kernel argument uses that
// address.
#include <hip/hip_runtime.h>

#include <mutex>

#include "device.h"

namespace psw {
namespace {

static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};

}  // namespace

int scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return static_cast<int>(e);
  if (dev < 0 || dev >= kMaxDevices) return static_cast<int>(hipErrorInvalidDevice);
  std::lock_guard<std::mutex> lock(g_mu);
  if (g_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return static_cast<int>(e);
    if (p == nullptr) return static_cast<int>(hipErrorInvalidSymbol);
    g_ptr[dev] = p;
  }
  *out = g_ptr[dev];
  return 0;
}

}  // namespace psw
