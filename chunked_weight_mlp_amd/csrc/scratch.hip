// Fixed device scratch area for callers that cannot allocate device memory
// (code under stream capture, tight serving loops, harnesses that forbid
// hipMalloc): ipttt_prefill_layer_noalloc runs the prefill with its workspace
// in this array instead of the descriptor's workspace.
//
// The array is a file-scope __device__ object: every device the library runs
// on holds its own copy (kScratchBytes) until the process ends. In host code
// its name is only a host-side handle for the symbol, not a device address;
// the device address is looked up once per device with hipGetSymbolAddress
// (with that device current) and kept here, and every host use of the memory
// goes through that address.
#include <atomic>
#include <mutex>

#include "internal.h"

static __device__ __align__(256) unsigned char scratch[ipttt::kScratchBytes];

namespace ipttt {
namespace {

constexpr int kMaxDevices = 64;
std::atomic<void *> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

}  // namespace

hipError_t scratch_setup(void **out) {
  *out = nullptr;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void *p = g_scratch[dev].load(std::memory_order_acquire);
  if (p) {
    *out = p;
    return hipSuccess;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  p = g_scratch[dev].load(std::memory_order_relaxed);
  if (!p) {
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p || ((uintptr_t)p & 255u)) return hipErrorInvalidSymbol;
    g_scratch[dev].store(p, std::memory_order_release);
  }
  *out = p;
  return hipSuccess;
}

}  // namespace ipttt
