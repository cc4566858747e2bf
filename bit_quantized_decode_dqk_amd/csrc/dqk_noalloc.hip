// Device scratch of the decode entry point that allocates nothing
// (dqk_decode_attention_noalloc): the split partials go to a file-scope device
// array instead of a caller's workspace.  Each GPU the library runs on holds
// its own copy of the array, from module load until the process ends; its
// device address is looked up once per device, with that device current, and
// kept.  Nothing in it needs to start at zero: every decode writes each partial
// it later reads.  Calls that overlap on one GPU share the array and race.
#include <atomic>
#include <mutex>

#include "dqk_internal.h"

namespace dqk {

static __device__ __align__(256) float scratch[kScratchBytes / sizeof(float)];

namespace {

constexpr int kMaxDevices = 64;
std::atomic<float *> scratch_at[kMaxDevices];   // per device: the array's address, null until looked up
std::mutex lookup_mu;

}  // namespace

hipError_t decode_scratch(float **ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  float *p = scratch_at[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(lookup_mu);
    p = scratch_at[dev].load(std::memory_order_relaxed);
    if (!p) {
      void *addr = nullptr;
      // the host-side name of the array is not a device address: only the
      // address looked up here is ever passed to a kernel
      e = hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return e;
      if (!addr) return hipErrorInvalidSymbol;
      p = static_cast<float *>(addr);
      scratch_at[dev].store(p, std::memory_order_release);
    }
  }
  *ptr = p;
  return hipSuccess;
}

}  // namespace dqk
