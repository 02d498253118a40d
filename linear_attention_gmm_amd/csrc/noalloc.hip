// noalloc.hip -- fixed device scratch for gma_forward_noalloc, the variant of
// gma_forward that allocates nothing (for callers that cannot call hipMalloc:
// code under graph capture, tight serving loops).
//
// The scratch is one file-scope device array, so every GPU the library runs on
// holds its own copy from module load until the process ends. Host code never
// passes the array's name to a kernel (on the host that name is a stand-in,
// not a device address): the device address is looked up once per device with
// hipGetSymbolAddress, with that device current, and that address is what the
// kernels receive as their workspace. Every call on one GPU shares the array,
// so calls that overlap in time on one GPU race; nothing in it has to start at
// zero (the kernels write every word they later read).
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>

#include "launch.hpp"

namespace lm {
namespace {

static __device__ __align__(256) char scratch[kNoallocScratchBytes];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_addr[kMaxDevices];
std::mutex g_mu;

}  // namespace

hipError_t noalloc_scratch(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void* p = g_addr[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_mu);
    p = g_addr[dev].load(std::memory_order_relaxed);
    if (!p) {
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return e;
      if (!p) return hipErrorInvalidSymbol;
      g_addr[dev].store(p, std::memory_order_release);
    }
  }
  *ptr = p;
  return hipSuccess;
}

}  // namespace lm
