// Scratch memory of the allocation-free entry point (swattn_decode_noalloc): a fixed
// array in device memory that holds the decode's per-split partials, for callers
// that cannot allocate (code under stream capture, serving loops that forbid
// allocation).  Each GPU the library runs on holds its own copy of the array until
// the process ends.
//
// In host code the array's name is not a device address: its address on a device is
// looked up once per device (with that device current) and kept; only that address
// is handed to kernels.
#include <atomic>
#include <mutex>

#include "launch.h"

namespace swattn {

static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::atomic<void *> g_scratch[kMaxDevices];
std::mutex g_lookup;
}  // namespace

void *noalloc_scratch(int device) {
  if (device < 0 || device >= kMaxDevices) return nullptr;
  void *p = g_scratch[device].load(std::memory_order_acquire);
  if (p != nullptr) return p;
  std::lock_guard<std::mutex> lock(g_lookup);
  p = g_scratch[device].load(std::memory_order_relaxed);
  if (p == nullptr) {
    // the caller made `device` current
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
    g_scratch[device].store(p, std::memory_order_release);
  }
  return p;
}

}  // namespace swattn
