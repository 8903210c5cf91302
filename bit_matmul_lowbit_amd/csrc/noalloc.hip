// Decode GEMV that allocates nothing (lowbit_gemv_noalloc): the same two
// kernels as lowbit_gemv -- prepare x, then stream the weights -- with the
// scratch they share (a copy of x for b <= 2, x in matrix-core operand
// order for b >= 3) in a static device array instead of a caller-provided
// workspace.  For callers that cannot allocate device memory.
//
// Each GPU holds its own copy of `scratch` at its own address until the
// process ends.  In host code the array's name is only a host-side stand-in,
// so its device address is looked up with hipGetSymbolAddress on the first
// call on each device (with that device current) and kept per device; the
// kernels get that address as their workspace argument.  Every call on a
// GPU shares that GPU's array: calls that overlap on one GPU (different
// streams, or different host threads) race.  Nothing in it must start at
// zero: the prepare kernel overwrites every byte the accumulate kernel
// reads, and zeroes y itself.
#include "common.h"

#include <atomic>
#include <mutex>

namespace lowbit {
namespace {

constexpr size_t kScratchBytes = size_t(1) << 20;  // 1 MiB per device

__device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_addr[kMaxDevices];
std::mutex g_scratch_mu;

// Device address of the current device's `scratch`, looked up once per device.
hipError_t scratch_addr(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void* p = g_scratch_addr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_addr[dev].load(std::memory_order_relaxed);
    if (p == nullptr) {
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return e;
      if (p == nullptr) return hipErrorInvalidSymbol;
      g_scratch_addr[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return hipSuccess;
}

}  // namespace

size_t gemv_noalloc_scratch_bytes() { return kScratchBytes; }

hipError_t launch_gemv_noalloc(int fmt, const uint8_t* codes, const uint16_t* scales, int64_t n,
                               int64_t k, const uint16_t* x, int64_t b, float* y,
                               hipStream_t st) {
  // small matrices need no scratch at all
  if (gemv_direct_ok(n, k, b)) return launch_gemv_direct(fmt, codes, scales, n, k, x, b, y, st);
  void* ws = nullptr;
  hipError_t e = scratch_addr(&ws);
  if (e != hipSuccess) return e;
  e = launch_gemv_prepare(n, k, x, b, y, ws, st);
  if (e != hipSuccess) return e;
  return launch_gemv_accumulate(fmt, codes, scales, n, k, b, y, ws, st);
}

}  // namespace lowbit
