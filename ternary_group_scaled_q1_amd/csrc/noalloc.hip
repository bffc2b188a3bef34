// Decode GEMV for callers that cannot allocate: the workspace of gemv_lowbit
// (arrival counters and K-range partial sums) lives in a file-scope device
// array of the library instead of a caller's buffer.
//
// In host code `scratch` names a host-side stand-in, not device memory: the
// array's device address on each GPU comes from hipGetSymbolAddress (every
// device holds its own copy at its own address), looked up once per device
// with that device current and kept in a table.  Only that address is ever
// handed to a kernel.  The counters must be zero before a call; every call
// leaves them at zero again, and the first call on a device clears them with
// a fill kernel (no memset node, so the call may also be captured in a graph).
// All calls on one device share its array: calls that may overlap in time on
// one device (two streams, two host threads) race on it.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/lowbit.h"
#include "kernels.hpp"

namespace lowbit {

namespace {

// The largest workspace any decode call asks for: 32 KiB of arrival counters
// plus at most 8 MiB of partial sums (gemv_split.hip).
constexpr int64_t kCounterBytes = 32 << 10;
constexpr int64_t kScratchBytes = kCounterBytes + (int64_t(8) << 20);

static __device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void *g_ptr[kMaxDevices] = {};
bool g_cleared[kMaxDevices] = {};

// The array's device address on the current device (nullptr on failure).
void *scratch_ptr(int dev) {
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_ptr[dev]) {
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
    g_ptr[dev] = p;
  }
  return g_ptr[dev];
}

}  // namespace

int64_t noalloc_scratch_bytes() { return kScratchBytes; }

// Returns a LOWBIT_* status.  The caller has validated every argument.
int gemv_noalloc(const LaunchArgs &in) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return LOWBIT_ERR_DEVICE;
  void *ptr = scratch_ptr(dev);
  if (!ptr) return LOWBIT_ERR_DEVICE;
  {
    std::lock_guard<std::mutex> lk(g_mu);
    if (!g_cleared[dev]) {
      if (launch_fill_zero(ptr, kCounterBytes, in.stream) != hipSuccess) return LOWBIT_ERR_DEVICE;
      g_cleared[dev] = true;
    }
  }
  LaunchArgs a = in;
  a.ws = ptr;
  a.ws_bytes = kScratchBytes;
  return launch_gemv(a) == hipSuccess ? LOWBIT_OK : LOWBIT_ERR_DEVICE;
}

}  // namespace lowbit
