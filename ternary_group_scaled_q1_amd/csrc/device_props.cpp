// Per-device properties used to size persistent grids; filled lazily and
// protected by a mutex (the only mutable state of the library).
#include <hip/hip_runtime.h>

#include <map>
#include <mutex>
#include <tuple>

#include "kernels.hpp"

namespace lowbit {

namespace {
std::mutex g_mu;
std::map<int, int> g_cus;
std::map<std::tuple<const void *, int, int, int>, int> g_blocks;

int current_device() {
  int d = 0;
  if (hipGetDevice(&d) != hipSuccess) d = 0;
  return d;
}
}  // namespace

int num_cus() {
  const int dev = current_device();
  std::lock_guard<std::mutex> lk(g_mu);
  auto it = g_cus.find(dev);
  if (it != g_cus.end()) return it->second;
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
  g_cus[dev] = n;
  return n;
}

int resident_blocks(const void *kernel, int threads, int lds) {
  const int dev = current_device();
  const auto key = std::make_tuple(kernel, threads, lds, dev);
  {
    std::lock_guard<std::mutex> lk(g_mu);
    auto it = g_blocks.find(key);
    if (it != g_blocks.end()) return it->second;
  }
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kernel, threads, size_t(lds)) != hipSuccess || n <= 0) n = 1;
  std::lock_guard<std::mutex> lk(g_mu);
  g_blocks[key] = n;
  return n;
}

}  // namespace lowbit
