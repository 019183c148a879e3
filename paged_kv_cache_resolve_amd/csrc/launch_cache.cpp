// Per-device launch sizing for the persistent decode kernels, cached so that
// a decode call does not query the runtime every time.

#include <stdlib.h>

#include <atomic>
#include <mutex>
#include <unordered_map>

#include "internal.h"

namespace pagedkv {

namespace {

struct Key {
  int dev;
  const void* fn;
  int threads;
  size_t lds;
  bool operator==(const Key& o) const {
    return dev == o.dev && fn == o.fn && threads == o.threads && lds == o.lds;
  }
};
struct KeyHash {
  size_t operator()(const Key& k) const {
    return std::hash<const void*>()(k.fn) ^ (size_t)k.dev * 0x9e3779b97f4a7c15ull ^
           (size_t)k.threads * 1315423911u ^ k.lds * 2654435761u;
  }
};

std::mutex g_mu;
std::unordered_map<Key, int, KeyHash> g_blocks;   // resident workgroups per device

}  // namespace

// Workgroups of `threads` threads using `lds` bytes of dynamic LDS that the
// whole device holds at once (CUs x resident workgroups per CU).
hipError_t resident_workgroups(const void* fn, int threads, size_t lds, int* out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const Key key{dev, fn, threads, lds};
  {
    std::lock_guard<std::mutex> lock(g_mu);
    auto it = g_blocks.find(key);
    if (it != g_blocks.end()) {
      *out = it->second;
      return hipSuccess;
    }
  }
  int cus = 0, per_cu = 0;
  e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, threads, lds);
  if (e != hipSuccess) return e;
  if (per_cu < 1) per_cu = 1;
  const int total = cus * per_cu;
  std::lock_guard<std::mutex> lock(g_mu);
  g_blocks[key] = total;
  *out = total;
  return hipSuccess;
}

namespace {
constexpr int kMaxDevices = 64;
std::atomic<int> g_cus[kMaxDevices];   // CU count per device, 0 = not yet queried
}  // namespace

// CUs of the current device (0 if the runtime cannot tell), queried once.
int device_cus() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (dev < 0 || dev >= kMaxDevices) {
    int cus = 0;
    return hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess
               ? cus : 0;
  }
  int cus = g_cus[dev].load(std::memory_order_relaxed);
  if (cus == 0) {
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      return 0;
    g_cus[dev].store(cus, std::memory_order_relaxed);
  }
  return cus;
}

int decode_workgroups(int resident) {
#ifdef PAGEDKV_LAUNCH_SWEEP
  // Launch-shape sweeps only: a library built with -DPAGEDKV_LAUNCH_SWEEP
  // reads the workgroups per CU from PAGEDKV_DECODE_WG_PER_CU.  The normal
  // build has no such override.
  static const int per_cu = [] {
    const char* v = getenv("PAGEDKV_DECODE_WG_PER_CU");
    const int x = v ? atoi(v) : 0;
    return x > 0 ? x : kDecodeWgPerCu;
  }();
#else
  constexpr int per_cu = kDecodeWgPerCu;
#endif
  const int cus = device_cus();
  if (cus <= 0) return resident;
  const int want = cus * per_cu;
  int n = want < resident ? want : resident;
  if (n > kMaxWaves / 4) n = kMaxWaves / 4;
  return n < 1 ? 1 : n;
}

}  // namespace pagedkv
