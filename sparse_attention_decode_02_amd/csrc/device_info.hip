// Device properties the launchers size their grids by: the compute-unit
// count of the current device and how many workgroups of a kernel it holds
// at once. Both are fixed for a device and kernel, so they are looked up once
// and kept (a lock guards the small table); each launch then costs one
// hipGetDevice instead of a device-attribute and an occupancy query.

#include <mutex>

#include "dsa_kernels.h"

namespace dsa {

namespace {

constexpr int kMaxDevices = 64;
constexpr int kMaxKernels = 64;

struct CapacityEntry {
  const void* kernel;
  int block;
  int device;
  int capacity;
};

std::mutex g_mutex;
int g_cus[kMaxDevices];               // 0 = not looked up yet
CapacityEntry g_cap[kMaxKernels];     // filled in order
int g_ncap = 0;

int current_device() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return -1;
  return dev;
}

int cus_locked(int dev) {
  if (g_cus[dev] == 0) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus <= 0)
      return 0;
    g_cus[dev] = cus;
  }
  return g_cus[dev];
}

}  // namespace

SideStream* side_stream() {
  static SideStream g_side[kMaxDevices];
  static bool g_side_ok[kMaxDevices];
  static std::mutex g_side_lock[kMaxDevices];
  const int dev = current_device();
  if (dev < 0) return nullptr;
  std::lock_guard<std::mutex> lock(g_mutex);
  if (!g_side_ok[dev]) {
    SideStream s{};
    if (hipStreamCreateWithFlags(&s.stream, hipStreamNonBlocking) != hipSuccess) return nullptr;
    if (hipEventCreateWithFlags(&s.fork, hipEventDisableTiming) != hipSuccess ||
        hipEventCreateWithFlags(&s.join, hipEventDisableTiming) != hipSuccess)
      return nullptr;
    s.lock = &g_side_lock[dev];
    g_side[dev] = s;
    g_side_ok[dev] = true;
  }
  return &g_side[dev];
}

int device_cus() {
  const int dev = current_device();
  if (dev < 0) return 0;
  std::lock_guard<std::mutex> lock(g_mutex);
  return cus_locked(dev);
}

int device_capacity(const void* kernel, int block) {
  const int dev = current_device();
  if (dev < 0) return 0;
  std::lock_guard<std::mutex> lock(g_mutex);
  for (int i = 0; i < g_ncap; ++i)
    if (g_cap[i].kernel == kernel && g_cap[i].block == block && g_cap[i].device == dev)
      return g_cap[i].capacity;
  const int cus = cus_locked(dev);
  int per_cu = 0;
  if (cus <= 0 || hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, block, 0) != hipSuccess)
    return 0;
  const int cap = cus * per_cu;
  if (g_ncap < kMaxKernels) g_cap[g_ncap++] = {kernel, block, dev, cap};
  return cap;
}

}  // namespace dsa
