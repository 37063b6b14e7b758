// Device property cache (the only state the library keeps besides the
// thread-local error message).

#include "workspace.hpp"

#include <mutex>
#include <vector>

namespace qlin {

int device_cus() {
  static std::mutex mu;
  static std::vector<int> cus;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  std::lock_guard<std::mutex> lk(mu);
  if (static_cast<int>(cus.size()) <= dev) cus.resize(dev + 1, 0);
  if (cus[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cus[dev] = n;
  }
  return cus[dev];
}

}  // namespace qlin
