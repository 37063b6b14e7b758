// Per-device workspace for the split-K GEMMs.  One buffer per device, grown on
// demand and kept until the process ends.  The counters return to zero at the
// end of every call (the last workgroup to finish a tile resets its counter), so
// they are cleared only when the buffer is (re)allocated.  Calls that use the
// workspace on one device must not run concurrently (they share it).

#include "workspace.hpp"

#include <mutex>
#include <string>
#include <vector>

namespace qlin {

namespace {

struct DeviceWs {
  void* base = nullptr;
  size_t partial_bytes = 0;
  size_t ncounters = 0;
};

std::mutex g_mu;
std::vector<DeviceWs> g_ws;
std::vector<int> g_cus;

size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

}  // namespace

int device_cus() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  std::lock_guard<std::mutex> lk(g_mu);
  if (static_cast<int>(g_cus.size()) <= dev) g_cus.resize(dev + 1, 0);
  if (g_cus[dev] == 0) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
    g_cus[dev] = cus;
  }
  return g_cus[dev];
}

qlin_status get_workspace(size_t partial_bytes, size_t ncounters, hipStream_t stream, const char* fn,
                          Workspace* out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return fail(QLIN_EHIP, std::string(fn) + ": hipGetDevice failed");
  std::lock_guard<std::mutex> lk(g_mu);
  if (static_cast<int>(g_ws.size()) <= dev) g_ws.resize(dev + 1);
  DeviceWs& w = g_ws[dev];
  if (w.base == nullptr || w.partial_bytes < partial_bytes || w.ncounters < ncounters) {
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(stream, &cs) == hipSuccess && cs != hipStreamCaptureStatusNone)
      return fail(QLIN_EUNSUPPORTED, std::string(fn) +
                                         ": the split-K workspace must grow, which cannot happen during graph "
                                         "capture; make one uncaptured call of this shape first");
    const size_t pb = round_up(std::max(partial_bytes, w.partial_bytes), 256);
    const size_t nc = round_up(std::max(ncounters, w.ncounters), 64);
    if (w.base) {
      if (hipDeviceSynchronize() != hipSuccess || hipFree(w.base) != hipSuccess)
        return fail(QLIN_EHIP, std::string(fn) + ": freeing the old workspace failed");
      w.base = nullptr;
    }
    void* p = nullptr;
    if (hipMalloc(&p, pb + nc * sizeof(int)) != hipSuccess)
      return fail(QLIN_EHIP, std::string(fn) + ": workspace allocation failed");
    if (hipMemset(static_cast<char*>(p) + pb, 0, nc * sizeof(int)) != hipSuccess ||
        hipDeviceSynchronize() != hipSuccess) {
      (void)hipFree(p);
      return fail(QLIN_EHIP, std::string(fn) + ": clearing the workspace counters failed");
    }
    w.base = p;
    w.partial_bytes = pb;
    w.ncounters = nc;
  }
  out->partials = static_cast<float*>(w.base);
  out->counters = reinterpret_cast<int*>(static_cast<char*>(w.base) + w.partial_bytes);
  return QLIN_OK;
}

}  // namespace qlin
