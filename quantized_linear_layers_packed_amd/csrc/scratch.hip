// The W4 forward for callers that cannot allocate device memory (code under
// HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
// qlin_w4_forward with the workspace taken from a fixed device array of the
// library instead of from the caller.
//
// The array lives in the code object (zero at load) on every device the
// library runs on, until the process ends.  Its device address is looked up
// once per device (hipGetSymbolAddress, with that device current) and only that
// address is ever handed to kernels.  Every call on a device shares the array:
// the arrival counters are cleared by a small fill kernel on the caller's
// stream before each split-K call, and calls that overlap in time on one
// device race on it.

#include <mutex>
#include <string>
#include <vector>

#include "common.hpp"
#include "launch.hpp"

namespace qlin {

namespace {

constexpr size_t kScratchBytes = static_cast<size_t>(80) << 20;

static __device__ __align__(256) char scratch[kScratchBytes];

__global__ void zero_words_kernel(int* p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0;
}

}  // namespace

size_t scratch_bytes() { return kScratchBytes; }

qlin_status scratch_base(char** out) {
  static std::mutex mu;
  static std::vector<char*> base;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return fail(QLIN_EHIP, "scratch: hipGetDevice failed");
  std::lock_guard<std::mutex> lk(mu);
  if (static_cast<int>(base.size()) <= dev) base.resize(dev + 1, nullptr);
  if (!base[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(QLIN_EHIP, std::string("scratch: hipGetSymbolAddress failed: ") + hipGetErrorString(e));
    base[dev] = static_cast<char*>(p);
  }
  *out = base[dev];
  return QLIN_OK;
}

void scratch_clear_counters(char* base, hipStream_t stream) {
  hipLaunchKernelGGL(zero_words_kernel, dim3(kCounterSlots / 256), dim3(256), 0, stream, reinterpret_cast<int*>(base),
                     kCounterSlots);
}

}  // namespace qlin
