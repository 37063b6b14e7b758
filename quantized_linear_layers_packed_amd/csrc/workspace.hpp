// Device workspace for kernels that split one output tile's K range over
// several workgroups (partial tiles + per-tile arrival counters).
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>

#include "common.hpp"

namespace qlin {

struct Workspace {
  float* partials = nullptr;   // fp32 partial tiles
  int* counters = nullptr;     // one arrival counter per output tile, zero between calls
};

// Returns a workspace of at least `partial_bytes` of partials and `ncounters`
// counters on the current device, growing the library's per-device buffer when
// needed.  Growing allocates (hipMalloc) and zeroes the counters synchronously,
// so it is refused while `stream` is being captured into a graph.
qlin_status get_workspace(size_t partial_bytes, size_t ncounters, hipStream_t stream, const char* fn,
                          Workspace* out);

// Compute units of the current device (cached per device).
int device_cus();

}  // namespace qlin
