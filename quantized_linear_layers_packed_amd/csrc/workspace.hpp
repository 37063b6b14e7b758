// Caller-owned device workspace of the forward calls, and device properties.
//
// Layout (byte offsets from the workspace base; every region starts on a
// 256-byte boundary):
//   [0, kCounterBytes)   arrival counters of the stream-K GEMMs, one per
//                        workgroup slot.  They must be zero before the first call
//                        that uses the workspace; every such call leaves them at
//                        zero again when it completes.  No other data is ever
//                        written here, so one workspace serves every call and
//                        shape (calls that share it must not overlap in time).
//   [kCounterBytes, ..)  fp32 / int32 partial tiles of the stream-K GEMMs
//   [.., ..)             fp16 copy of bf16 activations (row-scaled) and the
//                        per-row exponents, for the W4 MFMA paths
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>

#include "common.hpp"

namespace qlin {

constexpr int kCounterSlots = 4096;                                   // >= stream-K workgroups
constexpr size_t kCounterBytes = static_cast<size_t>(kCounterSlots) * sizeof(int);

inline size_t ws_round(size_t v) { return (v + 255) & ~static_cast<size_t>(255); }

// The caller's workspace as seen by a launcher.
struct WsView {
  char* base = nullptr;
  size_t bytes = 0;
  int* counters() const { return reinterpret_cast<int*>(base); }
  void* partials() const { return base + kCounterBytes; }
};

// Compute units of the current device (queried once per device, thread-safe).
int device_cus();

}  // namespace qlin
