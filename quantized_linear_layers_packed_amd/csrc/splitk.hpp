// Stream-K partition of a GEMM's (output tile, K step) iteration space over a
// fixed number of workgroups, and the fix-up of tiles whose K range is shared.
//
// Units u = tile * ksteps + kstep are dealt out in P contiguous ranges
// [begin(p), begin(p + 1)), begin(p) = floor(p * U / P), so every workgroup gets
// the same amount of multiply work whatever the tile count.  A tile covered by
// one range is finished in place; otherwise each contributing workgroup writes
// its fp32 partial tile to a workspace slot (two slots per workgroup: the tile
// its range starts in, and the tile it ends in), bumps the tile's counter, and
// the last one to arrive adds the partials in K order (the result does not
// depend on arrival order), writes the output and resets the counter.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>
#include <type_traits>

namespace qlin {

struct SkPlan {
  int ksteps;        // K steps per tile
  long long units;   // tiles * ksteps
  int P;             // workgroups
};

__device__ __forceinline__ long long sk_begin(const SkPlan& s, int p) {
  return (static_cast<long long>(p) * s.units) / s.P;
}

// Workgroup whose range holds unit u.
__device__ __forceinline__ int sk_owner(const SkPlan& s, long long u) {
  return static_cast<int>(((u + 1) * s.P + s.units - 1) / s.units) - 1;
}

// Hand-off of a shared tile.  Partial tiles cross XCDs, whose L2 caches are
// not coherent with each other, so every access to a partial is a device-scope
// (agent) atomic access: on gfx950 such stores are written through to the
// device coherence point and such loads are served from it, never from a stale
// line of an XCD's L2.  The ordering the last arriver relies on:
//   1. each contributor's threads store their part with agent-scope atomic
//      stores and then wait for all of them to complete (s_waitcnt vmcnt(0):
//      a vector store counts as complete once the memory side has acknowledged
//      it at the scope it was issued with);
//   2. a workgroup barrier orders every thread's wait before thread 0's
//      agent-scope atomic add on the tile's counter, which is performed at the
//      same coherence point, so when the add is performed every partial store
//      of that workgroup already is;
//   3. the workgroup whose add returns the final count issues its partial
//      loads only after the add has returned (the result is broadcast through
//      LDS behind a barrier), and those agent-scope loads read the coherence
//      point, so they see every contributor's stores.
// This is the hardware ordering of gfx950's memory pipeline, not the C++/HIP
// model's: under the model the counter would need release/acquire order, which
// the compiler implements with a write-back of the issuing XCD's whole L2 per
// arrival and an invalidate of the whole L2 per acquire.  Measured, that made
// the W4 GEMM at 256 rows 2x slower and the int8 GEMM 1.5x slower, while
// adding nothing the accesses above do not already have.  Repeat, graph
// replay and concurrent-stream tests check that the sums are bit-identical.
__device__ __forceinline__ void sk_store(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float sk_load(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void sk_store(int* p, int v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int sk_load(const int* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void sk_drain_stores() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Every thread of the workgroup calls this after storing its part of the
// partial tile.  Returns true (in every thread) for the workgroup that arrives
// last, i.e. sees `prior` earlier arrivals; that workgroup may then read the
// other partials (steps 1-3 above).  s_flag: a __shared__ int.
__device__ __forceinline__ bool sk_arrive_last(int* counter, int prior, int* s_flag) {
  sk_drain_stores();
  __syncthreads();
  if (threadIdx.x == 0)
    *s_flag = __hip_atomic_fetch_add(counter, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == prior;
  __syncthreads();
  return *s_flag != 0;
}

// The last arriver returns the counter to zero once it has read the partials
// (the next use is a later kernel, ordered by the kernel boundary).
__device__ __forceinline__ void sk_reset(int* counter) {
  __hip_atomic_store(counter, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Counter of a shared tile: indexed by the tile's first contributor.  A
// workgroup can be the first contributor of several tiles only when its range
// covers the earlier ones entirely, so at most one shared tile per workgroup:
// P counters suffice whatever the tile count.
__device__ __forceinline__ int sk_counter_index(const SkPlan& s, int t) {
  return sk_owner(s, static_cast<long long>(t) * s.ksteps);
}

// Workspace slot holding workgroup q's partial of tile t.
__device__ __forceinline__ int sk_slot(const SkPlan& s, int q, int t) {
  return 2 * q + ((sk_begin(s, q) / s.ksteps) == t ? 0 : 1);
}

}  // namespace qlin

namespace qlin {

// Calls f(I, kk) for I = 0 .. R-1 while kk < k1 (a K loop unrolled by the depth R
// of the register rings, so every ring index is a compile-time constant);
// returns false once the range is done.
template <int I, int R, class F>
__device__ __forceinline__ bool sk_run_steps(F& f, int& kk, int k1) {
  f(std::integral_constant<int, I>{}, kk);
  if (++kk >= k1) return false;
  if constexpr (I + 1 < R) return sk_run_steps<I + 1, R>(f, kk, k1);
  else return true;
}

template <int I, int R, class F>
__device__ __forceinline__ void sk_group_steps(F& f, int kk) {
  f(std::integral_constant<int, I>{}, kk + I);
  if constexpr (I + 1 < R) sk_group_steps<I + 1, R>(f, kk);
}

template <int I, int R, class F>
__device__ __forceinline__ void sk_tail_steps(F& f, int kk, int k1) {
  if (kk + I < k1) {
    f(std::integral_constant<int, I>{}, kk + I);
    if constexpr (I + 1 < R) sk_tail_steps<I + 1, R>(f, kk, k1);
  }
}

// The same steps kk .. k1-1, as a loop over whole groups of R steps whose body
// has no exit, then the remaining (fewer than R) steps after it.  With an exit
// after every step (sk_run_steps in a loop) the exit paths meet at the loop's
// latch, and the compiler's wait counts at the loop head then assume the ring
// order of the worst of them (a slot loaded last on one exit path), which for
// rings deeper than 2 drains the ring once per group.
template <int R, class F>
__device__ __forceinline__ void sk_ring_steps(F& f, int kk, int k1) {
  for (; kk + R <= k1; kk += R) sk_group_steps<0, R>(f, kk);
  sk_tail_steps<0, R>(f, kk, k1);
}

}  // namespace qlin
