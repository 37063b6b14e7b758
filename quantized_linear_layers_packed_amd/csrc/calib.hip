// Measurement aids: a plain streaming read of a device buffer (the achievable
// bandwidth reference for the memory-bound kernels), a plain copy (the
// known-size reference that scales the hardware byte counters) and a dense
// matrix-core loop per data type (the achievable MFMA rate).  Each thread reads 16-byte
// vectors (coalesced, 64 lanes x 16 B per instruction) and folds them with XOR;
// one word per workgroup is written so the loads cannot be removed.

#include <algorithm>

#include "common.hpp"
#include "device.hpp"

namespace qlin {
namespace {

constexpr int kThreads = 256;

template <int U, bool NT>
__global__ __launch_bounds__(kThreads) void stream_read_kernel(const uint4* __restrict__ p, size_t n16,
                                                               uint32_t* __restrict__ out) {
  __shared__ uint32_t red[kThreads / 64];
  uint32_t acc = 0;
  const size_t stride = static_cast<size_t>(gridDim.x) * kThreads * U;
  for (size_t base = static_cast<size_t>(blockIdx.x) * kThreads * U + threadIdx.x; base < n16; base += stride) {
    uint4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const size_t i = base + static_cast<size_t>(u) * kThreads;
      if (i < n16) v[u] = NT ? load_stream16(p + i) : p[i];
      else v[u] = make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) acc ^= __shfl_xor(acc, off, 64);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) out[blockIdx.x] = red[0] ^ red[1] ^ red[2] ^ red[3];
}

__global__ __launch_bounds__(kThreads) void stream_copy_kernel(uint4* __restrict__ dst, const uint4* __restrict__ src,
                                                               size_t n16) {
  const size_t stride = static_cast<size_t>(gridDim.x) * kThreads;
  for (size_t i = static_cast<size_t>(blockIdx.x) * kThreads + threadIdx.x; i < n16; i += stride) dst[i] = src[i];
}

// Every wave runs `iters` rounds of kChains independent matrix instructions on
// register operands (no memory traffic; the chains hide the instruction's
// latency) and writes one value, so nothing is removed.
constexpr int kChains = 4;

template <int KIND>   // 0: v_mfma_f32_32x32x16_f16, 1: _bf16, 2: v_mfma_i32_32x32x32_i8
__global__ __launch_bounds__(kThreads) void mfma_peak_kernel(int iters, float* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  const uint32_t seed = 0x3C003C00u ^ static_cast<uint32_t>(lane);
  if constexpr (KIND == 2) {
    const i32x4_t a = {static_cast<int>(seed), static_cast<int>(seed >> 1), 3, 5};
    const i32x4_t b = {7, static_cast<int>(seed >> 2), 11, 13};
    i32x16_t acc[kChains];
#pragma unroll
    for (int c = 0; c < kChains; ++c) acc[c] = i32x16_t{};
    for (int it = 0; it < iters; ++it)
#pragma unroll
      for (int c = 0; c < kChains; ++c) acc[c] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, acc[c], 0, 0, 0);
    int s = 0;
#pragma unroll
    for (int c = 0; c < kChains; ++c) s += acc[c][0] + acc[c][15];
    if (lane == 0) out[(blockIdx.x * kThreads + threadIdx.x) >> 6] = static_cast<float>(s);
  } else {
    typedef __bf16 bf8_t __attribute__((ext_vector_type(8)));
    h8_t ah, bh;
    bf8_t ab, bb;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      ah[j] = static_cast<_Float16>(1.0f / static_cast<float>(lane + j + 1));
      bh[j] = static_cast<_Float16>(0.5f);
      ab[j] = static_cast<__bf16>(1.0f / static_cast<float>(lane + j + 1));
      bb[j] = static_cast<__bf16>(0.5f);
    }
    f32x16_t acc[kChains];
#pragma unroll
    for (int c = 0; c < kChains; ++c) acc[c] = f32x16_t{};
    for (int it = 0; it < iters; ++it)
#pragma unroll
      for (int c = 0; c < kChains; ++c) {
        if constexpr (KIND == 0) acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ah, bh, acc[c], 0, 0, 0);
        else acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ab, bb, acc[c], 0, 0, 0);
      }
    float s = 0.0f;
#pragma unroll
    for (int c = 0; c < kChains; ++c) s += acc[c][0] + acc[c][15];
    if (lane == 0) out[(blockIdx.x * kThreads + threadIdx.x) >> 6] = s;
  }
}

}  // namespace
}  // namespace qlin

using namespace qlin;

extern "C" qlin_status qlin_mfma_peak(int kind, int iters, int grid, float* out, hipStream_t stream) {
  clear_error();
  if (kind < 0 || kind > 2 || iters <= 0 || grid <= 0 || !out)
    return fail(QLIN_EINVAL, "qlin_mfma_peak: kind 0..2, iters > 0, grid > 0, non-NULL out");
  if (kind == 0) hipLaunchKernelGGL(mfma_peak_kernel<0>, dim3(grid), dim3(kThreads), 0, stream, iters, out);
  else if (kind == 1) hipLaunchKernelGGL(mfma_peak_kernel<1>, dim3(grid), dim3(kThreads), 0, stream, iters, out);
  else hipLaunchKernelGGL(mfma_peak_kernel<2>, dim3(grid), dim3(kThreads), 0, stream, iters, out);
  return check_launch("qlin_mfma_peak");
}

extern "C" qlin_status qlin_stream_read(const void* buf, size_t bytes, int grid, int unroll, int nontemporal,
                                        uint32_t* out, hipStream_t stream) {
  clear_error();
  if (!buf || !out || bytes == 0 || bytes % 16 != 0 || grid <= 0)
    return fail(QLIN_EINVAL, "qlin_stream_read: need non-NULL buffers, bytes % 16 == 0, grid > 0");
  if (!aligned16(buf)) return fail(QLIN_EALIGN, "qlin_stream_read: buf is not 16-byte aligned");
  const size_t n16 = bytes / 16;
  const uint4* p = static_cast<const uint4*>(buf);
  if (unroll <= 1) {
    if (nontemporal) hipLaunchKernelGGL((stream_read_kernel<1, true>), dim3(grid), dim3(kThreads), 0, stream, p, n16, out);
    else hipLaunchKernelGGL((stream_read_kernel<1, false>), dim3(grid), dim3(kThreads), 0, stream, p, n16, out);
  } else if (unroll <= 4) {
    if (nontemporal) hipLaunchKernelGGL((stream_read_kernel<4, true>), dim3(grid), dim3(kThreads), 0, stream, p, n16, out);
    else hipLaunchKernelGGL((stream_read_kernel<4, false>), dim3(grid), dim3(kThreads), 0, stream, p, n16, out);
  } else {
    if (nontemporal) hipLaunchKernelGGL((stream_read_kernel<8, true>), dim3(grid), dim3(kThreads), 0, stream, p, n16, out);
    else hipLaunchKernelGGL((stream_read_kernel<8, false>), dim3(grid), dim3(kThreads), 0, stream, p, n16, out);
  }
  return check_launch("qlin_stream_read");
}

extern "C" qlin_status qlin_stream_copy(void* dst, const void* src, size_t bytes, hipStream_t stream) {
  clear_error();
  if (!dst || !src || bytes == 0 || bytes % 16 != 0)
    return fail(QLIN_EINVAL, "qlin_stream_copy: need non-NULL buffers and bytes % 16 == 0");
  if (!aligned16(dst) || !aligned16(src)) return fail(QLIN_EALIGN, "qlin_stream_copy: buffers must be 16-byte aligned");
  const size_t n16 = bytes / 16;
  const int grid = static_cast<int>(std::min<size_t>((n16 + kThreads - 1) / kThreads, 4096));
  hipLaunchKernelGGL(stream_copy_kernel, dim3(grid), dim3(kThreads), 0, stream, static_cast<uint4*>(dst),
                     static_cast<const uint4*>(src), n16);
  return check_launch("qlin_stream_copy");
}
