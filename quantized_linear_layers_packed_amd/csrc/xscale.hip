// bf16 activations -> row-scaled fp16 copy for the W4 matrix-core paths, gfx950.
//
// The W4 MFMA kernels multiply fp16 activations with fp16 weights (the GPTQ
// bulletin's weight-only 4-bit layer keeps 16-bit activations).  A bf16 value
// has an 8-bit significand, which fp16 (11 bits) holds exactly, but bf16's
// exponent range is far wider than fp16's.  Each row m is therefore scaled by
// a power of two 2^-e_m that puts its largest magnitude into [2^14, 2^15):
// every value down to 2^-31 of the row maximum converts exactly, smaller ones
// are rounded to the fp16 subnormal step 2^-24 (an error of at most 2^-39 of
// the row maximum), and the kernels multiply the row's outputs by 2^e_m, which
// is exact.  A row that is all zero
// or whose maximum is not finite keeps e_m = 0.
//
// One workgroup of 256 threads per row: the row maximum from the bf16 bit
// patterns (magnitudes compare as integers), then the conversion (round to
// nearest even) of 16-byte chunks held in registers.

#include "common.hpp"
#include "device.hpp"
#include "launch.hpp"

namespace qlin {

namespace {

constexpr int kThreads = 256;

// floor(log2 |x|) - 14 for the bf16 magnitude bits b (0 < b < 0x7F80).
__device__ __forceinline__ int rowscale_exponent(uint32_t b) {
  const int E = static_cast<int>(b >> 7);
  if (E == 0) return (31 - __clz(static_cast<int>(b))) - 133 - 14;   // subnormal: b * 2^-133
  return E - 127 - 14;
}

// bf16 value (bits in the low half of h) times 2^-e as fp32.  A bf16 subnormal
// is rebuilt from its integer mantissa (value = mantissa * 2^-133), so the
// result does not depend on how the arithmetic treats fp32 subnormal inputs.
__device__ __forceinline__ float bf16_times_pow2(uint32_t h, int e) {
  const uint32_t mag = h & 0x7FFFu;
  if ((mag >> 7) != 0) return ldexpf(bitcast<float>(h << 16), -e);
  const float v = ldexpf(static_cast<float>(mag), -133 - e);
  return (h & 0x8000u) ? -v : v;
}

// Largest magnitude (bf16 bits, sign cleared) of the 8 values of a chunk.
__device__ __forceinline__ uint32_t chunk_absmax(const uint4& v) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  uint32_t mx = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) mx = max(mx, max(w[j] & 0x7FFFu, (w[j] >> 16) & 0x7FFFu));
  return mx;
}

__device__ __forceinline__ uint4 chunk_convert(const uint4& v, int e) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  uint32_t o[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const h2_t hh = {static_cast<_Float16>(bf16_times_pow2(w[j] & 0xFFFFu, e)),
                     static_cast<_Float16>(bf16_times_pow2(w[j] >> 16, e))};
    o[j] = bitcast<uint32_t>(hh);
  }
  return make_uint4(o[0], o[1], o[2], o[3]);
}

// Rows of up to kThreads * CPT chunks (CPT * 2048 values) are read once: every
// chunk of a thread is loaded before the first use (indices clamped into the
// row, so no load is conditional), the row maximum taken, and the registers
// converted.  Longer rows loop over slices of that size and read the row twice.
template <int CPT>
__global__ __launch_bounds__(kThreads) void x_rowscale_kernel(const uint16_t* __restrict__ X, int K,
                                                              uint16_t* __restrict__ Xh, int* __restrict__ rowexp) {
  __shared__ uint32_t s_max[kThreads / 64];
  const int m = blockIdx.x, tid = threadIdx.x;
  const uint4* src = reinterpret_cast<const uint4*>(X + static_cast<size_t>(m) * K);
  uint4* dst = reinterpret_cast<uint4*>(Xh + static_cast<size_t>(m) * K);
  const int nchunk = K >> 3;
  constexpr int kSlice = kThreads * CPT;

  uint4 v[CPT];
  uint32_t mx = 0;
  for (int c0 = 0; c0 < nchunk; c0 += kSlice) {
#pragma unroll
    for (int j = 0; j < CPT; ++j) v[j] = src[min(c0 + tid + j * kThreads, nchunk - 1)];
#pragma unroll
    for (int j = 0; j < CPT; ++j) mx = max(mx, chunk_absmax(v[j]));
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) mx = max(mx, static_cast<uint32_t>(__shfl_xor(static_cast<int>(mx), off, 64)));
  if ((tid & 63) == 0) s_max[tid >> 6] = mx;
  __syncthreads();
  mx = s_max[0];
#pragma unroll
  for (int w = 1; w < kThreads / 64; ++w) mx = max(mx, s_max[w]);
  const int e = (mx == 0 || mx >= 0x7F80u) ? 0 : rowscale_exponent(mx);
  if (tid == 0) rowexp[m] = e;

  if (nchunk <= kSlice) {                       // the whole row is in registers
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
      const int c = tid + j * kThreads;
      if (c < nchunk) dst[c] = chunk_convert(v[j], e);
    }
    return;
  }
  for (int c0 = 0; c0 < nchunk; c0 += kSlice) {
#pragma unroll
    for (int j = 0; j < CPT; ++j) v[j] = src[min(c0 + tid + j * kThreads, nchunk - 1)];
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
      const int c = c0 + tid + j * kThreads;
      if (c < nchunk) dst[c] = chunk_convert(v[j], e);
    }
  }
}

}  // namespace

void x_rowscale_launch(const uint16_t* X, int M, int K, uint16_t* Xh, int* rowexp, hipStream_t stream) {
  const int nchunk = K / 8;
  if (nchunk <= kThreads * 4)
    hipLaunchKernelGGL(x_rowscale_kernel<4>, dim3(M), dim3(kThreads), 0, stream, X, K, Xh, rowexp);
  else
    hipLaunchKernelGGL(x_rowscale_kernel<16>, dim3(M), dim3(kThreads), 0, stream, X, K, Xh, rowexp);
}

}  // namespace qlin
