// Activation column gather for 4-bit storage kept in act-order (GPTQ bulletin,
// "Kod ve Entegrasyon Haritası": ordering the columns by activation size makes
// the groups irregular at run time).  The storage holds the columns in
// quantization order, so the forward needs Xp[m][t] = X[m][perm[t]]; this
// gather runs once per call, after which the regular kernels see contiguous
// groups.

#include "common.hpp"
#include "launch.hpp"

namespace qlin {

namespace {

__global__ __launch_bounds__(256) void permute_cols_kernel(const uint16_t* X, const int32_t* perm, int M, int K,
                                                           uint16_t* Xp) {
  const int t = blockIdx.x * 256 + threadIdx.x;
  if (t >= K) return;
  // clamped: a perm that is not a permutation gives a meaningless result, never
  // an access outside X
  const int j = min(max(perm[t], 0), K - 1);
  for (int m = blockIdx.y; m < M; m += gridDim.y)
    Xp[static_cast<size_t>(m) * K + t] = X[static_cast<size_t>(m) * K + j];
}

}  // namespace

void permute_cols_launch(const void* X, const int32_t* perm, int M, int K, void* Xp, hipStream_t stream) {
  const dim3 grid((K + 255) / 256, static_cast<unsigned>(std::min(M, 1024)));
  hipLaunchKernelGGL(permute_cols_kernel, grid, dim3(256), 0, stream, static_cast<const uint16_t*>(X), perm, M, K,
                     static_cast<uint16_t*>(Xp));
}

}  // namespace qlin
