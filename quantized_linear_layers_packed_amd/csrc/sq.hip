// SmoothQuant W8A8 on gfx950: per-token smooth + int8 quantize, then an int8
// MFMA GEMM with a per-token x per-channel rescale epilogue.
//
// SmoothQuant bulletin ("İddia ve Gerçeklik" and its equation
// Y = (X diag(s)^-1)(diag(s) W)): s is folded into the weights offline; online,
// the activations are divided by s per channel, quantized per token to int8 and
// multiplied against per-channel int8 weights on the INT8 matrix units.
//
// Activation kernel: one workgroup per token row.  x~ = fp32(x) * inv_s,
// a = max |x~| (wave shuffle, then LDS across the four waves),
// scale = a / 127, q = clamp(rint(x~ * (127 / a)), -127, 127) with correctly
// rounded fp32 divisions and round-half-even, so the int8 codes and scales
// equal the host definition bit for bit.
//
// GEMM kernel: v_mfma_i32_32x32x32_i8, exact int32 accumulation
// (|acc| <= K * 127^2 < 2^31 for K <= 131072).  The token tile of Xq is staged
// in LDS per 128-wide K step and shared by four waves, each of which streams its
// own 32 weight rows straight from HBM into MFMA operand registers (16 int8 per
// lane per step).  Epilogue: float(acc) * x_scale[m] * w_scale[n], rounded once.

#include "common.hpp"
#include "device.hpp"
#include "launch.hpp"

namespace qlin {

namespace {

constexpr int kActThreads = 256;

__global__ __launch_bounds__(kActThreads) void sq_act_kernel(const uint16_t* __restrict__ X,
                                                             const float* __restrict__ inv_s, int K,
                                                             int8_t* __restrict__ Xq, float* __restrict__ x_scale) {
  __shared__ float red[kActThreads / 64];
  const int m = blockIdx.x;
  const uint4* xr = reinterpret_cast<const uint4*>(X + static_cast<size_t>(m) * K);
  const int nv = K >> 3;                      // groups of 8 values
  float amax = 0.0f;
  for (int i = threadIdx.x; i < nv; i += kActThreads) {
    const uint4 v = xr[i];
    const uint32_t u[4] = {v.x, v.y, v.z, v.w};
    const float4 s0 = reinterpret_cast<const float4*>(inv_s)[2 * i];
    const float4 s1 = reinterpret_cast<const float4*>(inv_s)[2 * i + 1];
    const float sv[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float x = f16_bits_to_f32(static_cast<uint16_t>(u[j >> 1] >> (16 * (j & 1))));
      amax = fmaxf(amax, fabsf(x * sv[j]));
    }
  }
  amax = wave_max(amax);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = amax;
  __syncthreads();
  float a = red[0];
#pragma unroll
  for (int w = 1; w < kActThreads / 64; ++w) a = fmaxf(a, red[w]);
  const float r = (a == 0.0f) ? 0.0f : __fdiv_rn(127.0f, a);
  if (threadIdx.x == 0) x_scale[m] = (a == 0.0f) ? 0.0f : __fdiv_rn(a, 127.0f);

  uint2* qr = reinterpret_cast<uint2*>(Xq + static_cast<size_t>(m) * K);
  for (int i = threadIdx.x; i < nv; i += kActThreads) {
    const uint4 v = xr[i];
    const uint32_t u[4] = {v.x, v.y, v.z, v.w};
    const float4 s0 = reinterpret_cast<const float4*>(inv_s)[2 * i];
    const float4 s1 = reinterpret_cast<const float4*>(inv_s)[2 * i + 1];
    const float sv[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
    uint32_t packed[2] = {0u, 0u};
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float x = f16_bits_to_f32(static_cast<uint16_t>(u[j >> 1] >> (16 * (j & 1))));
      const float t = __fmul_rn(x * sv[j], r);
      const float q = fminf(fmaxf(rintf(t), -127.0f), 127.0f);
      const uint32_t b = static_cast<uint32_t>(static_cast<int32_t>(q)) & 0xFFu;
      packed[j >> 2] |= b << (8 * (j & 3));
    }
    qr[i] = make_uint2(packed[0], packed[1]);
  }
}

constexpr int kGemmThreads = 256;   // 4 waves x 32 output columns
constexpr int kBK = 128;            // K bytes staged per iteration (4 MFMA steps)

template <int TM, int OUTK>
__global__ __launch_bounds__(kGemmThreads) void sq_gemm_kernel(
    const int8_t* __restrict__ Xq, const float* __restrict__ x_scale,
    const int8_t* __restrict__ Wq, const float* __restrict__ w_scale,
    int M, int N, int K, void* __restrict__ Y, int32_t* __restrict__ acc_out) {
  constexpr int BM = 32 * TM;
  constexpr int ROW = kBK + 16;      // LDS row stride in bytes (padding against bank conflicts)
  __shared__ __attribute__((aligned(16))) int8_t As[BM * ROW];

  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int col = lane & 31, half = lane >> 5;
  const int m0 = blockIdx.y * BM;
  const int n = blockIdx.x * 128 + wv * 32 + col;
  const bool n_ok = n < N;
  const int8_t* wrow = Wq + static_cast<size_t>(n_ok ? n : 0) * K;

  i32x16_t acc[TM];
#pragma unroll
  for (int t = 0; t < TM; ++t) acc[t] = i32x16_t{};

  for (int k0 = 0; k0 < K; k0 += kBK) {
    __syncthreads();
    for (int it = threadIdx.x; it < BM * (kBK / 16); it += kGemmThreads) {
      const int r = it / (kBK / 16), c = it - r * (kBK / 16);
      const int m = m0 + r;
      uint4 v = make_uint4(0u, 0u, 0u, 0u);
      if (m < M && k0 + 16 * c < K) v = *reinterpret_cast<const uint4*>(Xq + static_cast<size_t>(m) * K + k0 + 16 * c);
      *reinterpret_cast<uint4*>(As + r * ROW + 16 * c) = v;
    }
    __syncthreads();
    const int steps = min(kBK, K - k0) / 32;
#pragma unroll
    for (int st = 0; st < kBK / 32; ++st) {
      if (st < steps) {
        i32x4_t b = i32x4_t{};
        if (n_ok) b = *reinterpret_cast<const i32x4_t*>(wrow + k0 + 32 * st + 16 * half);
#pragma unroll
        for (int t = 0; t < TM; ++t) {
          const i32x4_t a = *reinterpret_cast<const i32x4_t*>(As + (32 * t + col) * ROW + 32 * st + 16 * half);
          acc[t] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, acc[t], 0, 0, 0);
        }
      }
    }
  }

  if (!n_ok) return;
  const float ws = w_scale[n];
#pragma unroll
  for (int t = 0; t < TM; ++t) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int m = m0 + 32 * t + 8 * (r >> 2) + 4 * half + (r & 3);
      if (m < M) {
        const size_t idx = static_cast<size_t>(m) * N + n;
        store_out<OUTK>(Y, idx, static_cast<float>(acc[t][r]) * x_scale[m] * ws);
        if (acc_out) acc_out[idx] = acc[t][r];
      }
    }
  }
}

template <int TM>
void gemm_t(const int8_t* Xq, const float* xsc, const int8_t* Wq, const float* wsc, int M, int N, int K,
            void* Y, int y_dtype, int32_t* acc_out, hipStream_t stream) {
  dim3 grid((N + 127) / 128, (M + 32 * TM - 1) / (32 * TM));
  if (y_dtype == QLIN_F32)
    hipLaunchKernelGGL((sq_gemm_kernel<TM, OUT_F32>), grid, dim3(kGemmThreads), 0, stream, Xq, xsc, Wq, wsc, M, N, K, Y, acc_out);
  else
    hipLaunchKernelGGL((sq_gemm_kernel<TM, OUT_F16>), grid, dim3(kGemmThreads), 0, stream, Xq, xsc, Wq, wsc, M, N, K, Y, acc_out);
}

}  // namespace

void sq_act_launch(const uint16_t* X, const float* inv_s, int M, int K, int8_t* Xq, float* x_scale,
                   hipStream_t stream) {
  hipLaunchKernelGGL(sq_act_kernel, dim3(M), dim3(kActThreads), 0, stream, X, inv_s, K, Xq, x_scale);
}

void sq_gemm_launch(const int8_t* Xq, const float* x_scale, const int8_t* Wq, const float* w_scale,
                    int M, int N, int K, void* Y, int y_dtype, int32_t* acc_out, hipStream_t stream) {
  if (M <= 32) gemm_t<1>(Xq, x_scale, Wq, w_scale, M, N, K, Y, y_dtype, acc_out, stream);
  else if (M <= 64) gemm_t<2>(Xq, x_scale, Wq, w_scale, M, N, K, Y, y_dtype, acc_out, stream);
  else gemm_t<4>(Xq, x_scale, Wq, w_scale, M, N, K, Y, y_dtype, acc_out, stream);
}

}  // namespace qlin
