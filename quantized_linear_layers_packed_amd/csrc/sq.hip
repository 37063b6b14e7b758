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
// in LDS per 128-wide K step (double buffered) and shared by the waves; each
// wave streams its own weight rows from HBM into MFMA operand registers one K
// step ahead.  Epilogue: float(acc) * x_scale[m] * w_scale[n], rounded once.

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

constexpr int kGemmThreads = 256;   // 4 waves
constexpr int kBK = 128;            // K bytes per pipeline step (4 MFMA steps)

// Tiles of 32 x 32 outputs; waves WM x WN, each TM x TN tiles.  Within one
// 128-byte K step, MFMA step st and lane half h use bytes 64h + 16st .. +15 of
// both operands (a fixed permutation of k, identical for A and B), so each lane
// streams 64 contiguous bytes of its weight row per K step.  The next K step's
// weights are loaded into registers and its activation tile into the second
// LDS buffer while the current one is multiplied.
template <int WM, int WN, int TM, int TN, int OUTK>
__global__ __launch_bounds__(kGemmThreads) void sq_gemm_kernel(
    const int8_t* __restrict__ Xq, const float* __restrict__ x_scale,
    const int8_t* __restrict__ Wq, const float* __restrict__ w_scale,
    int M, int N, int K, void* __restrict__ Y, int32_t* __restrict__ acc_out) {
  static_assert(WM * WN == 4, "four waves");
  constexpr int BM = WM * TM * 32, BN = WN * TN * 32;
  constexpr int ROW = kBK + 16;                          // LDS row stride in bytes
  constexpr int PIECES = BM * kBK / 16;                  // 16-byte activation pieces per K step
  constexpr int APT = (PIECES + kGemmThreads - 1) / kGemmThreads;
  __shared__ __attribute__((aligned(16))) int8_t As[2][BM * ROW];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = tid >> 6;
  const int wm = wv / WN, wn = wv % WN;
  const int col = lane & 31, half = lane >> 5;
  const int MB = (M + BM - 1) / BM;
  const int tile = xcd_tile(blockIdx.x, gridDim.x);
  const int m0 = (tile % MB) * BM;
  const int n0 = (tile / MB) * BN + wn * TN * 32;
  const int nk = (K + kBK - 1) / kBK;

  const int8_t* wrow[TN];
  bool nok[TN];
#pragma unroll
  for (int t = 0; t < TN; ++t) {
    const int n = n0 + 32 * t + col;
    nok[t] = n < N;
    wrow[t] = Wq + static_cast<size_t>(nok[t] ? n : 0) * K;
  }

  uint4 av[APT];
  uint4 bq[TN][4];
  auto load_a = [&](int kk) {
#pragma unroll
    for (int p = 0; p < APT; ++p) {
      const int piece = tid + p * kGemmThreads;
      const int r = piece / (kBK / 16), c = piece - r * (kBK / 16);
      const int m = m0 + r;
      const int k = kk * kBK + 16 * c;
      av[p] = (piece < PIECES && m < M && k < K)
                  ? *reinterpret_cast<const uint4*>(Xq + static_cast<size_t>(m) * K + k)
                  : make_uint4(0u, 0u, 0u, 0u);
    }
  };
  auto store_a = [&](int buf) {
#pragma unroll
    for (int p = 0; p < APT; ++p) {
      const int piece = tid + p * kGemmThreads;
      if (piece < PIECES) {
        const int r = piece / (kBK / 16), c = piece - r * (kBK / 16);
        *reinterpret_cast<uint4*>(&As[buf][r * ROW + 16 * c]) = av[p];
      }
    }
  };
  auto load_b = [&](int kk) {
#pragma unroll
    for (int t = 0; t < TN; ++t) {
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        const int k = kk * kBK + 64 * half + 16 * st;
        bq[t][st] = (nok[t] && k < K) ? load_stream16(wrow[t] + k) : make_uint4(0u, 0u, 0u, 0u);
      }
    }
  };

  i32x16_t acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int t = 0; t < TN; ++t) acc[i][t] = i32x16_t{};

  load_a(0);
  load_b(0);
  store_a(0);
  __syncthreads();

  for (int kk = 0; kk < nk; ++kk) {
    const int buf = kk & 1;
    uint4 bcur[TN][4];
#pragma unroll
    for (int t = 0; t < TN; ++t)
#pragma unroll
      for (int st = 0; st < 4; ++st) bcur[t][st] = bq[t][st];
    if (kk + 1 < nk) {
      load_a(kk + 1);
      load_b(kk + 1);
    }
#pragma unroll
    for (int st = 0; st < 4; ++st) {
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const int r = (wm * TM + i) * 32 + col;
        const i32x4_t a = *reinterpret_cast<const i32x4_t*>(&As[buf][r * ROW + 64 * half + 16 * st]);
#pragma unroll
        for (int t = 0; t < TN; ++t) {
          const i32x4_t b = bitcast<i32x4_t>(bcur[t][st]);
          acc[i][t] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, acc[i][t], 0, 0, 0);
        }
      }
    }
    if (kk + 1 < nk) {
      store_a(buf ^ 1);
      __syncthreads();
    }
  }

#pragma unroll
  for (int t = 0; t < TN; ++t) {
    if (!nok[t]) continue;
    const int n = n0 + 32 * t + col;
    const float ws = w_scale[n];
#pragma unroll
    for (int i = 0; i < TM; ++i) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = m0 + (wm * TM + i) * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
        if (m < M) {
          const size_t idx = static_cast<size_t>(m) * N + n;
          store_out<OUTK>(Y, idx, static_cast<float>(acc[i][t][r]) * x_scale[m] * ws);
          if (acc_out) acc_out[idx] = acc[i][t][r];
        }
      }
    }
  }
}

template <int WM, int WN, int TM, int TN>
void gemm_t(const int8_t* Xq, const float* xsc, const int8_t* Wq, const float* wsc, int M, int N, int K,
            void* Y, int y_dtype, int32_t* acc_out, hipStream_t stream) {
  constexpr int BM = WM * TM * 32, BN = WN * TN * 32;
  dim3 grid(((N + BN - 1) / BN) * ((M + BM - 1) / BM));
  if (y_dtype == QLIN_F32)
    hipLaunchKernelGGL((sq_gemm_kernel<WM, WN, TM, TN, OUT_F32>), grid, dim3(kGemmThreads), 0, stream,
                       Xq, xsc, Wq, wsc, M, N, K, Y, acc_out);
  else
    hipLaunchKernelGGL((sq_gemm_kernel<WM, WN, TM, TN, OUT_F16>), grid, dim3(kGemmThreads), 0, stream,
                       Xq, xsc, Wq, wsc, M, N, K, Y, acc_out);
}

}  // namespace

void sq_act_launch(const uint16_t* X, const float* inv_s, int M, int K, int8_t* Xq, float* x_scale,
                   hipStream_t stream) {
  hipLaunchKernelGGL(sq_act_kernel, dim3(M), dim3(kActThreads), 0, stream, X, inv_s, K, Xq, x_scale);
}

void sq_gemm_launch(const int8_t* Xq, const float* x_scale, const int8_t* Wq, const float* w_scale,
                    int M, int N, int K, void* Y, int y_dtype, int32_t* acc_out, hipStream_t stream) {
  // Largest tile that still gives every CU a workgroup; small batches use one
  // 32-row tile with the four waves side by side along N.
  auto wgs = [&](int bm, int bn) { return static_cast<long>((M + bm - 1) / bm) * ((N + bn - 1) / bn); };
  if (M <= 32) gemm_t<1, 4, 1, 1>(Xq, x_scale, Wq, w_scale, M, N, K, Y, y_dtype, acc_out, stream);
  else if (wgs(128, 128) >= 256) gemm_t<2, 2, 2, 2>(Xq, x_scale, Wq, w_scale, M, N, K, Y, y_dtype, acc_out, stream);
  else if (wgs(64, 128) >= 256) gemm_t<2, 2, 1, 2>(Xq, x_scale, Wq, w_scale, M, N, K, Y, y_dtype, acc_out, stream);
  else gemm_t<2, 2, 1, 1>(Xq, x_scale, Wq, w_scale, M, N, K, Y, y_dtype, acc_out, stream);
}

}  // namespace qlin
