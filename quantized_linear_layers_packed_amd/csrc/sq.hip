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
// wave streams its own weight rows from HBM into MFMA operand registers, R - 1
// K steps ahead.  Epilogue: float(acc) * x_scale[m] * w_scale[n], rounded once.

#include <algorithm>

#include "common.hpp"
#include "device.hpp"
#include "launch.hpp"
#include "splitk.hpp"
#include "workspace.hpp"

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

constexpr int kGemmThreads = 256;   // 4 waves side by side along N
constexpr int kBN = 128;            // output columns per tile
constexpr int kBK = 128;            // K bytes per step (4 MFMA steps of 32)

// Tiles of BM = 32 TM rows x 128 columns; a wave owns all BM rows and 32
// columns.  Within one 128-byte K step, MFMA step st and lane half h use bytes
// 64h + 16st .. +15 of both operands (a fixed permutation of k, identical for A
// and B), so each lane streams 64 contiguous bytes of its weight row per step.
// Activation rows go to LDS as 128-byte rows whose 16-byte chunks are
// XOR-swizzled by row / 2, so the 32 rows an MFMA reads fall in distinct banks.
// Weights and activations are fetched R - 1 steps ahead into register rings,
// with every load unconditional (clamped addresses) so that the compiler's
// in-order wait counts never drain the rings.  The (tile, K step) space is
// split evenly over the workgroups (stream-K); shared tiles are summed (int32,
// exact) by the last workgroup to finish them.
template <int TM, int R, int OUTK>
__global__ __launch_bounds__(kGemmThreads) void sq_gemm_sk_kernel(
    const int8_t* Xq, const float* x_scale, const int8_t* Wq, const float* w_scale,
    int M, int N, int K, int tiles_n, SkPlan plan, void* Y, int32_t* acc_out, int* ws, int* counters) {
  // (no __restrict__: it would let the prefetch loads be sunk across the step
  // barriers to their first use)
  constexpr int BM = 32 * TM;
  constexpr int APT = BM * 8 / kGemmThreads;   // 16-byte activation pieces per thread per step
  static_assert(APT >= 1, "tile too small");
  extern __shared__ uint4 smem[];
  __shared__ int s_last;
  uint4* const As0 = smem;
  uint4* const As1 = smem + BM * 8;

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int col = lane & 31, h = lane >> 5;
  const int swz = (col >> 1) & 7;

  const int p = xcd_tile(blockIdx.x, gridDim.x);
  long long u = sk_begin(plan, p);
  const long long u_end = sk_begin(plan, p + 1);

  while (u < u_end) {
    const int t = static_cast<int>(u / plan.ksteps);
    const int k0 = static_cast<int>(u - static_cast<long long>(t) * plan.ksteps);
    const int k1 = static_cast<int>(std::min<long long>(plan.ksteps, k0 + (u_end - u)));
    const int klast = k1 - 1;
    const int m0 = (t / tiles_n) * BM;
    const int n = (t % tiles_n) * kBN + 32 * wv + col;
    const bool nok = n < N;
    const size_t nn = static_cast<size_t>(min(n, N - 1));
    const int8_t* wrow = Wq + nn * K;

    // Activation rows past M are read from row M - 1 and never stored.  When
    // K % 128 == 64 the last step is half full: its addresses are clamped into
    // the row and its activation chunks past K are zeroed at staging, so the
    // weight bytes they meet contribute nothing.
    uint4 av[R][APT];
    auto load_a = [&](int s, uint4 (&v)[APT]) {
#pragma unroll
      for (int j = 0; j < APT; ++j) {
        const int piece = tid + j * kGemmThreads;
        const int r = piece >> 3, c = piece & 7;
        const int m = min(m0 + r, M - 1);
        const int kb = min(s * kBK + 16 * c, K - 16);
        v[j] = *reinterpret_cast<const uint4*>(Xq + static_cast<size_t>(m) * K + kb);
      }
    };
    auto store_a = [&](uint4* dst, const uint4 (&src)[APT], int s) {
      const bool tail = s * kBK + kBK > K;      // uniform
#pragma unroll
      for (int j = 0; j < APT; ++j) {
        const int piece = tid + j * kGemmThreads;
        const int r = piece >> 3, c = piece & 7;
        uint4 v = src[j];
        if (tail && s * kBK + 16 * c >= K) v = make_uint4(0u, 0u, 0u, 0u);
        dst[r * 8 + (c ^ ((r >> 1) & 7))] = v;
      }
    };
    uint4 bq[R][4];
    auto load_b = [&](int s, uint4 (&w)[4]) {
#pragma unroll
      for (int st = 0; st < 4; ++st)
        w[st] = *reinterpret_cast<const uint4*>(wrow + min(s * kBK + 64 * h + 16 * st, K - 16));
    };

    i32x16_t acc[TM];
#pragma unroll
    for (int i = 0; i < TM; ++i) acc[i] = i32x16_t{};

    // prologue in the steady-state issue order (weights of step j, then
    // activations of step j + 1), so the wait counts agree at the loop head
    load_a(k0, av[0]);
#pragma unroll
    for (int j = 0; j < R - 1; ++j) {
      load_b(min(k0 + j, klast), bq[j]);
      load_a(min(k0 + j + 1, klast), av[j + 1]);
    }
    store_a(As0, av[0], k0);
    __syncthreads();

    auto step = [&](auto set_c, int kk) {
      constexpr int S = decltype(set_c)::value;
      constexpr int SB = (S + R - 1) % R;
      load_b(min(kk + R - 1, klast), bq[SB]);
      __builtin_amdgcn_sched_barrier(0);
      const uint4* Ab = ((kk - k0) & 1) ? As1 : As0;
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        const i32x4_t b = bitcast<i32x4_t>(bq[S][st]);
        const int c = 4 * h + st;
#pragma unroll
        for (int i = 0; i < TM; ++i) {
          const i32x4_t a = bitcast<i32x4_t>(Ab[(32 * i + col) * 8 + (c ^ swz)]);
          acc[i] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, acc[i], 0, 0, 0);
        }
      }
      store_a(((kk + 1 - k0) & 1) ? As1 : As0, av[(S + 1) % R], kk + 1);
      load_a(min(kk + R, klast), av[S]);
      __builtin_amdgcn_sched_barrier(0);
      __syncthreads();
    };
    int kk = k0;
    while (sk_run_steps<0, R>(step, kk, k1)) {
    }

    // ---- finish the tile: lane holds column n, rows 8*(r/4) + 4*h + r%4 of each 32-row block
    bool write = true;
    if (k0 != 0 || k1 != plan.ksteps) {
      const int first = sk_owner(plan, static_cast<long long>(t) * plan.ksteps);
      const int last = sk_owner(plan, static_cast<long long>(t + 1) * plan.ksteps - 1);
      int* mine = ws + static_cast<size_t>(sk_slot(plan, p, t)) * (BM * kBN);
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) sk_store(mine + ((wv * TM + i) * 16 + r) * 64 + lane, acc[i][r]);
      sk_drain_stores();
      __syncthreads();
      if (tid == 0) s_last = sk_arrive(&counters[t]) == last - first;
      __syncthreads();
      write = s_last != 0;
      if (write) {
        for (int q = first; q <= last; ++q) {
          if (q == p) continue;
          const int* other = ws + static_cast<size_t>(sk_slot(plan, q, t)) * (BM * kBN);
#pragma unroll
          for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][r] += sk_load(other + ((wv * TM + i) * 16 + r) * 64 + lane);
        }
        if (tid == 0) sk_reset(&counters[t]);
      }
    }
    if (write && nok) {
      const float wsc = w_scale[n];
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int m = m0 + 32 * i + 8 * (r >> 2) + 4 * h + (r & 3);
          if (m < M) {
            const size_t idx = static_cast<size_t>(m) * N + n;
            store_out<OUTK>(Y, idx, static_cast<float>(acc[i][r]) * x_scale[m] * wsc);
            if (acc_out) acc_out[idx] = acc[i][r];
          }
        }
    }
    u += k1 - k0;
  }
}

template <int TM, int R, int OUTK>
qlin_status gemm_t(const int8_t* Xq, const float* xsc, const int8_t* Wq, const float* wsc, int M, int N, int K,
                   void* Y, int32_t* acc_out, hipStream_t stream) {
  constexpr int BM = 32 * TM;
  const size_t lds = static_cast<size_t>(2) * BM * 8 * sizeof(uint4);
  static int occ = 0;                          // resident workgroups per CU
  if (occ == 0) {
    int o = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&o, sq_gemm_sk_kernel<TM, R, OUTK>, kGemmThreads, lds) !=
            hipSuccess || o <= 0)
      o = 1;
    occ = std::min(o, 2);
  }
  const int tiles_m = (M + BM - 1) / BM;
  const int tiles_n = (N + kBN - 1) / kBN;
  const long long tiles = static_cast<long long>(tiles_m) * tiles_n;
  SkPlan plan;
  plan.ksteps = (K + kBK - 1) / kBK;
  plan.units = tiles * plan.ksteps;
  plan.P = static_cast<int>(std::min<long long>(static_cast<long long>(occ) * device_cus(), plan.units));
  Workspace w;
  const qlin_status s = get_workspace(static_cast<size_t>(2) * plan.P * BM * kBN * sizeof(int),
                                      static_cast<size_t>(tiles), stream, "sq_int8_gemm", &w);
  if (s != QLIN_OK) return s;
  hipLaunchKernelGGL((sq_gemm_sk_kernel<TM, R, OUTK>), dim3(plan.P), dim3(kGemmThreads), lds, stream, Xq, xsc, Wq,
                     wsc, M, N, K, tiles_n, plan, Y, acc_out, reinterpret_cast<int*>(w.partials), w.counters);
  return QLIN_OK;
}

template <int TM, int R>
qlin_status gemm_o(const int8_t* Xq, const float* xsc, const int8_t* Wq, const float* wsc, int M, int N, int K,
                   void* Y, int y_dtype, int32_t* acc_out, hipStream_t stream) {
  return y_dtype == QLIN_F32 ? gemm_t<TM, R, OUT_F32>(Xq, xsc, Wq, wsc, M, N, K, Y, acc_out, stream)
                             : gemm_t<TM, R, OUT_F16>(Xq, xsc, Wq, wsc, M, N, K, Y, acc_out, stream);
}

}  // namespace

void sq_act_launch(const uint16_t* X, const float* inv_s, int M, int K, int8_t* Xq, float* x_scale,
                   hipStream_t stream) {
  hipLaunchKernelGGL(sq_act_kernel, dim3(M), dim3(kActThreads), 0, stream, X, inv_s, K, Xq, x_scale);
}

qlin_status sq_gemm_launch(const int8_t* Xq, const float* x_scale, const int8_t* Wq, const float* w_scale,
                           int M, int N, int K, void* Y, int y_dtype, int32_t* acc_out, hipStream_t stream) {
  if (M <= 32) return gemm_o<1, 4>(Xq, x_scale, Wq, w_scale, M, N, K, Y, y_dtype, acc_out, stream);
  if (M <= 64) return gemm_o<2, 4>(Xq, x_scale, Wq, w_scale, M, N, K, Y, y_dtype, acc_out, stream);
  return gemm_o<4, 4>(Xq, x_scale, Wq, w_scale, M, N, K, Y, y_dtype, acc_out, stream);
}

}  // namespace qlin
