// W4 fused unpack-dequant GEMV for small batches (M <= 16), gfx950.
//
// Y[m][n] = sum_g S[n][g] * sum_{k in g} x[m][k] * (q[n][k] - z[n][g])
//
// Weight-only 4-bit inference at small batch is bound by memory bandwidth
// (GPTQ bulletin, "İddia ve Gerçeklik"), so this kernel streams the packed words
// exactly once with 128-bit loads and keeps the per-code work at a few VALU
// operations:
//   * the activations of the whole batch are staged once per workgroup in LDS,
//     already arranged as the (x_j, x_{j+4}) pairs the code unpack produces,
//     together with per-chunk sums sum(x) (a chunk = 32 codes = one uint4);
//   * each wavefront owns whole output rows; its lanes stride over the row's
//     chunks (64 lanes x 16 B contiguous per load instruction);
//   * codes become exact 16-bit floats B + D q by an and-or into the mantissa,
//     and v_dot2 accumulates x * (B + D q) in fp32; the group's zero point and
//     the magic offset B fold into one fused multiply-add with sum(x):
//       sum x (q - z) = acc / D - (B / D + z) * sum(x);
//   * the per-group fp16 scale multiplies that chunk result in fp32, and a
//     64-lane shuffle reduction finishes the row.

#include "common.hpp"
#include "device.hpp"
#include "launch.hpp"

namespace qlin {

namespace {

constexpr int kWaves = 8;                 // waves (= output rows) per workgroup
constexpr int kThreads = 64 * kWaves;

// Value of lane `src` of v (ds_bpermute through the LDS crossbar).
__device__ __forceinline__ uint32_t lane_value(uint32_t v, int src) {
  return static_cast<uint32_t>(__builtin_amdgcn_ds_bpermute(src << 2, static_cast<int>(v)));
}

// One wavefront per output row; lane l reads chunks l, l + 64, ... so every load
// instruction covers 1 KB of contiguous packed words.  Per row the wave loads
// its scales and zero words once, coalesced (lane i holds scale i + 64t and
// zero word i); each chunk then picks its group's values with a cross-lane
// read instead of two more memory instructions.  The activation loads for the
// LDS staging are issued before the weight loads (vector loads return in order)
// so the staging overlaps the weight stream.
template <int MT, int BPL, typename Codec, bool XBF16, int OUTK>
__global__ __launch_bounds__(kThreads) void w4_gemv_kernel(
    const uint16_t* __restrict__ X, int M, int K,
    const uint32_t* __restrict__ qweight, const uint16_t* __restrict__ scales,
    const uint32_t* __restrict__ qzeros, int N, int G, void* __restrict__ Y) {
  extern __shared__ uint4 smem[];
  const int C = K >> 5;                        // chunks per row
  uint4* xl = smem;                            // [MT][4][C] activation pairs
  float* xs = reinterpret_cast<float*>(smem + static_cast<size_t>(MT) * 4 * C);   // [MT][C]

  const int lane = threadIdx.x & 63;
  const int n = blockIdx.x * kWaves + (threadIdx.x >> 6);
  const bool nok = n < N;
  const int ng = K / G, nzw = (ng + 7) >> 3;
  const int cshift = __builtin_ctz(static_cast<unsigned>(G >> 5));

  // ---- 1. activation loads for the staging (up to two 32-value items per thread)
  const int items = M * C;
  uint4 xv[2][4];
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int it = threadIdx.x + q * kThreads;
    if (it < items) {
      const int m = it / C, c = it - m * C;
      const uint4* src = reinterpret_cast<const uint4*>(X + static_cast<size_t>(m) * K) + 4 * c;
#pragma unroll
      for (int i = 0; i < 4; ++i) xv[q][i] = src[i];
    }
  }

  // ---- 2. weights, then this row's scales and zero words
  const size_t nn = nok ? static_cast<size_t>(n) : 0;
  const uint4* qrow = reinterpret_cast<const uint4*>(qweight + nn * (K >> 3));
  uint4 w[BPL];
#pragma unroll
  for (int b = 0; b < BPL; ++b) {
    const int c = 64 * b + lane;
    if (nok && c < C) w[b] = load_stream16(qrow + c);
  }
  // scale registers: lane i of register t holds the scale of group 64t + i
  // (a row has at most one group per chunk, so BPL registers always suffice)
  constexpr int SV = BPL;
  uint32_t sv[SV];
  uint32_t zv = 0;
  const uint16_t* srow = scales + nn * ng;
#pragma unroll
  for (int t = 0; t < SV; ++t) {
    const int g = 64 * t + lane;
    sv[t] = 0u;
    if (64 * t < ng && nok && g < ng) sv[t] = static_cast<uint32_t>(srow[g]);
  }
  if (nok && lane < nzw) zv = qzeros[nn * nzw + lane];

  // ---- 3. finish staging the activations
  for (int q = 0; q * kThreads < items; ++q) {
    const int it = threadIdx.x + q * kThreads;
    if (it < items) {
      const int m = it / C, c = it - m * C;
      uint4 v4[4];
      if (q < 2) {
#pragma unroll
        for (int i = 0; i < 4; ++i) v4[i] = xv[q & 1][i];
      } else {
        const uint4* src = reinterpret_cast<const uint4*>(X + static_cast<size_t>(m) * K) + 4 * c;
#pragma unroll
        for (int i = 0; i < 4; ++i) v4[i] = src[i];
      }
      // sum of the 32 activations: dot products with (1, 1) pairs
      const uint32_t ones = XBF16 ? 0x3F803F80u : 0x3C003C00u;
      float sum = 0.0f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t u[4] = {v4[i].x, v4[i].y, v4[i].z, v4[i].w};
        uint32_t P[4];
        pair_up(u, P);
        xl[(static_cast<size_t>(m) * 4 + i) * C + c] = make_uint4(P[0], P[1], P[2], P[3]);
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) sum = Codec::dot(u[jj], ones, sum);
      }
      xs[m * C + c] = sum;
    }
  }
  __syncthreads();
  if (!nok) return;

  // ---- 4. compute
  float res[MT];
#pragma unroll
  for (int m = 0; m < MT; ++m) res[m] = 0.0f;
#pragma unroll
  for (int b = 0; b < BPL; ++b) {
    const int c = 64 * b + lane;
    // cross-lane reads with every lane active (a read from a lane that is
    // inactive in a divergent branch returns 0): lanes past the row end read
    // the last group's values and discard them
    const int g = min(c, C - 1) >> cshift;
    uint32_t sbits = 0;
#pragma unroll
    for (int t = 0; t < SV; ++t) {
      if (64 * t < ng) {                             // uniform: registers holding real groups
        const uint32_t v = lane_value(sv[t], g & 63);
        if ((g >> 6) == t) sbits = v;
      }
    }
    const uint32_t zw = lane_value(zv, g >> 3);
    if (c < C) {
      const float s = f16_bits_to_f32(static_cast<uint16_t>(sbits));
      const float zc = Codec::B_OVER_D + static_cast<float>((zw >> (4 * (g & 7))) & 15u);
      uint32_t p[4][4];
      Codec::unpack(w[b].x, p[0]);
      Codec::unpack(w[b].y, p[1]);
      Codec::unpack(w[b].z, p[2]);
      Codec::unpack(w[b].w, p[3]);
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        if (m < M) {
          float acc = 0.0f;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const uint4 xp = xl[(static_cast<size_t>(m) * 4 + i) * C + c];
            acc = Codec::dot(p[i][0], xp.x, acc);
            acc = Codec::dot(p[i][1], xp.y, acc);
            acc = Codec::dot(p[i][2], xp.z, acc);
            acc = Codec::dot(p[i][3], xp.w, acc);
          }
          const float t = fmaf(acc, Codec::INV_D, -zc * xs[m * C + c]);
          res[m] = fmaf(s, t, res[m]);
        }
      }
    }
  }
  // ---- 5. reduce over the wave and store
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    if (m < M) {
      const float v = wave_sum(res[m]);
      if (lane == 0) store_out<OUTK>(Y, static_cast<size_t>(m) * N + n, v);
    }
  }
}

template <int MT, int BPL, typename Codec, bool XBF16, int OUTK>
void launch_t(const W4Args& a, hipStream_t stream) {
  const int C = a.K >> 5;
  const size_t lds = static_cast<size_t>(MT) * 4 * C * 16 + static_cast<size_t>(MT) * C * 4;
  const int grid = (a.N + kWaves - 1) / kWaves;
  hipLaunchKernelGGL((w4_gemv_kernel<MT, BPL, Codec, XBF16, OUTK>), dim3(grid), dim3(kThreads), lds, stream,
                     static_cast<const uint16_t*>(a.X), a.M, a.K, a.qweight, a.scales, a.qzeros, a.N, a.G, a.Y);
}

template <int MT, int BPL>
void launch_b(const W4Args& a, hipStream_t stream) {
  const bool bf = a.x_dtype == QLIN_BF16;
  const int ok = a.y_dtype == QLIN_F16 ? OUT_F16 : (a.y_dtype == QLIN_BF16 ? OUT_BF16 : OUT_F32);
  if (!bf) {
    if (ok == OUT_F16) launch_t<MT, BPL, W4F16, false, OUT_F16>(a, stream);
    else if (ok == OUT_BF16) launch_t<MT, BPL, W4F16, false, OUT_BF16>(a, stream);
    else launch_t<MT, BPL, W4F16, false, OUT_F32>(a, stream);
  } else {
    if (ok == OUT_F16) launch_t<MT, BPL, W4BF16, true, OUT_F16>(a, stream);
    else if (ok == OUT_BF16) launch_t<MT, BPL, W4BF16, true, OUT_BF16>(a, stream);
    else launch_t<MT, BPL, W4BF16, true, OUT_F32>(a, stream);
  }
}

template <int MT>
void launch_m(const W4Args& a, hipStream_t stream) {
  // blocks of 64 chunks per row (one per lane); the whole row is held in flight
  const int blocks = ((a.K >> 5) + 63) / 64;
  if (blocks <= 1) launch_b<MT, 1>(a, stream);
  else if (blocks <= 2) launch_b<MT, 2>(a, stream);
  else if (blocks <= 4) launch_b<MT, 4>(a, stream);
  else if (blocks <= 6) launch_b<MT, 6>(a, stream);
  else launch_b<MT, 8>(a, stream);
}

// Debug: codes recovered from the same and-or unpack the GEMV uses (the pair
// (n_j, n_{j+4}) of register j), zeros from the same nibble extraction.
__global__ void w4_unpack_kernel(const uint32_t* __restrict__ qweight, const uint32_t* __restrict__ qzeros,
                                 int N, int K, int G, uint8_t* __restrict__ codes, uint8_t* __restrict__ zeros) {
  const size_t words = static_cast<size_t>(N) * (K >> 3);
  for (size_t i = blockIdx.x * static_cast<size_t>(blockDim.x) + threadIdx.x; i < words;
       i += static_cast<size_t>(gridDim.x) * blockDim.x) {
    uint32_t p[4];
    W4F16::unpack(qweight[i], p);
    uint8_t* dst = codes + i * 8;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      dst[j] = static_cast<uint8_t>(W4F16::code_of(static_cast<uint16_t>(p[j])));
      dst[j + 4] = static_cast<uint8_t>(W4F16::code_of(static_cast<uint16_t>(p[j] >> 16)));
    }
  }
  const int ng = K / G, nzw = (ng + 7) >> 3;
  const size_t nz = static_cast<size_t>(N) * ng;
  for (size_t i = blockIdx.x * static_cast<size_t>(blockDim.x) + threadIdx.x; i < nz;
       i += static_cast<size_t>(gridDim.x) * blockDim.x) {
    const size_t n = i / ng;
    const int g = static_cast<int>(i - n * ng);
    zeros[i] = static_cast<uint8_t>((qzeros[n * nzw + (g >> 3)] >> (4 * (g & 7))) & 15u);
  }
}

}  // namespace

void w4_unpack_launch(const uint32_t* qweight, const uint32_t* qzeros, int N, int K, int G,
                      uint8_t* codes, uint8_t* zeros, hipStream_t stream) {
  hipLaunchKernelGGL(w4_unpack_kernel, dim3(1024), dim3(256), 0, stream, qweight, qzeros, N, K, G, codes, zeros);
}

size_t w4_gemv_lds_bytes(int M, int K) {
  const size_t MT = M <= 1 ? 1 : M <= 2 ? 2 : M <= 4 ? 4 : M <= 8 ? 8 : 16;
  const size_t C = static_cast<size_t>(K) / 32;
  return MT * 4 * C * 16 + MT * C * 4;
}

bool w4_gemv_supported(int M, int K, int G) {
  // one pass holds at most 8 blocks of 64 chunks per row (K <= 16384)
  return M <= 16 && K <= 16384 && w4_gemv_lds_bytes(M, K) <= 64 * 1024 && G >= 32;
}

void w4_gemv_launch(const W4Args& a, hipStream_t stream) {
  if (a.M <= 1) launch_m<1>(a, stream);
  else if (a.M <= 2) launch_m<2>(a, stream);
  else if (a.M <= 4) launch_m<4>(a, stream);
  else if (a.M <= 8) launch_m<8>(a, stream);
  else launch_m<16>(a, stream);
}

}  // namespace qlin
