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

constexpr int kThreads = 256;
constexpr int kUnroll = 4;

template <int MT, typename Codec, bool XBF16, int OUTK>
__global__ __launch_bounds__(kThreads) void w4_gemv_kernel(
    const uint16_t* __restrict__ X, int M, int K,
    const uint32_t* __restrict__ qweight, const uint16_t* __restrict__ scales,
    const uint32_t* __restrict__ qzeros, int N, int G, void* __restrict__ Y) {
  extern __shared__ uint4 smem[];
  const int C = K >> 5;                 // chunks per row
  uint4* xl = smem;                     // [MT][4][C] activation pairs
  float* xs = reinterpret_cast<float*>(smem + static_cast<size_t>(MT) * 4 * C);   // [MT][C]

  // ---- stage activations: one chunk (32 values) per item
  for (int it = threadIdx.x; it < M * C; it += kThreads) {
    const int m = it / C, c = it - m * C;
    const uint4* src = reinterpret_cast<const uint4*>(X + static_cast<size_t>(m) * K) + 4 * c;
    float sum = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint4 v = src[i];
      const uint32_t u[4] = {v.x, v.y, v.z, v.w};
      uint32_t P[4];
      pair_up(u, P);
      xl[(static_cast<size_t>(m) * 4 + i) * C + c] = make_uint4(P[0], P[1], P[2], P[3]);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if constexpr (XBF16) {
          sum += bf16_bits_to_f32(static_cast<uint16_t>(u[j])) + bf16_bits_to_f32(static_cast<uint16_t>(u[j] >> 16));
        } else {
          sum += f16_bits_to_f32(static_cast<uint16_t>(u[j])) + f16_bits_to_f32(static_cast<uint16_t>(u[j] >> 16));
        }
      }
    }
    xs[m * C + c] = sum;
  }
  __syncthreads();

  const int lane = threadIdx.x & 63;
  const int wave = blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
  const int nwaves = gridDim.x * (kThreads / 64);
  const int ng = K / G, nzw = (ng + 7) >> 3, cpg = G >> 5;

  for (int n = wave; n < N; n += nwaves) {
    const uint4* qrow = reinterpret_cast<const uint4*>(qweight + static_cast<size_t>(n) * (K >> 3));
    const uint16_t* srow = scales + static_cast<size_t>(n) * ng;
    const uint32_t* zrow = qzeros + static_cast<size_t>(n) * nzw;
    float res[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m) res[m] = 0.0f;

    for (int c0 = lane; c0 < C; c0 += 64 * kUnroll) {
      uint4 w[kUnroll];
      float s[kUnroll], zc[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int c = c0 + 64 * u;
        if (c < C) {
          w[u] = load_stream16(qrow + c);
          const int g = c / cpg;
          s[u] = f16_bits_to_f32(srow[g]);
          zc[u] = Codec::B_OVER_D + static_cast<float>((zrow[g >> 3] >> (4 * (g & 7))) & 15u);
        }
      }
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int c = c0 + 64 * u;
        if (c < C) {
          uint32_t p[4][4];
          Codec::unpack(w[u].x, p[0]);
          Codec::unpack(w[u].y, p[1]);
          Codec::unpack(w[u].z, p[2]);
          Codec::unpack(w[u].w, p[3]);
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
              const float t = fmaf(acc, Codec::INV_D, -zc[u] * xs[m * C + c]);
              res[m] = fmaf(s[u], t, res[m]);
            }
          }
        }
      }
    }
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      if (m < M) {
        const float r = wave_sum(res[m]);
        if (lane == 0) store_out<OUTK>(Y, static_cast<size_t>(m) * N + n, r);
      }
    }
  }
}

template <int MT, typename Codec, bool XBF16, int OUTK>
void launch_t(const W4Args& a, hipStream_t stream) {
  const int C = a.K >> 5;
  const size_t lds = static_cast<size_t>(MT) * 4 * C * 16 + static_cast<size_t>(MT) * C * 4;
  const int rows_per_wg = 2 * (kThreads / 64);
  int grid = (a.N + rows_per_wg - 1) / rows_per_wg;
  if (grid > 1024) grid = 1024;
  hipLaunchKernelGGL((w4_gemv_kernel<MT, Codec, XBF16, OUTK>), dim3(grid), dim3(kThreads), lds, stream,
                     static_cast<const uint16_t*>(a.X), a.M, a.K, a.qweight, a.scales, a.qzeros, a.N, a.G, a.Y);
}

template <int MT>
void launch_m(const W4Args& a, hipStream_t stream) {
  const bool bf = a.x_dtype == QLIN_BF16;
  const int ok = a.y_dtype == QLIN_F16 ? OUT_F16 : (a.y_dtype == QLIN_BF16 ? OUT_BF16 : OUT_F32);
  if (!bf) {
    if (ok == OUT_F16) launch_t<MT, W4F16, false, OUT_F16>(a, stream);
    else if (ok == OUT_BF16) launch_t<MT, W4F16, false, OUT_BF16>(a, stream);
    else launch_t<MT, W4F16, false, OUT_F32>(a, stream);
  } else {
    if (ok == OUT_F16) launch_t<MT, W4BF16, true, OUT_F16>(a, stream);
    else if (ok == OUT_BF16) launch_t<MT, W4BF16, true, OUT_BF16>(a, stream);
    else launch_t<MT, W4BF16, true, OUT_F32>(a, stream);
  }
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
  int MT = M <= 1 ? 1 : M <= 2 ? 2 : M <= 4 ? 4 : M <= 8 ? 8 : 16;
  const size_t C = static_cast<size_t>(K) / 32;
  return MT * 4 * C * 16 + MT * C * 4;
}

void w4_gemv_launch(const W4Args& a, hipStream_t stream) {
  if (a.M <= 1) launch_m<1>(a, stream);
  else if (a.M <= 2) launch_m<2>(a, stream);
  else if (a.M <= 4) launch_m<4>(a, stream);
  else if (a.M <= 8) launch_m<8>(a, stream);
  else launch_m<16>(a, stream);
}

}  // namespace qlin
