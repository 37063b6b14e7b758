// W4 MFMA GEMM for groups of 32 or 64 codes, gfx950.
//
// At large batch the weight-only layer turns compute-bound and the dequant
// work is what erodes the gain (GPTQ bulletin, "İddia ve Gerçeklik").  With
// small groups the per-group rescale is cheap relative to the few matrix
// instructions per group, so this kernel keeps the codes exact:
//   * B operand: each lane turns one packed word (8 codes of one output column)
//     into eight exact fp16 integers q - z: an and-or places each code in the
//     mantissa of 1024.0 (1024 + q) and one packed fp16 subtraction removes
//     1024 + z.  No rounding happens anywhere;
//   * A operand: the fp16 activation tile of one quantization group (BM rows x
//     G) staged in LDS (bf16 inputs arrive as a row-scaled fp16 copy whose
//     power of two the epilogue puts back);
//   * v_mfma_f32_32x32x16_f16 accumulates sum x (q - z) of one group in fp32,
//     which is then scaled by the group's fp16 scale into the running fp32
//     result (one fused multiply-add per output element and group);
//   * the epilogue rounds once to the output dtype.

#include "common.hpp"
#include "device.hpp"
#include "launch.hpp"

namespace qlin {

namespace {

constexpr int kThreads = 256;   // 4 waves

// One K step per quantization group (GW = G / 16 packed words per lane, one per
// MFMA step), no prefetch.  Groups of 128 and 256 take the stream-K kernel.
template <int TM, int GW, int OUTK>
__global__ __launch_bounds__(kThreads) void w4_gemm_group_kernel(
    const uint16_t* __restrict__ X, int M, int K,
    const uint32_t* __restrict__ qweight, const uint16_t* __restrict__ scales,
    const uint32_t* __restrict__ qzeros, int N, void* __restrict__ Y, const int* __restrict__ rowexp) {
  constexpr int G = GW * 16;
  constexpr int BM = 32 * TM;
  constexpr int WPG = G / 8;                 // words (of 8 codes) per group
  constexpr int ROW = WPG * 8 + 8;           // LDS row stride in fp16 (+16 B pad)
  extern __shared__ uint4 smem[];
  _Float16* As = reinterpret_cast<_Float16*>(smem);

  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int col = lane & 31, half = lane >> 5;
  const int m0 = blockIdx.y * BM;
  const int n = blockIdx.x * 128 + wv * 32 + col;
  const bool n_ok = n < N;
  const int ng = K / G, nzw = (ng + 7) >> 3;

  const uint32_t* qrow = qweight + static_cast<size_t>(n_ok ? n : 0) * (K >> 3);
  const uint16_t* srow = scales + static_cast<size_t>(n_ok ? n : 0) * ng;
  const uint32_t* zrow = qzeros + static_cast<size_t>(n_ok ? n : 0) * nzw;

  f32x16_t acc[TM];
#pragma unroll
  for (int t = 0; t < TM; ++t) acc[t] = f32x16_t{};

  for (int g = 0; g < ng; ++g) {
    // ---- stage A: rows m0..m0+BM, k in group g, permuted within each word
    __syncthreads();
    for (int it = threadIdx.x; it < BM * WPG; it += kThreads) {
      const int r = it / WPG, wd = it - r * WPG;
      const int m = m0 + r;
      uint32_t u[4] = {0u, 0u, 0u, 0u};
      if (m < M) {
        const uint4 v = *reinterpret_cast<const uint4*>(X + static_cast<size_t>(m) * K + g * G + wd * 8);
        u[0] = v.x; u[1] = v.y; u[2] = v.z; u[3] = v.w;
      }
      uint32_t P[4];
      pair_up(u, P);
      *reinterpret_cast<uint4*>(As + r * ROW + wd * 8) = make_uint4(P[0], P[1], P[2], P[3]);
    }
    __syncthreads();

    // ---- B: this lane's GW words of the group, zero point, scale
    uint32_t wq[GW];
    if (n_ok) {
      const uint32_t* src = qrow + g * WPG + half * GW;
#pragma unroll
      for (int i = 0; i < GW; i += 2) {
        const uint2 v = *reinterpret_cast<const uint2*>(src + i);
        wq[i] = v.x;
        wq[i + 1] = v.y;
      }
    } else {
#pragma unroll
      for (int i = 0; i < GW; ++i) wq[i] = 0x88888888u;   // any codes; the column is discarded
    }
    const uint32_t z = n_ok ? (zrow[g >> 3] >> (4 * (g & 7))) & 15u : 0u;
    const float s = n_ok ? f16_bits_to_f32(srow[g]) : 0.0f;
    const _Float16 zb = static_cast<_Float16>(1024.0f + static_cast<float>(z));
    const h2_t zz = {zb, zb};

    f32x16_t part[TM];
#pragma unroll
    for (int t = 0; t < TM; ++t) part[t] = f32x16_t{};
#pragma unroll
    for (int st = 0; st < GW; ++st) {
      const uint32_t w = wq[st];
      h8_t b;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t p = ((w >> (4 * j)) & 0x000F000Fu) | 0x64006400u;
        const h2_t d = bitcast<h2_t>(p) - zz;          // exact q - z
        b[2 * j] = d[0];
        b[2 * j + 1] = d[1];
      }
#pragma unroll
      for (int t = 0; t < TM; ++t) {
        const h8_t a = *reinterpret_cast<const h8_t*>(As + (32 * t + col) * ROW + (half * GW + st) * 8);
        part[t] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, part[t], 0, 0, 0);
      }
    }
#pragma unroll
    for (int t = 0; t < TM; ++t) acc[t] += s * part[t];
  }

  // ---- epilogue: lane holds column n, rows 8*(r/4) + 4*half + r%4 of each tile
  if (n_ok) {
    if (rowexp) {
      int ex[TM][16];
#pragma unroll
      for (int t = 0; t < TM; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) ex[t][r] = rowexp[min(m0 + 32 * t + 8 * (r >> 2) + 4 * half + (r & 3), M - 1)];
#pragma unroll
      for (int t = 0; t < TM; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[t][r] = ldexpf(acc[t][r], ex[t][r]);
    }
#pragma unroll
    for (int t = 0; t < TM; ++t) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = m0 + 32 * t + 8 * (r >> 2) + 4 * half + (r & 3);
        if (m < M) store_out<OUTK>(Y, static_cast<size_t>(m) * N + n, acc[t][r]);
      }
    }
  }
}

template <int TM, int GW>
void launch_small_o(const W4Args& a, hipStream_t stream) {
  constexpr int G = GW * 16, ROW = G + 8;
  const size_t lds = static_cast<size_t>(32 * TM) * ROW * 2;
  dim3 grid((a.N + 127) / 128, (a.M + 32 * TM - 1) / (32 * TM));
  const uint16_t* X = static_cast<const uint16_t*>(a.X);
  if (a.y_dtype == QLIN_F16)
    hipLaunchKernelGGL((w4_gemm_group_kernel<TM, GW, OUT_F16>), grid, dim3(kThreads), lds, stream,
                       X, a.M, a.K, a.qweight, a.scales, a.qzeros, a.N, a.Y, a.rowexp);
  else if (a.y_dtype == QLIN_BF16)
    hipLaunchKernelGGL((w4_gemm_group_kernel<TM, GW, OUT_BF16>), grid, dim3(kThreads), lds, stream,
                       X, a.M, a.K, a.qweight, a.scales, a.qzeros, a.N, a.Y, a.rowexp);
  else
    hipLaunchKernelGGL((w4_gemm_group_kernel<TM, GW, OUT_F32>), grid, dim3(kThreads), lds, stream,
                       X, a.M, a.K, a.qweight, a.scales, a.qzeros, a.N, a.Y, a.rowexp);
}

template <int GW>
void launch_small_g(const W4Args& a, hipStream_t stream) {
  // the A tile (32*TM rows x (G + 8) fp16) must stay within 64 KiB of LDS
  constexpr int TMAX = (GW * 16 + 8) * 2 * 32 * 4 <= 64 * 1024 ? 4 : 2;
  if (a.M <= 32) launch_small_o<1, GW>(a, stream);
  else if (a.M <= 64 || TMAX == 2) launch_small_o<2, GW>(a, stream);
  else launch_small_o<TMAX, GW>(a, stream);
}

}  // namespace

void w4_gemm_group_launch(const W4Args& a, hipStream_t stream) {
  if (a.G == 32) launch_small_g<2>(a, stream);
  else launch_small_g<4>(a, stream);
}

}  // namespace qlin
