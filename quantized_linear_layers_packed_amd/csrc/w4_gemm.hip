// W4 dequant -> fp16 MFMA GEMM for batches past the GEMV range, gfx950.
//
// At large batch the weight-only layer turns compute-bound and the dequant
// work is what erodes the gain (GPTQ bulletin, "İddia ve Gerçeklik"), so the
// weights are dequantized once per workgroup tile, in registers, and the
// products run on the matrix cores:
//   * B operand: each lane turns one packed word (8 codes of one output column)
//     into eight exact fp16 integers q - z: an and-or places each code in the
//     mantissa of 1024.0 (1024 + q) and one packed fp16 subtraction removes
//     1024 + z.  No rounding happens anywhere;
//   * A operand: the activation tile of one quantization group (BM rows x G)
//     is staged in LDS as fp16, already in the within-word order of the codes
//     (bf16 inputs are converted, exactly for values in fp16 range), double
//     buffered: the next group's activations and packed words are fetched
//     into registers while the current group is multiplied;
//   * v_mfma_f32_32x32x16_f16 accumulates sum x (q - z) of one group in fp32,
//     which is then scaled by the group's fp16 scale into the running fp32
//     result (one fused multiply-add per output element and group);
//   * the epilogue rounds once to the output dtype.
// Waves are arranged WM x WN over the workgroup tile; each wave owns TM x TN
// tiles of 32 x 32 outputs.

#include "common.hpp"
#include "device.hpp"
#include "launch.hpp"

namespace qlin {

namespace {

constexpr int kThreads = 256;   // 4 waves

__device__ __forceinline__ uint32_t to_f16_pair(uint32_t bfpair) {
  const float lo = bitcast<float>(bfpair << 16);
  const float hi = bitcast<float>(bfpair & 0xFFFF0000u);
  const h2_t h = {static_cast<_Float16>(lo), static_cast<_Float16>(hi)};
  return bitcast<uint32_t>(h);
}

// Eight fp16 values q - z from one packed word, in the order
// (n0, n4, n1, n5, n2, n6, n3, n7) that the activation staging uses.
__device__ __forceinline__ h8_t dequant_word(uint32_t w, h2_t zz) {
  const uint32_t mask = 0x000F000Fu;
  h8_t b;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t p = and_or(w >> (4 * j), mask, 0x64006400u);
    const h2_t d = bitcast<h2_t>(p) - zz;          // exact: (1024 + q) - (1024 + z)
    b[2 * j] = d[0];
    b[2 * j + 1] = d[1];
  }
  return b;
}

template <int WM, int WN, int TM, int TN, bool XBF16, int OUTK>
__global__ __launch_bounds__(kThreads) void w4_gemm_kernel(
    const uint16_t* __restrict__ X, int M, int K,
    const uint32_t* __restrict__ qweight, const uint16_t* __restrict__ scales,
    const uint32_t* __restrict__ qzeros, int N, int Gq, void* __restrict__ Y) {
  static_assert(WM * WN == 4, "four waves");
  constexpr int G = 128;                     // K step of the tile (quantization group 128 or 256)
  constexpr int WPG = G / 8;                 // packed words per column per group (16)
  constexpr int BM = WM * TM * 32, BN = WN * TN * 32;
  constexpr int ROW = G + 8;                 // LDS row stride in fp16 (+16 B against bank conflicts)
  constexpr int APT = BM * WPG / kThreads;   // 16-byte activation pieces per thread per group
  static_assert(APT >= 1 && BM * WPG % kThreads == 0, "tile too small for the staging split");
  __shared__ __attribute__((aligned(16))) _Float16 As[2][BM * ROW];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = tid >> 6;
  const int wm = wv / WN, wn = wv % WN;
  const int col = lane & 31, half = lane >> 5;
  const int MB = (M + BM - 1) / BM;
  const int tile = xcd_tile(blockIdx.x, gridDim.x);
  const int m0 = (tile % MB) * BM;
  const int n0 = (tile / MB) * BN + wn * TN * 32;
  const int ng = K / G;                      // K steps
  const int nq = K / Gq, nzw = (nq + 7) >> 3; // quantization groups, zero words per row
  const int gsh = Gq == 256 ? 1 : 0;         // K step -> group index shift

  // this lane's output columns (one per N tile) and their packed rows
  const uint32_t* qrow[TN];
  const uint16_t* srow[TN];
  const uint32_t* zrow[TN];
  bool nok[TN];
#pragma unroll
  for (int t = 0; t < TN; ++t) {
    const int n = n0 + 32 * t + col;
    nok[t] = n < N;
    const size_t nn = nok[t] ? static_cast<size_t>(n) : 0;
    qrow[t] = qweight + nn * (K >> 3);
    srow[t] = scales + nn * nq;
    zrow[t] = qzeros + nn * nzw;
  }

  // ---- prefetch helpers
  uint4 av[APT];                                // raw activation pieces of the next group
  uint4 wq[TN][2];                              // 8 packed words (this lane's half of the group) per N tile
  auto load_a = [&](int g) {
#pragma unroll
    for (int p = 0; p < APT; ++p) {
      const int piece = tid + p * kThreads;
      const int r = piece / WPG, wd = piece - r * WPG;
      const int m = m0 + r;
      av[p] = (m < M) ? *reinterpret_cast<const uint4*>(X + static_cast<size_t>(m) * K + g * G + wd * 8)
                      : make_uint4(0u, 0u, 0u, 0u);
    }
  };
  auto store_a = [&](int buf) {
#pragma unroll
    for (int p = 0; p < APT; ++p) {
      const int piece = tid + p * kThreads;
      const int r = piece / WPG, wd = piece - r * WPG;
      uint32_t u[4] = {av[p].x, av[p].y, av[p].z, av[p].w};
      if constexpr (XBF16) {
#pragma unroll
        for (int j = 0; j < 4; ++j) u[j] = to_f16_pair(u[j]);
      }
      uint32_t P[4];
      pair_up(u, P);
      *reinterpret_cast<uint4*>(&As[buf][r * ROW + wd * 8]) = make_uint4(P[0], P[1], P[2], P[3]);
    }
  };
  auto load_b = [&](int g) {
#pragma unroll
    for (int t = 0; t < TN; ++t) {
      if (nok[t]) {
        const uint4* src = reinterpret_cast<const uint4*>(qrow[t] + g * WPG + half * (WPG / 2));
        wq[t][0] = load_stream16(src);
        wq[t][1] = load_stream16(src + 1);
      } else {
        wq[t][0] = wq[t][1] = make_uint4(0x88888888u, 0x88888888u, 0x88888888u, 0x88888888u);
      }
    }
  };

  f32x16_t acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int t = 0; t < TN; ++t) acc[i][t] = f32x16_t{};

  load_a(0);
  load_b(0);
  store_a(0);
  __syncthreads();

  for (int g = 0; g < ng; ++g) {
    const int buf = g & 1;
    // current group's packed words, zero points and scales
    uint4 wcur[TN][2];
    float sc[TN];
    h2_t zz[TN];
#pragma unroll
    for (int t = 0; t < TN; ++t) {
      wcur[t][0] = wq[t][0];
      wcur[t][1] = wq[t][1];
      const int gq = g >> gsh;
      const uint32_t z = nok[t] ? (zrow[t][gq >> 3] >> (4 * (gq & 7))) & 15u : 0u;
      sc[t] = nok[t] ? f16_bits_to_f32(srow[t][gq]) : 0.0f;
      const _Float16 zb = static_cast<_Float16>(1024.0f + static_cast<float>(z));
      zz[t] = h2_t{zb, zb};
    }
    // prefetch the next group
    if (g + 1 < ng) {
      load_a(g + 1);
      load_b(g + 1);
    }

    f32x16_t part[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int t = 0; t < TN; ++t) part[i][t] = f32x16_t{};

#pragma unroll
    for (int st = 0; st < WPG / 2; ++st) {
      h8_t b[TN];
#pragma unroll
      for (int t = 0; t < TN; ++t) {
        const uint4 q4 = wcur[t][st >> 2];
        const uint32_t w = (st & 3) == 0 ? q4.x : (st & 3) == 1 ? q4.y : (st & 3) == 2 ? q4.z : q4.w;
        b[t] = dequant_word(w, zz[t]);
      }
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const int r = (wm * TM + i) * 32 + col;
        const h8_t a = *reinterpret_cast<const h8_t*>(&As[buf][r * ROW + (half * (WPG / 2) + st) * 8]);
#pragma unroll
        for (int t = 0; t < TN; ++t) part[i][t] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b[t], part[i][t], 0, 0, 0);
      }
    }
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int t = 0; t < TN; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][t][r] = fmaf(sc[t], part[i][t][r], acc[i][t][r]);

    if (g + 1 < ng) {
      store_a(buf ^ 1);
      __syncthreads();
    }
  }

  // ---- epilogue: lane holds column n, rows 8*(r/4) + 4*half + r%4 of each tile
#pragma unroll
  for (int t = 0; t < TN; ++t) {
    if (!nok[t]) continue;
    const int n = n0 + 32 * t + col;
#pragma unroll
    for (int i = 0; i < TM; ++i) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = m0 + (wm * TM + i) * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
        if (m < M) store_out<OUTK>(Y, static_cast<size_t>(m) * N + n, acc[i][t][r]);
      }
    }
  }
}

template <int WM, int WN, int TM, int TN, bool XBF16>
void launch_o(const W4Args& a, hipStream_t stream) {
  constexpr int BM = WM * TM * 32, BN = WN * TN * 32;
  dim3 grid(((a.N + BN - 1) / BN) * ((a.M + BM - 1) / BM));
  const uint16_t* X = static_cast<const uint16_t*>(a.X);
  if (a.y_dtype == QLIN_F16)
    hipLaunchKernelGGL((w4_gemm_kernel<WM, WN, TM, TN, XBF16, OUT_F16>), grid, dim3(kThreads), 0, stream,
                       X, a.M, a.K, a.qweight, a.scales, a.qzeros, a.N, a.G, a.Y);
  else if (a.y_dtype == QLIN_BF16)
    hipLaunchKernelGGL((w4_gemm_kernel<WM, WN, TM, TN, XBF16, OUT_BF16>), grid, dim3(kThreads), 0, stream,
                       X, a.M, a.K, a.qweight, a.scales, a.qzeros, a.N, a.G, a.Y);
  else
    hipLaunchKernelGGL((w4_gemm_kernel<WM, WN, TM, TN, XBF16, OUT_F32>), grid, dim3(kThreads), 0, stream,
                       X, a.M, a.K, a.qweight, a.scales, a.qzeros, a.N, a.G, a.Y);
}

template <bool XBF16>
void launch_x(const W4Args& a, hipStream_t stream) {
  // Tile choice: small batches stream the weights (all four waves side by side
  // along N, one 32-row tile); large batches use 2 x 2 waves of 64 x 32 (a
  // 128 x 64 tile keeps about one workgroup per CU busy on 8192-wide layers).
  if (a.M <= 32) launch_o<1, 4, 1, 1, XBF16>(a, stream);
  else if (a.M <= 64) launch_o<1, 4, 2, 1, XBF16>(a, stream);
  else launch_o<2, 2, 2, 1, XBF16>(a, stream);
}

// Groups of 32 or 64 codes: one K step per quantization group (GW = G / 16
// packed words per lane, one per MFMA step), no prefetch.  Used only for those
// group sizes; 128 and 256 take the pipelined kernel above.
template <int TM, int GW, bool XBF16, int OUTK>
__global__ __launch_bounds__(kThreads) void w4_gemm_group_kernel(
    const uint16_t* __restrict__ X, int M, int K,
    const uint32_t* __restrict__ qweight, const uint16_t* __restrict__ scales,
    const uint32_t* __restrict__ qzeros, int N, void* __restrict__ Y) {
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
        if constexpr (XBF16) {
#pragma unroll
          for (int j = 0; j < 4; ++j) u[j] = to_f16_pair(u[j]);
        }
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

template <int TM, int GW, bool XBF16>
void launch_small_o(const W4Args& a, hipStream_t stream) {
  constexpr int G = GW * 16, ROW = G + 8;
  const size_t lds = static_cast<size_t>(32 * TM) * ROW * 2;
  dim3 grid((a.N + 127) / 128, (a.M + 32 * TM - 1) / (32 * TM));
  const void* X = a.X;
  if (a.y_dtype == QLIN_F16)
    hipLaunchKernelGGL((w4_gemm_group_kernel<TM, GW, XBF16, OUT_F16>), grid, dim3(kThreads), lds, stream,
                       static_cast<const uint16_t*>(X), a.M, a.K, a.qweight, a.scales, a.qzeros, a.N, a.Y);
  else if (a.y_dtype == QLIN_BF16)
    hipLaunchKernelGGL((w4_gemm_group_kernel<TM, GW, XBF16, OUT_BF16>), grid, dim3(kThreads), lds, stream,
                       static_cast<const uint16_t*>(X), a.M, a.K, a.qweight, a.scales, a.qzeros, a.N, a.Y);
  else
    hipLaunchKernelGGL((w4_gemm_group_kernel<TM, GW, XBF16, OUT_F32>), grid, dim3(kThreads), lds, stream,
                       static_cast<const uint16_t*>(X), a.M, a.K, a.qweight, a.scales, a.qzeros, a.N, a.Y);
}

template <int GW>
void launch_small_g(const W4Args& a, hipStream_t stream) {
  // the A tile (32*TM rows x (G + 8) fp16) must stay within 64 KiB of LDS
  constexpr int TMAX = (GW * 16 + 8) * 2 * 32 * 4 <= 64 * 1024 ? 4 : 2;
  const bool bf = a.x_dtype == QLIN_BF16;
  if (a.M <= 32) { bf ? launch_small_o<1, GW, true>(a, stream) : launch_small_o<1, GW, false>(a, stream); }
  else if (a.M <= 64 || TMAX == 2) { bf ? launch_small_o<2, GW, true>(a, stream) : launch_small_o<2, GW, false>(a, stream); }
  else { bf ? launch_small_o<TMAX, GW, true>(a, stream) : launch_small_o<TMAX, GW, false>(a, stream); }
}

}  // namespace

void w4_gemm_launch(const W4Args& a, hipStream_t stream) {
  if (a.G == 32) { launch_small_g<2>(a, stream); return; }
  if (a.G == 64) { launch_small_g<4>(a, stream); return; }
  if (a.x_dtype == QLIN_BF16) launch_x<true>(a, stream);
  else launch_x<false>(a, stream);
}

}  // namespace qlin
