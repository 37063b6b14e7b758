// W4 dequant -> fp16 MFMA product for small batches (4 .. 16 rows, groups of
// 128 or 256), gfx950.
//
// Y[m][n] = sum_g S[n][g] * sum_{k in g} x[m][k] * (q[n][k] - z[n][g])
//
// At small batch the layer is bound by memory bandwidth (GPTQ bulletin,
// "İddia ve Gerçeklik"), and an N-tiled GEMM runs out of output tiles long
// before it fills 256 compute units; splitting K across workgroups then needs
// a global hand-off of partial sums whose latency dominates a layer of a few
// microseconds.  Here the K split stays inside one workgroup:
//   * a workgroup owns 16 output columns; its NWV (4) waves each take a
//     contiguous run of 128-wide K blocks of those columns and accumulate a
//     16 x 16 tile (two for TM = 2) with v_mfma_f32_16x16x32_f16; the partial
//     tiles are added in wave order through LDS at the end (deterministic, no
//     atomics, no workspace); four-wave workgroups keep every workgroup of an
//     11008-column layer resident at once;
//   * B operand: per K block a lane loads one 16-byte piece (4 packed words of
//     its column) and turns each word into 8 fp16 weights s * (q - z) (q - z
//     exact, one rounding of the product), one word per matrix instruction;
//   * A operand: straight from global memory into registers (16 bytes = 8
//     consecutive k per lane and instruction; rows past M re-read row M - 1);
//     within a 128-wide block, instruction i of lane quarter h covers the
//     8-wide chunk 4 h + i for both operands;
//   * packed words, scales, zeros and activations are fetched D blocks ahead
//     into register rings with unconditional (clamped) loads, so the compiler's
//     in-order wait counts never drain the rings.

#include <algorithm>
#include <type_traits>

#include "common.hpp"
#include "device.hpp"
#include "launch.hpp"
#include "splitk.hpp"

namespace qlin {

namespace {

constexpr int kCols = 16;           // output columns per workgroup

// Eight fp16 weights s * (q - z) in natural k order from one packed word.
__device__ __forceinline__ h8_t dequant_word(uint32_t w, h2_t zz, h2_t ss) {
  const uint32_t t = w >> 4;
  h8_t b;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    // byte j of w holds codes 2j (low nibble) and 2j + 1; t's byte j has code 2j + 1 low
    const uint32_t sel = static_cast<uint32_t>(j) | (0x0Cu << 8) | (static_cast<uint32_t>(4 + j) << 16) | (0x0Cu << 24);
    const uint32_t pr = __builtin_amdgcn_perm(t, w, sel);
    const h2_t d = (bitcast<h2_t>(and_or(pr, 0x000F000Fu, 0x64006400u)) - zz) * ss;
    b[2 * j] = d[0];
    b[2 * j + 1] = d[1];
  }
  return b;
}

__device__ __forceinline__ uint32_t bf16x2_to_f16x2(uint32_t u) {
  const float lo = bitcast<float>(u << 16);
  const float hi = bitcast<float>(u & 0xFFFF0000u);
  return bitcast<uint32_t>(__builtin_amdgcn_cvt_pkrtz(lo, hi));
}

template <int NWV, int TM, int D, bool XBF16, int OUTK>
__global__ __launch_bounds__(64 * NWV) void w4_skinny_kernel(const uint16_t* X, int M, int K,
                                                               const uint32_t* qweight, const uint16_t* scales,
                                                               const uint32_t* qzeros, int N, int gsh, void* Y) {
  __shared__ f32x4_t red[NWV][TM][64];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform: scalar loop control
  const int col = lane & 15, h = lane >> 4;
  const int n0 = blockIdx.x * kCols;
  const int n = n0 + col;
  const size_t nn = static_cast<size_t>(min(n, N - 1));
  const int nb = K >> 7;                        // 128-wide K blocks
  const int ng = K >> (7 + gsh);
  const int nzw = (ng + 7) >> 3;
  const int b0 = (wv * nb) / NWV, b1 = ((wv + 1) * nb) / NWV;
  const uint4* qrow = reinterpret_cast<const uint4*>(qweight + nn * (K >> 3));
  const uint16_t* srow = scales + nn * ng;
  const uint32_t* zrow = qzeros + nn * nzw;

  f32x4_t acc[TM];
#pragma unroll
  for (int t = 0; t < TM; ++t) acc[t] = f32x4_t{};

  if (b0 < b1) {
    const int blast = b1 - 1;
    uint4 wq[D];
    uint4 av[D][TM][4];
    uint32_t sv[D], zv[D];
    // block b: the lane's 4 words 4h .. 4h+3 of its column; scale and zero
    // word of the block's group; activations of chunks 4h + i, rows
    // col (+ 16 t) of the batch, clamped to M - 1
    auto load = [&](int b, uint4& w, uint4 (&a)[TM][4], uint32_t& s, uint32_t& z) {
      w = qrow[4 * b + h];
      const int g = b >> gsh;
      s = srow[g];
      z = zrow[g >> 3];
#pragma unroll
      for (int t = 0; t < TM; ++t) {
        const int m = min(16 * t + col, M - 1);
        const uint4* xr = reinterpret_cast<const uint4*>(X + static_cast<size_t>(m) * K + 128 * b);
#pragma unroll
        for (int i = 0; i < 4; ++i) a[t][i] = xr[4 * h + i];
      }
    };
    auto compute = [&](int b, const uint4& w, const uint4 (&a)[TM][4], uint32_t s, uint32_t zw) {
      const int g = b >> gsh;
      const uint32_t z = (zw >> (4 * (g & 7))) & 15u;
      const _Float16 zb = static_cast<_Float16>(1024.0f + static_cast<float>(z));
      const h2_t zz = {zb, zb};
      const _Float16 sh = bitcast<_Float16>(static_cast<uint16_t>(s));
      const h2_t ss = {sh, sh};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t word = i == 0 ? w.x : i == 1 ? w.y : i == 2 ? w.z : w.w;
        const h8_t bw = dequant_word(word, zz, ss);
#pragma unroll
        for (int t = 0; t < TM; ++t) {
          uint4 av4 = a[t][i];
          if constexpr (XBF16) {
            av4.x = bf16x2_to_f16x2(av4.x);
            av4.y = bf16x2_to_f16x2(av4.y);
            av4.z = bf16x2_to_f16x2(av4.z);
            av4.w = bf16x2_to_f16x2(av4.w);
          }
          acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(bitcast<h8_t>(av4), bw, acc[t], 0, 0, 0);
        }
      }
    };
#pragma unroll
    for (int j = 0; j < D - 1; ++j) load(min(b0 + j, blast), wq[j], av[j], sv[j], zv[j]);
    // ring step for block b in slot S: fetch block b + D - 1 into the slot freed
    // by block b - 1, then consume block b
    auto step = [&](auto slot_c, int b) {
      constexpr int S = decltype(slot_c)::value;
      constexpr int SF = (S + D - 1) % D;
      load(min(b + D - 1, blast), wq[SF], av[SF], sv[SF], zv[SF]);
      __builtin_amdgcn_sched_barrier(0);     // keep the prefetch issued ahead of the math
      compute(b, wq[S], av[S], sv[S], zv[S]);
    };
    int b = b0;
    while (sk_run_steps<0, D>(step, b, b1)) {
    }
  }

  // fixed-order sum of the 8 waves' tiles; lane l of the tile holds column
  // l % 16, rows 4 (l / 16) + r
#pragma unroll
  for (int t = 0; t < TM; ++t) red[wv][t][lane] = acc[t];
  __syncthreads();
  if (wv < TM) {
    const int t = wv;
    f32x4_t tot = red[0][t][lane];
#pragma unroll
    for (int w = 1; w < NWV; ++w) tot += red[w][t][lane];
    if (n < N) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = 16 * t + 4 * h + r;
        if (m < M) store_out<OUTK>(Y, static_cast<size_t>(m) * N + n, tot[r]);
      }
    }
  }
}

template <int NWV, int TM, int D, bool XBF16, int OUTK>
void launch_k(const W4Args& a, hipStream_t stream) {
  const int gsh = a.G == 256 ? 1 : 0;
  hipLaunchKernelGGL((w4_skinny_kernel<NWV, TM, D, XBF16, OUTK>), dim3((a.N + kCols - 1) / kCols), dim3(64 * NWV), 0,
                     stream, static_cast<const uint16_t*>(a.X), a.M, a.K, a.qweight, a.scales, a.qzeros, a.N, gsh,
                     a.Y);
}

template <int NWV, int TM, int D, bool XBF16>
void launch_o(const W4Args& a, hipStream_t stream) {
  if (a.y_dtype == QLIN_F16) launch_k<NWV, TM, D, XBF16, OUT_F16>(a, stream);
  else if (a.y_dtype == QLIN_BF16) launch_k<NWV, TM, D, XBF16, OUT_BF16>(a, stream);
  else launch_k<NWV, TM, D, XBF16, OUT_F32>(a, stream);
}

template <int NWV, int TM, int D>
void launch_x(const W4Args& a, hipStream_t stream) {
  if (a.x_dtype == QLIN_BF16) launch_o<NWV, TM, D, true>(a, stream);
  else launch_o<NWV, TM, D, false>(a, stream);
}

}  // namespace

bool w4_skinny_supported(int M, int K, int G) { return M >= 1 && M <= 16 && (G == 128 || G == 256) && K % 128 == 0; }

void w4_skinny_launch(const W4Args& a, hipStream_t stream) { launch_x<4, 1, 4>(a, stream); }

}  // namespace qlin
