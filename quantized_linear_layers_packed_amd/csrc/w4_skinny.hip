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
//   * a workgroup owns CT tiles of 16 output columns (CT = 4 or 2 on wide
//     layers while that leaves at least 160 workgroups, else 1); its NWV (4)
//     waves each take a contiguous run of 128-wide K blocks of those columns
//     and accumulate a 16 x 16 tile per column tile (two for TM = 2) with
//     v_mfma_f32_16x16x32_f16, one activation fragment feeding the CT tiles;
//     the partial tiles are added in wave order through LDS at the end
//     (deterministic, no atomics, no workspace); four-wave workgroups keep
//     every workgroup of an 11008-column layer resident at once;
//   * B operand: per K block a lane loads one 16-byte piece (4 packed words of
//     its column) and turns each word into 8 fp16 weights s * (q - z) (q - z
//     exact, one rounding of the product), one word per matrix instruction;
//   * A operand: fp16 straight from global memory into registers (16 bytes =
//     8 consecutive k per lane and instruction; rows past M re-read row M - 1);
//     bf16 inputs arrive as a row-scaled fp16 copy, scaled back at the store;
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

constexpr int kCols = 16;           // output columns per column tile

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

template <int NWV, int TM, int D, int CT, int OUTK>
__global__ __launch_bounds__(64 * NWV) void w4_skinny_kernel(const uint16_t* X, int M, int K,
                                                               const uint32_t* qweight, const uint16_t* scales,
                                                               const uint32_t* qzeros, int N, int gsh, void* Y,
                                                               const int* rowexp) {
  __shared__ f32x4_t red[NWV][CT * TM][64];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform: scalar loop control
  const int col = lane & 15, h = lane >> 4;
  const int n0 = blockIdx.x * (CT * kCols);
  const int nb = K >> 7;                        // 128-wide K blocks
  const int ng = K >> (7 + gsh);
  const int nzw = (ng + 7) >> 3;
  const int b0 = (wv * nb) / NWV, b1 = ((wv + 1) * nb) / NWV;
  const uint4* qrow[CT];                        // column tile c: column n0 + 16 c + col
  const uint16_t* srow[CT];
  const uint32_t* zrow[CT];
#pragma unroll
  for (int c = 0; c < CT; ++c) {
    const size_t nn = static_cast<size_t>(min(n0 + kCols * c + col, N - 1));
    qrow[c] = reinterpret_cast<const uint4*>(qweight + nn * (K >> 3));
    srow[c] = scales + nn * ng;
    zrow[c] = qzeros + nn * nzw;
  }

  f32x4_t acc[CT][TM];
#pragma unroll
  for (int c = 0; c < CT; ++c)
#pragma unroll
    for (int t = 0; t < TM; ++t) acc[c][t] = f32x4_t{};

  if (b0 < b1) {
    const int blast = b1 - 1;
    uint4 wq[D][CT];
    uint4 av[D][TM][4];
    uint32_t sv[D][CT], zv[D][CT];
    // block b: the lane's 4 words 4h .. 4h+3 of its column in each column tile;
    // scale and zero word of the block's group; activations of chunks 4h + i,
    // rows col (+ 16 t) of the batch, clamped to M - 1 (shared by the tiles)
    auto load = [&](int b, uint4 (&w)[CT], uint4 (&a)[TM][4], uint32_t (&s)[CT], uint32_t (&z)[CT]) {
      const int g = b >> gsh;
#pragma unroll
      for (int c = 0; c < CT; ++c) {
        w[c] = qrow[c][4 * b + h];
        s[c] = srow[c][g];
        z[c] = zrow[c][g >> 3];
      }
#pragma unroll
      for (int t = 0; t < TM; ++t) {
        const int m = min(16 * t + col, M - 1);
        const uint4* xr = reinterpret_cast<const uint4*>(X + static_cast<size_t>(m) * K + 128 * b);
#pragma unroll
        for (int i = 0; i < 4; ++i) a[t][i] = xr[4 * h + i];
      }
    };
    auto compute = [&](int b, const uint4 (&w)[CT], const uint4 (&a)[TM][4], const uint32_t (&s)[CT],
                       const uint32_t (&zw)[CT]) {
      const int g = b >> gsh;
      h2_t zz[CT], ss[CT];
#pragma unroll
      for (int c = 0; c < CT; ++c) {
        const uint32_t z = (zw[c] >> (4 * (g & 7))) & 15u;
        const _Float16 zb = static_cast<_Float16>(1024.0f + static_cast<float>(z));
        zz[c] = h2_t{zb, zb};
        const _Float16 sh = bitcast<_Float16>(static_cast<uint16_t>(s[c]));
        ss[c] = h2_t{sh, sh};
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        h8_t at[TM];
#pragma unroll
        for (int t = 0; t < TM; ++t) at[t] = bitcast<h8_t>(a[t][i]);
#pragma unroll
        for (int c = 0; c < CT; ++c) {
          const uint32_t word = i == 0 ? w[c].x : i == 1 ? w[c].y : i == 2 ? w[c].z : w[c].w;
          const h8_t bw = dequant_word(word, zz[c], ss[c]);
#pragma unroll
          for (int t = 0; t < TM; ++t) acc[c][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(at[t], bw, acc[c][t], 0, 0, 0);
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
    sk_ring_steps<D>(step, b0, b1);
  }

  // fixed-order sum of the waves' tiles; lane l of a tile holds column
  // l % 16, rows 4 (l / 16) + r; wave c TM + t sums tile (c, t)
#pragma unroll
  for (int c = 0; c < CT; ++c)
#pragma unroll
    for (int t = 0; t < TM; ++t) red[wv][c * TM + t][lane] = acc[c][t];
  __syncthreads();
  if (wv < CT * TM) {
    const int t = wv % TM;
    const int n = n0 + kCols * (wv / TM) + col;
    f32x4_t tot = red[0][wv][lane];
#pragma unroll
    for (int w = 1; w < NWV; ++w) tot += red[w][wv][lane];
    if (n < N) {
      if (rowexp) {
        int ex[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) ex[r] = rowexp[min(16 * t + 4 * h + r, M - 1)];
#pragma unroll
        for (int r = 0; r < 4; ++r) tot[r] = ldexpf(tot[r], ex[r]);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = 16 * t + 4 * h + r;
        if (m < M) store_out<OUTK>(Y, static_cast<size_t>(m) * N + n, tot[r]);
      }
    }
  }
}

template <int NWV, int TM, int D, int CT, int OUTK>
void launch_k(const W4Args& a, hipStream_t stream) {
  static_assert(CT * TM <= NWV, "one summing wave per output tile");
  const int gsh = a.G == 256 ? 1 : 0;
  hipLaunchKernelGGL((w4_skinny_kernel<NWV, TM, D, CT, OUTK>), dim3((a.N + CT * kCols - 1) / (CT * kCols)),
                     dim3(64 * NWV), 0, stream, static_cast<const uint16_t*>(a.X), a.M, a.K, a.qweight, a.scales,
                     a.qzeros, a.N, gsh, a.Y, a.rowexp);
}

template <int NWV, int TM, int D, int CT = 1>
void launch_o(const W4Args& a, hipStream_t stream) {
  if (a.y_dtype == QLIN_F16) launch_k<NWV, TM, D, CT, OUT_F16>(a, stream);
  else if (a.y_dtype == QLIN_BF16) launch_k<NWV, TM, D, CT, OUT_BF16>(a, stream);
  else launch_k<NWV, TM, D, CT, OUT_F32>(a, stream);
}

}  // namespace

bool w4_skinny_supported(int M, int K, int G) { return M >= 1 && M <= 16 && (G == 128 || G == 256) && K % 128 == 0; }

// Wide layers: 4 or 2 column tiles per workgroup (each activation fragment then
// feeds 4 or 2 matrix instructions, so the activations are re-read from cache 4
// or 2 times less) as long as that leaves at least 160 workgroups; one tile
// otherwise (a 4096-column layer keeps its 256 workgroups), with a ring 3 deep,
// or 2 deep on long rows: measured at 8 / 16 rows against the former 4 deep,
// 4096 x 4096 8.3 -> 6.9 / 10.0 -> 8.2 us (3 deep), 4096 x 11008 13.5 -> 13.1 /
// 18.1 -> 17.1 us (2 deep).
void w4_skinny_launch(const W4Args& a, hipStream_t stream) {
  const long long wg4 = (a.N + 4 * kCols - 1) / (4 * kCols), wg2 = (a.N + 2 * kCols - 1) / (2 * kCols);
  if (wg4 >= 160) launch_o<4, 1, 3, 4>(a, stream);
  else if (wg2 >= 160) launch_o<4, 1, 2, 2>(a, stream);
  else if (a.K > 8192) launch_o<4, 1, 2, 1>(a, stream);
  else launch_o<4, 1, 3, 1>(a, stream);
}

}  // namespace qlin
