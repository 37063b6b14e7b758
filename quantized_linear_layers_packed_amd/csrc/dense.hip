// Dense fp16 GEMM, Y = X W^T with fp32 accumulation, gfx950.
//
// The unquantized layer every page measures its format against: the GPTQ
// bulletin ("İddia ve Gerçeklik") and the SmoothQuant bulletin ("Ticari Etki")
// both describe the weight-only gain fading as the batch grows and the layer
// turns compute bound, and the SpQR and SmoothQuant bulletins ("İddia ve
// Gerçeklik") quote their speedups against 16-bit inference.  This kernel is
// that 16-bit layer, built on the same tiling as the int8 GEMM (tile_gemm.hpp):
// X [M][K] and W [N][K] as rows of 2K bytes through v_mfma_f32_32x32x16_f16
// (same operand bytes and output layout as the int8 instruction), fp32
// accumulators, float split-K partials summed in K order, one rounding to the
// output type.

#include "common.hpp"
#include "device.hpp"
#include "launch.hpp"
#include "tile_gemm.hpp"

namespace qlin {

namespace {

struct DenseF16Op {
  using acc_t = f32x16_t;
  using part_t = float;
  static constexpr bool kExact = false;
  __device__ __forceinline__ static acc_t mfma(i32x4_t a, i32x4_t b, acc_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(bitcast<h8_t>(a), bitcast<h8_t>(b), c, 0, 0, 0);
  }
  // one 32 x 32 block's column n, rows mb + 8 (r / 4) + r % 4
  template <int OUTK>
  __device__ __forceinline__ void store(void* Y, int M, int N, int mb, int n, const acc_t& acc) const {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int m = mb + 8 * (r >> 2) + (r & 3);
      if (m < M) store_out<OUTK>(Y, static_cast<size_t>(m) * N + n, acc[r]);
    }
  }
};

template <int WM, int WN, int TM, int TN, int NS, int WPE = WM * WN / 4>
qlin_status launch_o(const uint16_t* X, const uint16_t* W, int M, int N, int K, void* Y, int y_dtype, WsView ws,
                     size_t* need, hipStream_t stream) {
  static const char* fn = "qlin_f16_gemm";
  const DenseF16Op op{};
  const int Kb = 2 * K;
  if (y_dtype == QLIN_F32)
    return tile_gemm_launch<DenseF16Op, WM, WN, TM, TN, 128, NS, OUT_F32, WPE>(fn, X, W, M, N, Kb, op, Y, ws, need,
                                                                          stream);
  if (y_dtype == QLIN_BF16)
    return tile_gemm_launch<DenseF16Op, WM, WN, TM, TN, 128, NS, OUT_BF16, WPE>(fn, X, W, M, N, Kb, op, Y, ws, need,
                                                                           stream);
  return tile_gemm_launch<DenseF16Op, WM, WN, TM, TN, 128, NS, OUT_F16, WPE>(fn, X, W, M, N, Kb, op, Y, ws, need, stream);
}

}  // namespace

qlin_status dense_f16_gemm_launch(const uint16_t* X, const uint16_t* W, int M, int N, int K, void* Y, int y_dtype,
                                  WsView ws, size_t* need, hipStream_t stream) {
  // K steps of 128 bytes (64 values).  Up to 64 rows: a 2 x 4 grid of 32 x 32
  // wave tiles (64 x 128), six stages deep (the layer is bound by the weight
  // stream).  Larger batches: a 4 x 2 grid and the largest tile of 256 x 128,
  // 128 x 128 or 128 x 64 that still gives at least 160 tiles (the smallest one
  // otherwise), as for the int8 GEMM.
  if (M <= 64) return launch_o<2, 4, 1, 1, 6>(X, W, M, N, K, Y, y_dtype, ws, need, stream);
  auto tiles = [&](int bm, int bn) { return static_cast<long long>((M + bm - 1) / bm) * ((N + bn - 1) / bn); };
  if (tiles(256, 128) >= 160) return launch_o<4, 2, 2, 2, 3>(X, W, M, N, K, Y, y_dtype, ws, need, stream);
  if (tiles(128, 128) >= 160) return launch_o<4, 2, 1, 2, 4>(X, W, M, N, K, Y, y_dtype, ws, need, stream);
  return launch_o<4, 2, 1, 1, 6>(X, W, M, N, K, Y, y_dtype, ws, need, stream);
}

}  // namespace qlin
