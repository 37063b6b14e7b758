// Internal launcher interfaces between the C-ABI layer and the kernels.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

#include "../../include/qlin.h"
#include "workspace.hpp"

namespace qlin {

struct W4Args {
  const void* X;
  int x_dtype;
  int M, K, N, G;
  const uint32_t* qweight;
  const uint16_t* scales;
  const uint32_t* qzeros;
  void* Y;
  int y_dtype;
  const int* rowexp;   // non-NULL: X is a row-scaled fp16 copy of bf16 input, row m scaled by 2^-rowexp[m]
};

// Fused GEMV for M <= 16 (activations staged in LDS).
size_t w4_gemv_lds_bytes(int M, int K);
bool w4_gemv_supported(int M, int K, int G);
void w4_gemv_launch(const W4Args& a, hipStream_t stream);
// MFMA GEMM for larger batches, groups of 128 / 256: stream-K over the
// caller's workspace.  With need != NULL only the partial-tile bytes it needs
// are reported (nothing is launched).
qlin_status w4_gemm_sk_launch(const W4Args& a, WsView ws, size_t* need, hipStream_t stream);
// The same product on an LDS ring fed by direct loads (same workspace
// contract), for the shapes w4_tile_supported accepts.
bool w4_tile_supported(const W4Args& a);
qlin_status w4_tile_launch(const W4Args& a, WsView ws, size_t* need, hipStream_t stream);
// Groups of 32 / 64: one K step per group, exact codes and an fp32 rescale.
void w4_gemm_group_launch(const W4Args& a, hipStream_t stream);
// bf16 X [M][K] -> fp16 Xh = X * 2^-e_m per row (round to nearest even) and
// e_m (int32 [M]) with the row maximum scaled into [2^14, 2^15).
void x_rowscale_launch(const uint16_t* X, int M, int K, uint16_t* Xh, int* rowexp, hipStream_t stream);
// Small batches (M <= 16, G = 128 / 256): 16 columns per workgroup, K split
// over its waves, fp16 MFMA, no workspace.
bool w4_skinny_supported(int M, int K, int G);
void w4_skinny_launch(const W4Args& a, hipStream_t stream);
// Xp[m][t] = X[m][perm[t]] for 16-bit activations (act-order storage).
void permute_cols_launch(const void* X, const int32_t* perm, int M, int K, void* Xp, hipStream_t stream);
void w4_unpack_launch(const uint32_t* qweight, const uint32_t* qzeros, int N, int K, int G,
                      uint8_t* codes, uint8_t* zeros, hipStream_t stream);

// The library's fixed device scratch (see scratch.hip): its size, its address on
// the current device (looked up once per device), and a fill kernel that zeroes
// its arrival counters on `stream`.
size_t scratch_bytes();
qlin_status scratch_base(char** out);
void scratch_clear_counters(char* base, hipStream_t stream);

struct SpqrArgs {
  const uint16_t* X;
  int M, K, N;
  const uint32_t* codes;
  const uint32_t* stats1;
  const uint16_t* stats2;
  const int32_t* row_ptr;
  const int32_t* col_idx;
  const uint16_t* vals;
  void* Y;
  int y_dtype;
};

// one token (M == 1); rows of any length (the router sends it those up to 8192)
void spqr_gemv_launch(const SpqrArgs& a, hipStream_t stream);
// 1 .. 8 tokens: four rows per wave on the 4 x 4 x 4 matrix instruction (no
// workspace); the forward's routing is spqr_use_quad.
void spqr_quad_launch(const SpqrArgs& a, hipStream_t stream);

// Matrix-core path for small batches: activations laid out by a prepass in the
// workspace (Xp: MFMA operand order, Xs: group sums, XT: transposed copy).
struct SpqrPrep {
  const uint4* Xp;
  const float* Xs;
  const uint16_t* XT;
};
// Routing of the SpQR forward by batch: one token runs the GEMV (spqr_gemv),
// 2 .. 6 the four-rows-per-wave kernel on the 4 x 4 x 4 matrix instruction
// (spqr_quad), 7 and 8 that kernel on layers wider than deep (N > K) and the
// matrix-core path (16 tokens per 16 x 16 x 16 instruction, spqr_mfma)
// otherwise, 9 .. 16 the matrix-core path.  33B-shaped layers (us), quad vs
// matrix-core: M = 7: 6656 x 6656 24.5 vs 22.3, 17920 x 6656 52.5 vs 57.4,
// 6656 x 17920 56.0 vs 56.0; M = 8: 25.5 vs 22.3, 56.2 vs 57.3, 58.3 vs 56.0
// (the matrix-core time hardly moves with M); at M = 6 the quad kernel is
// level or ahead on all three.
inline bool spqr_use_mfma(int M, int K, int N) { return M >= 9 || (M >= 7 && N <= K); }
// Single tokens on rows longer than 8192 also go to the four-row kernel: there
// the GEMV splits a row over several waves whose 64-chunk blocks leave a
// quarter of its lanes idle (6656 x 17920: 30.5 against 33.1 us).
inline bool spqr_use_quad(int M, int K, int N) {
  return (M >= 2 && M <= 6) || (M == 1 && K > 8192) || (M >= 7 && M <= 8 && N > K);
}
size_t spqr_prep_bytes(int K);
SpqrPrep spqr_prep_view(char* base, int K);
void spqr_mfma_launch(const SpqrArgs& a, const SpqrPrep& p, hipStream_t stream);
void spqr_unpack_launch(const uint32_t* codes, const uint32_t* stats1, int N, int K,
                        uint8_t* q, uint8_t* cs, uint8_t* cz, hipStream_t stream);

void sq_act_launch(const uint16_t* X, const float* inv_s, int M, int K, int8_t* Xq, float* x_scale,
                   hipStream_t stream);
// With need != NULL only the workspace bytes beyond the counters are reported
// (0 if the kernel chosen needs none); nothing is launched.
qlin_status sq_gemm_launch(const int8_t* Xq, const float* x_scale, const int8_t* Wq, const float* w_scale,
                           int M, int N, int K, void* Y, int y_dtype, int32_t* acc_out, WsView ws, size_t* need,
                           hipStream_t stream);

// Dense fp16 GEMM Y = X W^T (K % 64 == 0); need / workspace as for sq_gemm_launch.
qlin_status dense_f16_gemm_launch(const uint16_t* X, const uint16_t* W, int M, int N, int K, void* Y, int y_dtype,
                                  WsView ws, size_t* need, hipStream_t stream);

}  // namespace qlin
