// C-ABI device entry points: argument validation, kernel selection, launch.
//
// Every check happens on the host before anything is enqueued; device arrays
// are never read here.

#include <string>

#include "common.hpp"
#include "launch.hpp"

using namespace qlin;

namespace {

bool is_out_dtype(int d) { return d == QLIN_F16 || d == QLIN_BF16 || d == QLIN_F32; }

qlin_status need_aligned(const char* fn, const char* name, const void* p) {
  if (!aligned16(p)) return fail(QLIN_EALIGN, std::string(fn) + ": " + name + " is not 16-byte aligned");
  return QLIN_OK;
}

#define QLIN_TRY(expr)                      \
  do {                                      \
    const qlin_status _s = (expr);          \
    if (_s != QLIN_OK) return _s;           \
  } while (0)

// Validation and kernel choice of the W4 forward; with perm != NULL the
// activations are first gathered into Xp (act-order storage).
qlin_status w4_forward_checked(const char* fn, const void* X, int x_dtype, int M, int K,
                               const uint32_t* qweight, const uint16_t* scales, const uint32_t* qzeros, int N, int G,
                               void* Y, int y_dtype, hipStream_t stream, bool gather, const int32_t* perm,
                               void* Xp) {
  if (M <= 0 || N <= 0 || K <= 0 || G <= 0) return fail(QLIN_EINVAL, std::string(fn) + ": M, N, K, G must be positive");
  if (!X || !qweight || !scales || !qzeros || !Y) return fail(QLIN_EINVAL, std::string(fn) + ": NULL pointer");
  if (x_dtype != QLIN_F16 && x_dtype != QLIN_BF16) return fail(QLIN_EINVAL, std::string(fn) + ": x_dtype must be F16 or BF16");
  if (!is_out_dtype(y_dtype)) return fail(QLIN_EINVAL, std::string(fn) + ": y_dtype must be F16, BF16 or F32");
  if (K % G != 0) return fail(QLIN_EINVAL, std::string(fn) + ": K must be a multiple of G");
  if (G % 32 != 0 || G > 256) return fail(QLIN_EUNSUPPORTED, std::string(fn) + ": G must be 32, 64, 128 or 256 (multiple of 32, at most 256)");
  if (G != 32 && G != 64 && G != 128 && G != 256)
    return fail(QLIN_EUNSUPPORTED, std::string(fn) + ": G must be 32, 64, 128 or 256");
  QLIN_TRY(need_aligned(fn, "X", X));
  QLIN_TRY(need_aligned(fn, "qweight", qweight));
  QLIN_TRY(need_aligned(fn, "scales", scales));
  QLIN_TRY(need_aligned(fn, "qzeros", qzeros));
  QLIN_TRY(need_aligned(fn, "Y", Y));
  if (gather) {
    if (!perm || !Xp) return fail(QLIN_EINVAL, std::string(fn) + ": NULL perm or Xp");
    QLIN_TRY(need_aligned(fn, "Xp", Xp));
    const char* x0 = static_cast<const char*>(X);
    const char* p0 = static_cast<const char*>(Xp);
    const size_t bytes = static_cast<size_t>(M) * K * 2;
    if (p0 < x0 + bytes && x0 < p0 + bytes) return fail(QLIN_EINVAL, std::string(fn) + ": Xp overlaps X");
    permute_cols_launch(X, perm, M, K, Xp, stream);
    X = Xp;
  }
  W4Args a{X, x_dtype, M, K, N, G, qweight, scales, qzeros, Y, y_dtype};
  // M = 1 (and M <= 3 while the activations fit its LDS staging): the GEMV;
  // M = 4 .. 16: the small-batch MFMA kernel; larger: the GEMMs.
  if (w4_gemv_supported(M, K, G) && (M <= 3 || !w4_skinny_supported(M, K, G))) {
    w4_gemv_launch(a, stream);
  } else if (w4_skinny_supported(M, K, G)) {
    w4_skinny_launch(a, stream);
  } else if (G >= 128) {
    QLIN_TRY(w4_gemm_sk_launch(a, stream));
  } else {
    w4_gemm_launch(a, stream);
  }
  return check_launch(fn);
}

}  // namespace

extern "C" {

qlin_status qlin_w4_forward(const void* X, int x_dtype, int M, int K,
                            const uint32_t* qweight, const uint16_t* scales,
                            const uint32_t* qzeros, int N, int G,
                            void* Y, int y_dtype, hipStream_t stream) {
  clear_error();
  return w4_forward_checked("qlin_w4_forward", X, x_dtype, M, K, qweight, scales, qzeros, N, G, Y, y_dtype, stream,
                            false, nullptr, nullptr);
}

qlin_status qlin_w4_forward_perm(const void* X, int x_dtype, int M, int K, const int32_t* perm, void* Xp,
                                 const uint32_t* qweight, const uint16_t* scales,
                                 const uint32_t* qzeros, int N, int G,
                                 void* Y, int y_dtype, hipStream_t stream) {
  clear_error();
  return w4_forward_checked("qlin_w4_forward_perm", X, x_dtype, M, K, qweight, scales, qzeros, N, G, Y, y_dtype,
                            stream, true, perm, Xp);
}

qlin_status qlin_w4_unpack(const uint32_t* qweight, const uint32_t* qzeros, int N, int K, int G,
                           uint8_t* codes, uint8_t* zeros, hipStream_t stream) {
  static const char* fn = "qlin_w4_unpack";
  clear_error();
  if (N <= 0 || K <= 0 || G <= 0 || K % G != 0 || K % 8 != 0) return fail(QLIN_EINVAL, std::string(fn) + ": bad N, K or G");
  if (!qweight || !qzeros || !codes || !zeros) return fail(QLIN_EINVAL, std::string(fn) + ": NULL pointer");
  w4_unpack_launch(qweight, qzeros, N, K, G, codes, zeros, stream);
  return check_launch(fn);
}

qlin_status spqr_forward(const uint16_t* X, int M, int K,
                         const uint32_t* codes, const uint32_t* stats1, const uint16_t* stats2,
                         const int32_t* row_ptr, const int32_t* col_idx, const uint16_t* vals,
                         int64_t nnz, int N, void* Y, int y_dtype, hipStream_t stream) {
  static const char* fn = "spqr_forward";
  clear_error();
  if (M <= 0 || N <= 0 || K <= 0) return fail(QLIN_EINVAL, std::string(fn) + ": M, N, K must be positive");
  if (M > 16) return fail(QLIN_EUNSUPPORTED, std::string(fn) + ": M must be at most 16");
  if (K % 256 != 0) return fail(QLIN_EINVAL, std::string(fn) + ": K must be a multiple of 256");
  if (nnz < 0 || nnz > INT32_MAX) return fail(QLIN_EINVAL, std::string(fn) + ": nnz out of range");
  if (!X || !codes || !stats1 || !stats2 || !row_ptr || !Y) return fail(QLIN_EINVAL, std::string(fn) + ": NULL pointer");
  if (nnz > 0 && (!col_idx || !vals)) return fail(QLIN_EINVAL, std::string(fn) + ": NULL CSR arrays with nnz > 0");
  if (y_dtype != QLIN_F16 && y_dtype != QLIN_F32) return fail(QLIN_EINVAL, std::string(fn) + ": y_dtype must be F16 or F32");
  QLIN_TRY(need_aligned(fn, "X", X));
  QLIN_TRY(need_aligned(fn, "codes", codes));
  QLIN_TRY(need_aligned(fn, "stats1", stats1));
  QLIN_TRY(need_aligned(fn, "stats2", stats2));
  QLIN_TRY(need_aligned(fn, "Y", Y));
  SpqrArgs a{X, M, K, N, codes, stats1, stats2, row_ptr, col_idx, vals, Y, y_dtype};
  spqr_gemv_launch(a, stream);
  return check_launch(fn);
}

qlin_status spqr_unpack(const uint32_t* codes, const uint32_t* stats1, int N, int K,
                        uint8_t* q, uint8_t* cs, uint8_t* cz, hipStream_t stream) {
  static const char* fn = "spqr_unpack";
  clear_error();
  if (N <= 0 || K <= 0 || K % 256 != 0) return fail(QLIN_EINVAL, std::string(fn) + ": bad N or K");
  if (!codes || !stats1 || !q || !cs || !cz) return fail(QLIN_EINVAL, std::string(fn) + ": NULL pointer");
  spqr_unpack_launch(codes, stats1, N, K, q, cs, cz, stream);
  return check_launch(fn);
}

qlin_status sq_smooth_quant_act(const uint16_t* X, const float* inv_s, int M, int K,
                                int8_t* Xq, float* x_scale, hipStream_t stream) {
  static const char* fn = "sq_smooth_quant_act";
  clear_error();
  if (M <= 0 || K <= 0) return fail(QLIN_EINVAL, std::string(fn) + ": M and K must be positive");
  if (K % 8 != 0) return fail(QLIN_EINVAL, std::string(fn) + ": K must be a multiple of 8");
  if (!X || !inv_s || !Xq || !x_scale) return fail(QLIN_EINVAL, std::string(fn) + ": NULL pointer");
  QLIN_TRY(need_aligned(fn, "X", X));
  QLIN_TRY(need_aligned(fn, "inv_s", inv_s));
  QLIN_TRY(need_aligned(fn, "Xq", Xq));
  sq_act_launch(X, inv_s, M, K, Xq, x_scale, stream);
  return check_launch(fn);
}

qlin_status sq_int8_gemm(const int8_t* Xq, const float* x_scale, const int8_t* Wq, const float* w_scale,
                         int M, int N, int K, void* Y, int y_dtype, int32_t* acc_out, hipStream_t stream) {
  static const char* fn = "sq_int8_gemm";
  clear_error();
  if (M <= 0 || N <= 0 || K <= 0) return fail(QLIN_EINVAL, std::string(fn) + ": M, N, K must be positive");
  if (K % 64 != 0) return fail(QLIN_EINVAL, std::string(fn) + ": K must be a multiple of 64");
  if (K > 131072) return fail(QLIN_EUNSUPPORTED, std::string(fn) + ": K above 131072 could overflow int32");
  if (!Xq || !x_scale || !Wq || !w_scale || !Y) return fail(QLIN_EINVAL, std::string(fn) + ": NULL pointer");
  if (y_dtype != QLIN_F16 && y_dtype != QLIN_F32) return fail(QLIN_EINVAL, std::string(fn) + ": y_dtype must be F16 or F32");
  QLIN_TRY(need_aligned(fn, "Xq", Xq));
  QLIN_TRY(need_aligned(fn, "Wq", Wq));
  QLIN_TRY(need_aligned(fn, "Y", Y));
  if (acc_out) QLIN_TRY(need_aligned(fn, "acc_out", acc_out));
  QLIN_TRY(sq_gemm_launch(Xq, x_scale, Wq, w_scale, M, N, K, Y, y_dtype, acc_out, stream));
  return check_launch(fn);
}

}  // extern "C"
