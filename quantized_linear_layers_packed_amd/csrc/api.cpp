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

qlin_status need_workspace(const char* fn, const void* ws, size_t ws_bytes, size_t total) {
  if (total == 0) return QLIN_OK;
  if (!ws || ws_bytes < total)
    return fail(QLIN_EINVAL, std::string(fn) + ": this shape needs a workspace of " + std::to_string(total) +
                                 " bytes (ask the matching *_workspace_bytes call); got " +
                                 (ws ? std::to_string(ws_bytes) + " bytes" : std::string("NULL")));
  return need_aligned(fn, "workspace", ws);
}

// The W4 GEMM past the small-batch kernel: the direct-load tile kernel where
// it measured faster, the register-ring stream-K kernel elsewhere.
qlin_status w4_big_launch(const W4Args& a, WsView ws, size_t* need, hipStream_t stream) {
  return w4_tile_supported(a) ? w4_tile_launch(a, ws, need, stream) : w4_gemm_sk_launch(a, ws, need, stream);
}

// Kernel choice of the W4 forward and the workspace it needs.
enum class W4Path { kGemv, kSkinny, kSplitK, kGroup };

struct W4Plan {
  W4Path path = W4Path::kGemv;
  bool prep = false;           // bf16 X converted to a row-scaled fp16 copy first
  size_t prep_off = 0;         // offset of that copy in the workspace
  size_t total = 0;            // workspace bytes (0: none)
};

qlin_status w4_plan(const W4Args& a, W4Plan* p) {
  // M = 1 (and M <= 3 while the activations fit its LDS staging): the GEMV;
  // M = 4 .. 16: the small-batch MFMA kernel; larger: the GEMMs.
  if (w4_gemv_supported(a.M, a.K, a.G) && (a.M <= 3 || !w4_skinny_supported(a.M, a.K, a.G))) p->path = W4Path::kGemv;
  else if (w4_skinny_supported(a.M, a.K, a.G)) p->path = W4Path::kSkinny;
  else if (a.G >= 128) p->path = W4Path::kSplitK;
  else p->path = W4Path::kGroup;
  p->prep = a.x_dtype == QLIN_BF16 && p->path != W4Path::kGemv;
  size_t partial = 0;
  if (p->path == W4Path::kSplitK) QLIN_TRY(w4_big_launch(a, WsView{}, &partial, nullptr));
  if (p->path != W4Path::kSplitK && !p->prep) {
    p->total = 0;
    return QLIN_OK;
  }
  p->prep_off = kCounterBytes + ws_round(partial);
  p->total = p->prep_off;
  if (p->prep) p->total += ws_round(static_cast<size_t>(a.M) * a.K * 2) + ws_round(static_cast<size_t>(a.M) * 4);
  return QLIN_OK;
}

qlin_status w4_check_shape(const char* fn, int x_dtype, int M, int K, int N, int G, int y_dtype) {
  if (M <= 0 || N <= 0 || K <= 0 || G <= 0) return fail(QLIN_EINVAL, std::string(fn) + ": M, N, K, G must be positive");
  if (x_dtype != QLIN_F16 && x_dtype != QLIN_BF16) return fail(QLIN_EINVAL, std::string(fn) + ": x_dtype must be F16 or BF16");
  if (!is_out_dtype(y_dtype)) return fail(QLIN_EINVAL, std::string(fn) + ": y_dtype must be F16, BF16 or F32");
  if (K % G != 0) return fail(QLIN_EINVAL, std::string(fn) + ": K must be a multiple of G");
  if (G != 32 && G != 64 && G != 128 && G != 256)
    return fail(QLIN_EUNSUPPORTED, std::string(fn) + ": G must be 32, 64, 128 or 256");
  return QLIN_OK;
}

// Validation and kernel choice of the W4 forward; with gather the activations
// are first gathered through perm into Xp (act-order storage).
qlin_status w4_forward_checked(const char* fn, const void* X, int x_dtype, int M, int K,
                               const uint32_t* qweight, const uint16_t* scales, const uint32_t* qzeros, int N, int G,
                               void* Y, int y_dtype, void* workspace, size_t workspace_bytes, hipStream_t stream,
                               bool gather, const int32_t* perm, void* Xp, bool clear_counters = false) {
  QLIN_TRY(w4_check_shape(fn, x_dtype, M, K, N, G, y_dtype));
  if (!X || !qweight || !scales || !qzeros || !Y) return fail(QLIN_EINVAL, std::string(fn) + ": NULL pointer");
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
  }
  W4Args a{X, x_dtype, M, K, N, G, qweight, scales, qzeros, Y, y_dtype, nullptr};
  W4Plan plan;
  QLIN_TRY(w4_plan(a, &plan));
  QLIN_TRY(need_workspace(fn, workspace, workspace_bytes, plan.total));
  const WsView ws{static_cast<char*>(workspace), workspace_bytes};
  // nothing is enqueued before this point
  if (clear_counters && plan.path == W4Path::kSplitK) scratch_clear_counters(ws.base, stream);
  if (gather) {
    permute_cols_launch(X, perm, M, K, Xp, stream);
    a.X = Xp;
  }
  if (plan.prep) {
    uint16_t* xh = reinterpret_cast<uint16_t*>(ws.base + plan.prep_off);
    int* rowexp = reinterpret_cast<int*>(ws.base + plan.prep_off + ws_round(static_cast<size_t>(M) * K * 2));
    x_rowscale_launch(static_cast<const uint16_t*>(a.X), M, K, xh, rowexp, stream);
    a.X = xh;
    a.x_dtype = QLIN_F16;
    a.rowexp = rowexp;
  }
  switch (plan.path) {
    case W4Path::kGemv: w4_gemv_launch(a, stream); break;
    case W4Path::kSkinny: w4_skinny_launch(a, stream); break;
    case W4Path::kSplitK: QLIN_TRY(w4_big_launch(a, ws, nullptr, stream)); break;
    case W4Path::kGroup: w4_gemm_group_launch(a, stream); break;
  }
  return check_launch(fn);
}

qlin_status sq_check(const char* fn, int M, int N, int K, int y_dtype) {
  if (M <= 0 || N <= 0 || K <= 0) return fail(QLIN_EINVAL, std::string(fn) + ": M, N, K must be positive");
  if (K % 64 != 0) return fail(QLIN_EINVAL, std::string(fn) + ": K must be a multiple of 64");
  if (K > 131072) return fail(QLIN_EUNSUPPORTED, std::string(fn) + ": K above 131072 could overflow int32");
  if (y_dtype != QLIN_F16 && y_dtype != QLIN_F32) return fail(QLIN_EINVAL, std::string(fn) + ": y_dtype must be F16 or F32");
  return QLIN_OK;
}

qlin_status sq_workspace_total(int M, int N, int K, int y_dtype, size_t* total) {
  size_t partial = 0;
  QLIN_TRY(sq_gemm_launch(nullptr, nullptr, nullptr, nullptr, M, N, K, nullptr, y_dtype, nullptr, WsView{}, &partial,
                          nullptr));
  // a kernel with a K split needs the counters even when its plan splits no tile
  *total = partial ? kCounterBytes + ws_round(partial) : 0;
  return QLIN_OK;
}

qlin_status dense_check(const char* fn, int M, int N, int K, int y_dtype) {
  if (M <= 0 || N <= 0 || K <= 0) return fail(QLIN_EINVAL, std::string(fn) + ": M, N, K must be positive");
  if (K % 64 != 0) return fail(QLIN_EINVAL, std::string(fn) + ": K must be a multiple of 64");
  if (K > (1 << 29)) return fail(QLIN_EUNSUPPORTED, std::string(fn) + ": K above 2^29");
  if (!is_out_dtype(y_dtype)) return fail(QLIN_EINVAL, std::string(fn) + ": bad y_dtype");
  return QLIN_OK;
}

qlin_status dense_workspace_total(int M, int N, int K, int y_dtype, size_t* total) {
  size_t partial = 0;
  QLIN_TRY(dense_f16_gemm_launch(nullptr, nullptr, M, N, K, nullptr, y_dtype, WsView{}, &partial, nullptr));
  *total = kCounterBytes + ws_round(partial);
  return QLIN_OK;
}

}  // namespace

extern "C" {

qlin_status qlin_w4_workspace_bytes(int x_dtype, int M, int K, int N, int G, int y_dtype, size_t* bytes) {
  static const char* fn = "qlin_w4_workspace_bytes";
  clear_error();
  if (!bytes) return fail(QLIN_EINVAL, std::string(fn) + ": NULL bytes");
  QLIN_TRY(w4_check_shape(fn, x_dtype, M, K, N, G, y_dtype));
  W4Args a{nullptr, x_dtype, M, K, N, G, nullptr, nullptr, nullptr, nullptr, y_dtype, nullptr};
  W4Plan plan;
  QLIN_TRY(w4_plan(a, &plan));
  *bytes = plan.total;
  return QLIN_OK;
}

qlin_status qlin_w4_forward(const void* X, int x_dtype, int M, int K,
                            const uint32_t* qweight, const uint16_t* scales,
                            const uint32_t* qzeros, int N, int G,
                            void* Y, int y_dtype, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  clear_error();
  return w4_forward_checked("qlin_w4_forward", X, x_dtype, M, K, qweight, scales, qzeros, N, G, Y, y_dtype,
                            workspace, workspace_bytes, stream, false, nullptr, nullptr);
}

qlin_status qlin_w4_forward_perm(const void* X, int x_dtype, int M, int K, const int32_t* perm, void* Xp,
                                 const uint32_t* qweight, const uint16_t* scales,
                                 const uint32_t* qzeros, int N, int G,
                                 void* Y, int y_dtype, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  clear_error();
  return w4_forward_checked("qlin_w4_forward_perm", X, x_dtype, M, K, qweight, scales, qzeros, N, G, Y, y_dtype,
                            workspace, workspace_bytes, stream, true, perm, Xp);
}

qlin_status qlin_w4_forward_scratch(const void* X, int x_dtype, int M, int K,
                                    const uint32_t* qweight, const uint16_t* scales,
                                    const uint32_t* qzeros, int N, int G,
                                    void* Y, int y_dtype, hipStream_t stream) {
  static const char* fn = "qlin_w4_forward_scratch";
  clear_error();
  QLIN_TRY(w4_check_shape(fn, x_dtype, M, K, N, G, y_dtype));
  W4Args a{X, x_dtype, M, K, N, G, qweight, scales, qzeros, Y, y_dtype, nullptr};
  W4Plan plan;
  QLIN_TRY(w4_plan(a, &plan));
  if (plan.total > scratch_bytes())
    return fail(QLIN_EUNSUPPORTED, std::string(fn) + ": this shape needs " + std::to_string(plan.total) +
                                       " bytes of scratch, the library's fixed scratch holds " +
                                       std::to_string(scratch_bytes()) + "; use qlin_w4_forward with a workspace");
  char* base = nullptr;
  if (plan.total > 0) QLIN_TRY(scratch_base(&base));
  // split-K shapes clear the shared counters first (after every argument check):
  // the previous call on this device left them zero unless calls overlapped
  return w4_forward_checked(fn, X, x_dtype, M, K, qweight, scales, qzeros, N, G, Y, y_dtype, base,
                            base ? scratch_bytes() : 0, stream, false, nullptr, nullptr, true);
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

qlin_status spqr_workspace_bytes(int M, int K, int N, int y_dtype, size_t* bytes) {
  static const char* fn = "spqr_workspace_bytes";
  clear_error();
  if (!bytes) return fail(QLIN_EINVAL, std::string(fn) + ": NULL bytes");
  if (M <= 0 || N <= 0 || K <= 0) return fail(QLIN_EINVAL, std::string(fn) + ": M, N, K must be positive");
  if (M > 16) return fail(QLIN_EUNSUPPORTED, std::string(fn) + ": M must be at most 16");
  if (K % 256 != 0) return fail(QLIN_EINVAL, std::string(fn) + ": K must be a multiple of 256");
  if (y_dtype != QLIN_F16 && y_dtype != QLIN_F32) return fail(QLIN_EINVAL, std::string(fn) + ": y_dtype must be F16 or F32");
  *bytes = spqr_use_mfma(M, K, N) ? kCounterBytes + spqr_prep_bytes(K) : 0;
  return QLIN_OK;
}

qlin_status spqr_forward(const uint16_t* X, int M, int K,
                         const uint32_t* codes, const uint32_t* stats1, const uint16_t* stats2,
                         const int32_t* row_ptr, const int32_t* col_idx, const uint16_t* vals,
                         int64_t nnz, int N, void* Y, int y_dtype, void* workspace, size_t workspace_bytes,
                         hipStream_t stream) {
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
  // the prepass area starts after the counter slots, which stay untouched, so
  // one workspace can serve this call and the split-K calls in any order
  const size_t total = spqr_use_mfma(M, K, N) ? kCounterBytes + spqr_prep_bytes(K) : 0;
  QLIN_TRY(need_workspace(fn, workspace, workspace_bytes, total));
  // with no outliers the CSR arrays may be NULL; the kernels that read CSR
  // entries unconditionally (flagging those past a row) then read row_ptr
  if (nnz == 0) {
    col_idx = row_ptr;
    vals = reinterpret_cast<const uint16_t*>(row_ptr);
  }
  SpqrArgs a{X, M, K, N, codes, stats1, stats2, row_ptr, col_idx, vals, Y, y_dtype};
  if (total) spqr_mfma_launch(a, spqr_prep_view(static_cast<char*>(workspace) + kCounterBytes, K), stream);
  else if (spqr_use_quad(M, K, N)) spqr_quad_launch(a, stream);
  else if (M == 1) spqr_gemv_launch(a, stream);
  else return fail(QLIN_EUNSUPPORTED, std::string(fn) + ": no kernel for this batch size");
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

qlin_status sq_int8_gemm_workspace_bytes(int M, int N, int K, int y_dtype, size_t* bytes) {
  static const char* fn = "sq_int8_gemm_workspace_bytes";
  clear_error();
  if (!bytes) return fail(QLIN_EINVAL, std::string(fn) + ": NULL bytes");
  QLIN_TRY(sq_check(fn, M, N, K, y_dtype));
  return sq_workspace_total(M, N, K, y_dtype, bytes);
}

qlin_status sq_int8_gemm(const int8_t* Xq, const float* x_scale, const int8_t* Wq, const float* w_scale,
                         int M, int N, int K, void* Y, int y_dtype, int32_t* acc_out, void* workspace,
                         size_t workspace_bytes, hipStream_t stream) {
  static const char* fn = "sq_int8_gemm";
  clear_error();
  QLIN_TRY(sq_check(fn, M, N, K, y_dtype));
  if (!Xq || !x_scale || !Wq || !w_scale || !Y) return fail(QLIN_EINVAL, std::string(fn) + ": NULL pointer");
  QLIN_TRY(need_aligned(fn, "Xq", Xq));
  QLIN_TRY(need_aligned(fn, "Wq", Wq));
  QLIN_TRY(need_aligned(fn, "Y", Y));
  if (acc_out) QLIN_TRY(need_aligned(fn, "acc_out", acc_out));
  size_t total = 0;
  QLIN_TRY(sq_workspace_total(M, N, K, y_dtype, &total));
  QLIN_TRY(need_workspace(fn, workspace, workspace_bytes, total));
  QLIN_TRY(sq_gemm_launch(Xq, x_scale, Wq, w_scale, M, N, K, Y, y_dtype, acc_out,
                          WsView{static_cast<char*>(workspace), workspace_bytes}, nullptr, stream));
  return check_launch(fn);
}

qlin_status qlin_f16_gemm_workspace_bytes(int M, int N, int K, int y_dtype, size_t* bytes) {
  static const char* fn = "qlin_f16_gemm_workspace_bytes";
  clear_error();
  if (!bytes) return fail(QLIN_EINVAL, std::string(fn) + ": NULL bytes");
  QLIN_TRY(dense_check(fn, M, N, K, y_dtype));
  return dense_workspace_total(M, N, K, y_dtype, bytes);
}

qlin_status qlin_f16_gemm(const uint16_t* X, const uint16_t* W, int M, int N, int K, void* Y, int y_dtype,
                          void* workspace, size_t workspace_bytes, hipStream_t stream) {
  static const char* fn = "qlin_f16_gemm";
  clear_error();
  QLIN_TRY(dense_check(fn, M, N, K, y_dtype));
  if (!X || !W || !Y) return fail(QLIN_EINVAL, std::string(fn) + ": NULL pointer");
  QLIN_TRY(need_aligned(fn, "X", X));
  QLIN_TRY(need_aligned(fn, "W", W));
  QLIN_TRY(need_aligned(fn, "Y", Y));
  size_t total = 0;
  QLIN_TRY(dense_workspace_total(M, N, K, y_dtype, &total));
  QLIN_TRY(need_workspace(fn, workspace, workspace_bytes, total));
  QLIN_TRY(dense_f16_gemm_launch(X, W, M, N, K, Y, y_dtype, WsView{static_cast<char*>(workspace), workspace_bytes},
                                 nullptr, stream));
  return check_launch(fn);
}

}  // extern "C"
