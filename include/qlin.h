/*
 * qlin.h — C ABI of the packed quantized linear layer library for MI355X (gfx950).
 *
 * One operation, three weight encodings:  Y[M][N] = X[M][K] . W_hat[N][K]^T
 * (rows of W_hat are output channels, "out x in").
 *
 *   W4     4-bit weights in groups of G along K with an fp16 scale and a 4-bit
 *          zero per group (GPTQ-style storage).  Source: GPTQ bulletin
 *          ("Makale Bülteni — GPTQ"), lead and "İddia ve Gerçeklik": 4-bit
 *          weights quantized in blocks such as groups of 128; weight-only, the
 *          activations stay 16-bit.
 *   SpQR   a dense 3-bit matrix (groups of 16, bi-level statistics) plus a CSR
 *          fp16 outlier matrix holding about 1% of the weights, both applied in
 *          one pass.  Source: SpQR bulletin ("Makale Bülteni — SpQR"),
 *          "İddia ve Gerçeklik".
 *   W8A8   SmoothQuant: Y = (X diag(s)^-1)(diag(s) W) with s folded into the
 *          weights offline, per-token int8 activations, per-channel int8
 *          weights, int32 accumulation.  Source: SmoothQuant bulletin
 *          ("Makale Bülteni — SmoothQuant"), "İddia ve Gerçeklik" and its
 *          equation.
 *
 * Conventions for every call:
 *   - The caller owns every buffer, the device workspace of the W4 and int8
 *     GEMMs included.  Nothing here allocates or frees device memory or
 *     synchronizes the device.
 *   - *_forward / sq_* device calls take DEVICE pointers and a HIP stream and are
 *     asynchronous: they validate arguments on the host, enqueue kernels on
 *     `stream` and return.  A device-side fault surfaces at the caller's next
 *     synchronization.  Device pointers must be 16-byte aligned.
 *   - *_pack / *_sizes / sq_act_absmax / sq_compute_smoothing / sq_pack_weight
 *     are synchronous host code on HOST pointers; they never touch the GPU and
 *     are deterministic (bit-identical output for identical input).
 *   - All arrays are row-major and contiguous.  fp16 and bf16 values travel as
 *     uint16_t bit patterns.
 *   - Errors: every call returns a qlin_status.  Invalid arguments are reported
 *     before anything is enqueued; qlin_last_error() then returns a
 *     thread-local message naming the argument.
 *   - Calls on distinct streams may run concurrently as long as they do not
 *     share a workspace.  The library keeps no state besides the thread-local
 *     error message and a per-device cache of the compute-unit count.
 *   - Workspace (qlin_w4_forward, qlin_w4_forward_perm, spqr_forward,
 *     sq_int8_gemm, qlin_f16_gemm): device
 *     memory of at least the size the matching *_workspace_bytes call reports
 *     for the shape (0 means none is needed and NULL may be passed), 16-byte
 *     aligned.  Fill the whole buffer with zeros once after allocating it:
 *     the split-K kernels keep arrival counters in its first 16 KiB, which
 *     must be zero when a call starts; every call leaves them zero again when
 *     it completes, and calls that need no counters keep their data after
 *     them, so one workspace, sized for the largest shape, can serve any
 *     sequence of calls, entry points and shapes on one stream.  Calls sharing a workspace
 *     must not overlap in time.  Everything else in it is scratch.  A too small
 *     or NULL workspace where one is needed gives EINVAL, with the needed size
 *     in qlin_last_error().
 */
#ifndef QLIN_H
#define QLIN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t* hipStream_t;

typedef enum {
  QLIN_OK = 0,
  QLIN_EINVAL = 1,        /* bad size, NULL pointer, inconsistent arguments     */
  QLIN_EALIGN = 2,        /* a device pointer is not 16-byte aligned            */
  QLIN_EUNSUPPORTED = 3,  /* valid but not implemented (e.g. a group size)      */
  QLIN_EHIP = 4           /* the HIP runtime reported an error at launch        */
} qlin_status;

typedef enum { QLIN_F16 = 1, QLIN_BF16 = 2, QLIN_F32 = 3 } qlin_dtype;

/* Library version (major*10000 + minor*100 + patch). */
int qlin_version(void);
/* Static name of a status code. */
const char* qlin_status_str(int status);
/* Thread-local description of the last failure in this thread ("" if none). */
const char* qlin_last_error(void);

/* ======================================================================== */
/* W4: 4-bit group quantization                                              */
/* ======================================================================== */
/* Storage for an N x K weight, group size G (G divides K, G % 8 == 0):
 *   qweight uint32 [N][K/8]          code of k in bits 4*(k%8) of word k/8
 *   scales  fp16   [N][K/G]          per-group scale S
 *   qzeros  uint32 [N][ceil(K/G/8)]  zero z of group g in bits 4*(g%8) of word g/8
 * Dequantized weight: w_hat = S * (q - z).                                    */

/* Byte sizes of the three arrays.  EINVAL if N, K, G <= 0 or G does not divide K
 * or G % 8 != 0. */
qlin_status qlin_w4_sizes(int N, int K, int G,
                          size_t* qweight_bytes, size_t* scales_bytes, size_t* qzeros_bytes);

/* Round-to-nearest encode of fp32 W [N][K] (host) into the three host arrays.
 * Per (row, group): lo = min(0, min w), hi = max(0, max w),
 * S = fp16((hi - lo) / 15) (S = 1 if that is 0), z = clamp(rint(-lo / S), 0, 15),
 * q = clamp(rint(w / S) + z, 0, 15); fp32 arithmetic, round half to even.
 * This is the round-to-nearest baseline named by the GPTQ bulletin
 * ("İddia ve Gerçeklik"); a second-order encoder would fill the same storage. */
qlin_status qlin_w4_pack(const float* W, int N, int K, int G,
                         uint32_t* qweight, uint16_t* scales, uint32_t* qzeros);

/* Device workspace bytes qlin_w4_forward / qlin_w4_forward_perm need for this
 * shape and these dtypes on the current device (0: none).  Errors as the
 * forward's shape checks (EINVAL / EUNSUPPORTED), EINVAL for a NULL bytes. */
qlin_status qlin_w4_workspace_bytes(int x_dtype, int M, int K, int N, int G, int y_dtype, size_t* bytes);

/* Y = X . W_hat^T on the GPU.
 *   X  device, [M][K], x_dtype QLIN_F16 or QLIN_BF16
 *   Y  device, [M][N], y_dtype QLIN_F16, QLIN_BF16 or QLIN_F32
 *   workspace / workspace_bytes: see the conventions at the top
 * Accumulation is fp32.  Kernel by batch size:
 *   - M <= 3 (up to 16 for G = 32 / 64), K <= 16384, staged activations within
 *     64 KB of LDS: a fused unpack-dequant GEMV on exact codes, fp16 or bf16
 *     activations as given;
 *   - 4 <= M <= 16, G = 128 / 256: a small-batch fp16 MFMA kernel (16 columns
 *     per workgroup, K split over its waves) on weights S * (q - z) rounded
 *     once to fp16;
 *   - larger M, G = 128 / 256: an fp16 MFMA GEMM split over the device's
 *     compute units (stream-K, workspace); up to 64 rows per tile it takes the
 *     exact codes q - z and applies S per 128-wide K step in fp32, 128-row
 *     tiles take the same fp16 weights as the small-batch kernel;
 *   - larger M, G = 32 / 64: an fp16 MFMA GEMM on exact codes q - z with a
 *     per-group fp32 rescale.
 * The MFMA paths take fp16 activations.  bf16 X on those paths is first
 * converted (one extra kernel, workspace) into an fp16 copy in which each row
 * m is scaled by 2^-e_m so that its largest magnitude lies in [2^14, 2^15);
 * the outputs of row m are multiplied back by 2^e_m (exact).  Values down to
 * 2^-31 of their row's maximum keep every bit; smaller ones are rounded to the
 * fp16 subnormal step (an error of at most 2^-39 of the row maximum).
 * Requirements: M, N, K > 0; G in {32, 64, 128, 256} (EUNSUPPORTED for other
 * G); K % G == 0. */
qlin_status qlin_w4_forward(const void* X, int x_dtype, int M, int K,
                            const uint32_t* qweight, const uint16_t* scales,
                            const uint32_t* qzeros, int N, int G,
                            void* Y, int y_dtype, void* workspace, size_t workspace_bytes,
                            hipStream_t stream);

/* qlin_w4_forward for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc): no
 * workspace argument; the workspace comes from a fixed device array of the
 * library (80 MiB, zero at load, held on every device the library runs on
 * until the process ends; its address is looked up on the first call on each
 * device).  Allocates nothing.  Split-K shapes first clear the array's arrival
 * counters with a small kernel on `stream`.  Every call on one device shares the
 * array, so calls that overlap in time on one device (concurrent streams,
 * threads) race and give wrong results; serialize them.  A shape whose
 * workspace (qlin_w4_workspace_bytes) exceeds 80 MiB returns EUNSUPPORTED and
 * enqueues nothing.  Other arguments, requirements, results and errors as
 * qlin_w4_forward; results are bit-identical to it. */
qlin_status qlin_w4_forward_scratch(const void* X, int x_dtype, int M, int K,
                                    const uint32_t* qweight, const uint16_t* scales,
                                    const uint32_t* qzeros, int N, int G,
                                    void* Y, int y_dtype, hipStream_t stream);

/* Forward of act-order storage (qlin_w4_pack_gptq_actorder without static
 * groups): the stored columns are in quantization order and stored column t is
 * input column perm[t], so Y = X[:, perm] . W_hat^T.  The GPTQ bulletin
 * ("Kod ve Entegrasyon Haritası") notes that act-order makes the groups
 * irregular at run time; here a gather
 * Xp[m][t] = X[m][perm[t]] runs first (one extra small kernel on `stream`), then
 * qlin_w4_forward's kernels on Xp.
 *   perm device int32 [K], a permutation of 0 .. K-1 (entries are clamped into
 *        range, so a non-permutation gives a meaningless result, never a fault)
 *   Xp   device scratch [M][K] of x_dtype, overwritten, 16-byte aligned, must
 *        not overlap X
 * Other arguments (the workspace as sized by qlin_w4_workspace_bytes),
 * requirements and errors as qlin_w4_forward (EINVAL for a NULL perm or Xp,
 * or Xp overlapping X). */
qlin_status qlin_w4_forward_perm(const void* X, int x_dtype, int M, int K, const int32_t* perm, void* Xp,
                                 const uint32_t* qweight, const uint16_t* scales,
                                 const uint32_t* qzeros, int N, int G,
                                 void* Y, int y_dtype, void* workspace, size_t workspace_bytes,
                                 hipStream_t stream);

/* Debug: unpack codes (uint8 [N][K]) and zeros (uint8 [N][K/G]) on the GPU with
 * the same unpack routine the forward kernels use. */
qlin_status qlin_w4_unpack(const uint32_t* qweight, const uint32_t* qzeros,
                           int N, int K, int G, uint8_t* codes, uint8_t* zeros,
                           hipStream_t stream);

/* ======================================================================== */
/* SpQR: 3-bit groups of 16 with bi-level statistics + CSR fp16 outliers     */
/* ======================================================================== */
/* Storage for an N x K weight (K % 256 == 0):
 *   codes   uint32 [N][K/32][3]   one 32-code chunk per 3 words (k = 32c..32c+31):
 *           codes a0..a15 (group 2c) and b0..b15 (group 2c+1); word j has five
 *           3-bit fields per 16-bit half (field i at bit 16h + 3i):
 *             word 0: a0..a4 | a5..a9
 *             word 1: a10 a11 a12 b0 b1 | a13 a14 a15 b2 b3
 *             word 2: b4..b8 | b9..b13
 *           b14 bit j -> bit 15 of word j; b15 bit j -> bit 31 of word j.
 *   stats1  uint32 [N][K/256][3]  16 six-bit fields per 256-weight block; field g
 *           at bit 6g of the 96-bit little-endian stream = c_s | c_z << 3
 *   stats2  fp16   [N][K/256][4]  SS_s, ZS_s, SS_z, ZS_z
 *   row_ptr int32 [N+1], col_idx int32 [nnz] (ascending per row), vals fp16 [nnz]
 * Dequantized weight: s_hat = SS_s (c_s - ZS_s), z_hat = SS_z (c_z - ZS_z),
 * w_hat = s_hat (q - z_hat) + (the CSR value at (n, k), if any).
 * Source: SpQR bulletin, "İddia ve Gerçeklik" (dense 3-bit groups of 16,
 * quantized statistics, sparse fp16 outliers of about 1%).                   */

/* Byte sizes and the outlier count nnz = floor(outlier_frac * (N*K)).
 * EINVAL unless N > 0, K > 0, K % 256 == 0 and 0 <= outlier_frac < 1. */
qlin_status spqr_sizes(int N, int K, double outlier_frac,
                       size_t* codes_bytes, size_t* stats1_bytes, size_t* stats2_bytes,
                       int64_t* nnz);

/* Encode fp32 W [N][K] (host).  Outliers: the nnz largest |w| of the whole
 * matrix, ties to the lower row-major index (magnitude stands in for the
 * Hessian-sensitivity criterion of the page).  The rest is quantized in fp32:
 * first level s = (max-min)/7, z = -min/s per group of 16 (s = 1, z = -min if
 * max == min); second level per 16 groups, separately for the scales and the
 * zeros: SS = fp16((max-min)/7), ZS = fp16(-min/SS) (SS = 1 if SS == 0 or ZS
 * is not finite), c = clamp(rint(v/SS + ZS), 0, 7); codes
 * q = clamp(rint(w/s_hat + z_hat), 0, 7) against the decoded statistics.
 * nnz_cap is the capacity of col_idx/vals; EINVAL if smaller than nnz. */
qlin_status spqr_pack(const float* W, int N, int K, double outlier_frac,
                      uint32_t* codes, uint32_t* stats1, uint16_t* stats2,
                      int32_t* row_ptr, int32_t* col_idx, uint16_t* vals,
                      int64_t nnz_cap, int64_t* nnz_out);

/* Device workspace bytes spqr_forward needs for this batch size (0: none) on
 * the current device.  Errors as spqr_forward's shape checks, EINVAL for a NULL
 * bytes. */
qlin_status spqr_workspace_bytes(int M, int K, int N, int y_dtype, size_t* bytes);

/* Y = X . (W_dense + W_sparse)^T on the GPU.  X fp16 [M][K] (device), Y [M][N]
 * (device, y_dtype QLIN_F16 or QLIN_F32).  The CSR row of output n is added into
 * the same fp32 accumulator as the dense dot product, in the same kernel pass.
 * Small batches run fused kernels on the exact codes (no workspace): M = 1 a
 * GEMV (v_dot2 on fp16 code pairs; rows longer than 8192 take the next
 * kernel), M = 2..6, and 7..8 where N > K, four rows per wave on the 4x4x4
 * matrix instruction (16 chunks x 4 tokens x 4 rows per instruction), both with
 * the group statistics applied in fp32.  Other batches up to M = 16 run a
 * matrix-core kernel:
 * a small prepass lays the activations out in the
 * workspace (operand order, group sums and a transposed copy, K * 68 bytes),
 * then each group's exact codes go through v_mfma_f32_16x16x16_f16 with the
 * group statistics applied in fp32.  workspace / workspace_bytes: as for
 * qlin_w4_forward (conventions at the top; size from spqr_workspace_bytes).
 * Requirements: 1 <= M <= 16, K % 256 == 0, row_ptr consistent with nnz
 * (row_ptr[0] = 0, row_ptr[N] = nnz, checked only for nnz >= 0 on the host:
 * the device arrays are trusted). */
qlin_status spqr_forward(const uint16_t* X, int M, int K,
                         const uint32_t* codes, const uint32_t* stats1, const uint16_t* stats2,
                         const int32_t* row_ptr, const int32_t* col_idx, const uint16_t* vals,
                         int64_t nnz, int N, void* Y, int y_dtype, void* workspace, size_t workspace_bytes,
                         hipStream_t stream);

/* Debug: unpack the dense codes (uint8 [N][K]) and the first-level statistic
 * codes c_s, c_z (uint8 [N][K/16]) on the GPU with the forward kernel's routine. */
qlin_status spqr_unpack(const uint32_t* codes, const uint32_t* stats1, int N, int K,
                        uint8_t* q, uint8_t* cs, uint8_t* cz, hipStream_t stream);

/* ======================================================================== */
/* SmoothQuant W8A8                                                          */
/* ======================================================================== */
/* Per-channel max |x| over the calibration rows (host, fp16 [Mcal][K]). */
qlin_status sq_act_absmax(const uint16_t* Xcal, int Mcal, int K, float* amax);

/* Smoothing vector (host): b_j = max_n |W[n][j]| over fp32 W [N][K];
 * s_j = amax_j^alpha / b_j^(1 - alpha) in fp64 (s_j = 1 if amax_j or b_j is 0);
 * s = fp32(s_j), inv_s = 1 / s in fp32.  alpha in [0, 1]; the page's range is
 * about 0.8-0.85 (SmoothQuant bulletin, "İddia ve Gerçeklik"). */
qlin_status sq_compute_smoothing(const float* amax, const float* W, int N, int K,
                                 double alpha, float* s, float* inv_s);

/* Fold s into W and quantize per output channel (host):
 * W' = W . diag(s); c_n = max_j |W'[n][j]|; w_scale_n = c_n / 127;
 * Wq = clamp(rint(W' * (127 / c_n)), -127, 127) (zero row: scale 0, codes 0). */
qlin_status sq_pack_weight(const float* W, const float* s, int N, int K,
                           int8_t* Wq, float* w_scale);

/* GPU: x~ = fp32(X) * inv_s per channel; per token a_m = max |x~|,
 * x_scale_m = a_m / 127, Xq = clamp(rint(x~ * (127 / a_m)), -127, 127)
 * (zero row: scale 0, codes 0).  Bit-exact with the host definition.
 * X fp16 [M][K], inv_s fp32 [K], Xq int8 [M][K], x_scale fp32 [M] (all device).
 * Requirements: M > 0, K > 0, K % 8 == 0. */
qlin_status sq_smooth_quant_act(const uint16_t* X, const float* inv_s, int M, int K,
                                int8_t* Xq, float* x_scale, hipStream_t stream);

/* Device workspace bytes sq_int8_gemm needs for this shape and output dtype on
 * the current device (0: none).  Errors as sq_int8_gemm's shape checks, EINVAL
 * for a NULL bytes. */
qlin_status sq_int8_gemm_workspace_bytes(int M, int N, int K, int y_dtype, size_t* bytes);

/* GPU: acc[m][n] = sum_k Xq[m][k] * Wq[n][k] (int32, exact);
 * Y[m][n] = y_dtype(float(acc) * x_scale[m] * w_scale[n]).
 * Y device [M][N] with y_dtype QLIN_F16 or QLIN_F32; acc_out, if not NULL,
 * receives acc (int32 [M][N], device).  Requirements: K % 64 == 0, K <= 131072.
 * Batches of more than 32 tokens (or more than 4 where K % 128 != 0) split the
 * K range of a tile over several workgroups (stream-K) through the caller's
 * workspace (conventions at the top); smaller batches need none. */
qlin_status sq_int8_gemm(const int8_t* Xq, const float* x_scale,
                         const int8_t* Wq, const float* w_scale,
                         int M, int N, int K, void* Y, int y_dtype,
                         int32_t* acc_out, void* workspace, size_t workspace_bytes,
                         hipStream_t stream);

/* ======================================================================== */
/* Dense fp16 layer (the unquantized baseline)                               */
/* ======================================================================== */
/* The 16-bit layer the pages measure their formats against: the SpQR and
 * SmoothQuant bulletins ("İddia ve Gerçeklik") quote speedups over 16-bit
 * inference, and the GPTQ bulletin ("İddia ve Gerçeklik") and the SmoothQuant
 * bulletin ("Ticari Etki") describe the weight-only gain fading as the batch
 * grows and the layer turns compute bound.  Used for that batch comparison. */

/* Device workspace bytes qlin_f16_gemm needs for this shape and output dtype
 * on the current device (never 0: every shape runs split-K).  Errors as
 * qlin_f16_gemm's shape checks, EINVAL for a NULL bytes. */
qlin_status qlin_f16_gemm_workspace_bytes(int M, int N, int K, int y_dtype, size_t* bytes);

/* GPU: Y[m][n] = y_dtype(sum_k X[m][k] W[n][k]), X fp16 [M][K], W fp16 [N][K]
 * (device, row-major), fp32 accumulation on v_mfma_f32_32x32x16_f16 (every
 * product exact), the K range of a tile split over workgroups (stream-K) with
 * the fp32 partials summed in K order: the result does not depend on timing.
 * Y device [M][N], y_dtype QLIN_F16, QLIN_BF16 or QLIN_F32, rounded once.
 * Requirements: K % 64 == 0, K <= 2^29; X, W, Y 16-byte aligned; workspace as
 * in the conventions at the top. */
qlin_status qlin_f16_gemm(const uint16_t* X, const uint16_t* W, int M, int N, int K, void* Y, int y_dtype,
                          void* workspace, size_t workspace_bytes, hipStream_t stream);

/* ======================================================================== */
/* Second-order encoders (host, offline): same storage, same forward calls   */
/* ======================================================================== */
/* The GPTQ bulletin ("İddia ve Gerçeklik") quantizes column by column with a
 * second-order error model: the inverse Hessian comes from the covariance of
 * the layer inputs, a Cholesky decomposition keeps it stable, and each
 * column's rounding error is pushed onto the columns not yet quantized.  The
 * SpQR bulletin ("İddia ve Gerçeklik") picks its outliers by Hessian-based
 * sensitivity.  All three calls are deterministic host functions; inputs and
 * outputs are host arrays owned by the caller; nothing is enqueued. */

/* H = (2 / n) X^T X in fp64 (host, [K][K], symmetric) from n calibration rows
 * X (fp32 [n][K], host), each entry summed over the rows in order.
 * EINVAL if n <= 0, K <= 0 or a pointer is NULL.  Cost O(n K^2). */
qlin_status qlin_hessian(const float* X, int n, int K, double* H);

/* Error-feedback (GPTQ-style) encode of fp32 W [N][K] into the storage of
 * qlin_w4_pack, given the undamped Hessian H (fp64 [K][K], finite, symmetric).
 * Damping: H + lam I with lam = damp * mean(diag H) (damp >= 0, 0.01 typical;
 * H = I when that mean is 0).  U = upper Cholesky factor of (H + lam I)^-1.
 * Columns j = 0 .. K-1 in order: a group's scale and zero are the
 * round-to-nearest ones (qlin_w4_pack's rule) of its current weights rounded to
 * fp32, computed at its first column; column j's code is that rule's code of its
 * current weight rounded to fp32; then, in fp64, e = (w_j - S (q - z)) / U[j][j]
 * and every later column k moves by -e U[j][k].  H proportional to I reproduces
 * qlin_w4_pack bit for bit.  EINVAL for bad sizes (as qlin_w4_sizes), NULL
 * pointers, damp < 0, a non-symmetric or non-finite H, or H + lam I not
 * positive definite.  Host memory: about 3 K^2 doubles; time O(K^3 + N K^2)
 * (a 4096 x 4096 layer takes seconds on a few host threads; K in the tens of
 * thousands needs tens of GB and hours). */
qlin_status qlin_w4_pack_gptq(const float* W, int N, int K, int G, const double* H, double damp,
                              uint32_t* qweight, uint16_t* scales, uint32_t* qzeros);

/* Act-order variant of qlin_w4_pack_gptq: columns are quantized in decreasing
 * order of diag(H), ties to the lower index (GPTQ bulletin, "Kod ve
 * Entegrasyon Haritası": act-order, and its advice to keep groups static).
 *   static_groups != 0: groups stay the natural runs of G columns, with the
 *     round-to-nearest statistics of the original weights (qlin_w4_pack's
 *     scales and zeros, bit for bit); storage in natural order, perm = identity;
 *     run it with qlin_w4_forward.
 *   static_groups == 0: groups are G consecutive columns of the quantization
 *     order (qlin_w4_pack_gptq applied to W[:, order] with H[order][:, order]);
 *     storage in that order, perm[t] = order[t]; run it with
 *     qlin_w4_forward_perm.
 * perm: host int32 [K] output.  Errors as qlin_w4_pack_gptq (EINVAL for a NULL
 * perm). */
qlin_status qlin_w4_pack_gptq_actorder(const float* W, int N, int K, int G, const double* H, double damp,
                                       int static_groups, uint32_t* qweight, uint16_t* scales, uint32_t* qzeros,
                                       int32_t* perm);

/* SpQR encode (outputs and sizes as spqr_pack) whose floor(p N K) outliers are
 * the weights of largest sensitivity, ties to the lower row-major index.  The
 * sensitivity of a weight is the drop of its group's (16 consecutive k of one
 * row) weighted 3-bit quantization error, sum_k c_k (w_k - w_hat_k)^2 with
 * c_k = diag(H + lam I) (damping as above) and real-valued min/max statistics
 * (s = (hi - lo) / 7, z = -lo / s; s = 1, z = -lo if hi == lo), when the weight
 * leaves the group and the other 15 are re-quantized without it; fp64, summed in
 * index order.  The rest of the encoding is spqr_pack's.  Errors as spqr_pack,
 * plus EINVAL for damp < 0 or a non-symmetric or non-finite H. */
qlin_status spqr_pack_hessian(const float* W, int N, int K, double outlier_frac, const double* H, double damp,
                              uint32_t* codes, uint32_t* stats1, uint16_t* stats2,
                              int32_t* row_ptr, int32_t* col_idx, uint16_t* vals,
                              int64_t nnz_cap, int64_t* nnz_out);

/* ======================================================================== */
/* Measurement aid                                                           */
/* ======================================================================== */
/* Plain streaming read of `bytes` (multiple of 16) from device buffer `buf`
 * with 16-byte vector loads: `grid` workgroups of 256 threads, `unroll` (1, 4
 * or 8) loads in flight per thread, optionally marked non-temporal.  Writes one
 * XOR word per workgroup to out[grid] (device) so the loads are kept.  It is the
 * achievable-bandwidth reference for the memory-bound kernels above (not part
 * of the layer computation). */
qlin_status qlin_stream_read(const void* buf, size_t bytes, int grid, int unroll, int nontemporal,
                             uint32_t* out, hipStream_t stream);

/* Plain device-to-device copy of `bytes` (multiple of 16, both buffers 16-byte
 * aligned) with 16-byte loads and stores: a kernel of known traffic (bytes read
 * + bytes written) against which hardware fetch/write counters are scaled. */
qlin_status qlin_stream_copy(void* dst, const void* src, size_t bytes, hipStream_t stream);

/* Dense matrix-core throughput reference: `grid` workgroups of 256 threads, each
 * wave issuing `iters` rounds of 4 independent register-only instructions of
 * kind 0 (v_mfma_f32_32x32x16_f16, 32768 flops each), 1 (..._bf16, 32768) or
 * 2 (v_mfma_i32_32x32x32_i8, 65536 ops); out (device float [grid * 4]) gets one
 * value per wave.  Not part of the layer computation. */
qlin_status qlin_mfma_peak(int kind, int iters, int grid, float* out, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* QLIN_H */
