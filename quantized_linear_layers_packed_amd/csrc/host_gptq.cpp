// Second-order (Hessian-aware) host encoders, offline and untimed:
//   * GPTQ-style error feedback into the 4-bit storage (GPTQ bulletin,
//     "İddia ve Gerçeklik": inverse Hessian from the covariance of the layer
//     inputs, stabilised with a Cholesky decomposition; columns quantized in
//     blocks; each column's rounding error pushed onto the columns not yet
//     quantized);
//   * SpQR outliers chosen by a Hessian-weighted sensitivity (SpQR bulletin,
//     "İddia ve Gerçeklik").
//
// Definitions implemented (the pages give no formulas):
//   H = (2 / n) X^T X in fp64; damped H + lam I with lam = damp * mean(diag H)
//   (diagonal summed left to right), or I when that mean is 0.  U = upper
//   Cholesky factor of (H + lam I)^-1.  Columns j = 0 .. K-1 in order: at the
//   first column of a group the round-to-nearest statistics of the 4-bit storage
//   are taken from the group's current weights rounded to fp32; the code of
//   column j is the round-to-nearest code of its current weight rounded to fp32;
//   then e = (w_j - S (q - z)) / U[j][j] and w_k -= e * U[j][k] for k > j, in
//   fp64.  Columns are processed in blocks of 128 with the updates of later
//   blocks deferred and applied in column order, which gives the same numbers
//   as updating every later column immediately.
//
// Built without floating-point contraction, so every product and sum rounds on
// its own, in the written order.

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <string>
#include <thread>
#include <vector>

#include "common.hpp"
#include "host_pack.hpp"

using namespace qlin;

namespace {

// Static partition of [0, n) over the host threads; `work` is the rough cost of
// one item in multiply-adds (small loops stay on the calling thread).
template <class F>
void parallel_for(int64_t n, int64_t work, F&& f) {
  const int64_t hw = std::max<int64_t>(1, static_cast<int64_t>(std::thread::hardware_concurrency()));
  const int64_t nt = std::min<int64_t>({hw, std::max<int64_t>(1, n / 4), std::max<int64_t>(1, n * work / 200000)});
  if (nt <= 1) {
    for (int64_t i = 0; i < n; ++i) f(i);
    return;
  }
  std::vector<std::thread> pool;
  pool.reserve(nt);
  for (int64_t t = 0; t < nt; ++t)
    pool.emplace_back([&, t] {
      for (int64_t i = t; i < n; i += nt) f(i);    // interleaved: triangular loops stay balanced
    });
  for (auto& th : pool) th.join();
}

// In-place lower Cholesky factor of the symmetric K x K row-major matrix A
// (only the lower triangle is read; the strict upper triangle is zeroed).
// Returns false if A is not positive definite.
bool cholesky_lower(std::vector<double>& A, int K) {
  for (int j = 0; j < K; ++j) {
    double* rj = &A[static_cast<size_t>(j) * K];
    double d = rj[j];
    for (int k = 0; k < j; ++k) d -= rj[k] * rj[k];
    if (!(d > 0.0) || !std::isfinite(d)) return false;
    const double ljj = std::sqrt(d);
    rj[j] = ljj;
    parallel_for(K - j - 1, j, [&](int64_t t) {
      const int i = j + 1 + static_cast<int>(t);
      double* ri = &A[static_cast<size_t>(i) * K];
      double v = ri[j];
      for (int k = 0; k < j; ++k) v -= ri[k] * rj[k];
      ri[j] = v / ljj;
    });
  }
  for (int i = 0; i < K; ++i)
    for (int k = i + 1; k < K; ++k) A[static_cast<size_t>(i) * K + k] = 0.0;
  return true;
}

// (H + lam I)^-1 from the lower Cholesky factor L: with Linv = L^-1,
// H^-1 = Linv^T Linv.  Returns false if H + lam I is not positive definite.
bool spd_inverse(std::vector<double>& A, int K) {
  if (!cholesky_lower(A, K)) return false;
  // Columns of Linv (stored as rows of T: T[c][i] = Linv[i][c], zero for i < c)
  std::vector<double> T(static_cast<size_t>(K) * K, 0.0);
  parallel_for(K, static_cast<int64_t>(K) * K / 4, [&](int64_t cc) {
    const int c = static_cast<int>(cc);
    double* x = &T[static_cast<size_t>(c) * K];
    for (int i = c; i < K; ++i) {
      const double* li = &A[static_cast<size_t>(i) * K];
      double v = (i == c) ? 1.0 : 0.0;
      for (int k = c; k < i; ++k) v -= li[k] * x[k];
      x[i] = v / li[i];
    }
  });
  // H^-1[a][b] = sum_{k >= max(a, b)} Linv[k][a] Linv[k][b]
  parallel_for(K, static_cast<int64_t>(K) * K / 4, [&](int64_t aa) {
    const int a = static_cast<int>(aa);
    const double* ta = &T[static_cast<size_t>(a) * K];
    for (int b = 0; b <= a; ++b) {
      const double* tb = &T[static_cast<size_t>(b) * K];
      double v = 0.0;
      for (int k = a; k < K; ++k) v += ta[k] * tb[k];
      A[static_cast<size_t>(a) * K + b] = v;
      A[static_cast<size_t>(b) * K + a] = v;
    }
  });
  return true;
}

// Damped copy of H (lam = damp * mean(diag H); identity if that mean is 0).
std::vector<double> damped(const double* H, int K, double damp) {
  std::vector<double> A(H, H + static_cast<size_t>(K) * K);
  double total = 0.0;
  for (int i = 0; i < K; ++i) total += A[static_cast<size_t>(i) * K + i];
  const double mean = total / K;
  if (mean == 0.0) {
    std::fill(A.begin(), A.end(), 0.0);
    for (int i = 0; i < K; ++i) A[static_cast<size_t>(i) * K + i] = 1.0;
    return A;
  }
  const double lam = damp * mean;
  for (int i = 0; i < K; ++i) A[static_cast<size_t>(i) * K + i] += lam;
  return A;
}

bool finite_and_symmetric(const double* H, int K) {
  for (int i = 0; i < K; ++i)
    for (int j = 0; j <= i; ++j) {
      const double a = H[static_cast<size_t>(i) * K + j], b = H[static_cast<size_t>(j) * K + i];
      if (!std::isfinite(a) || a != b) return false;
    }
  return true;
}

// Weighted 3-bit min/max quantization error of one set of weights (fp64, real
// statistics), summed in index order.
double group_error(const double* w, const double* c, int n) {
  double lo = w[0], hi = w[0];
  for (int i = 1; i < n; ++i) { lo = std::min(lo, w[i]); hi = std::max(hi, w[i]); }
  double s, z;
  if (hi == lo) { s = 1.0; z = -lo; }
  else { s = (hi - lo) / 7.0; z = -lo / s; }
  double err = 0.0;
  for (int i = 0; i < n; ++i) {
    const double q = std::min(std::max(std::nearbyint(w[i] / s + z), 0.0), 7.0);
    const double d = w[i] - s * (q - z);
    err += c[i] * (d * d);
  }
  return err;
}

constexpr int kBlock = 128;     // columns per deferred-update block
constexpr int kRowBatch = 32;   // rows per worker batch (U streams once per batch)

// Shared GPTQ core.  Columns are quantized in the order `order` (natural order
// unless act_order: decreasing diag(H), ties to the lower index).  Groups:
//   * static_groups: natural groups of G columns, with round-to-nearest
//     statistics of the original weights; storage in natural order;
//   * otherwise: G consecutive columns of the quantization order, statistics of
//     the current weights at the group's first column; storage in quantization
//     order (column t of the storage is original column order[t]).
qlin_status gptq_encode(const char* fn, const float* W, int N, int K, int G, const double* H, double damp,
                        bool act_order, bool static_groups, uint32_t* qweight, uint16_t* scales,
                        uint32_t* qzeros, int32_t* perm) {
  qlin_status st = qlin_w4_sizes(N, K, G, nullptr, nullptr, nullptr);
  if (st != QLIN_OK) return st;
  if (!W || !H || !qweight || !scales || !qzeros) return fail(QLIN_EINVAL, std::string(fn) + ": NULL pointer");
  if (!(damp >= 0.0) || !std::isfinite(damp)) return fail(QLIN_EINVAL, std::string(fn) + ": damp must be >= 0");
  if (!finite_and_symmetric(H, K)) return fail(QLIN_EINVAL, std::string(fn) + ": H must be finite and symmetric");

  std::vector<int> order(K);
  for (int k = 0; k < K; ++k) order[k] = k;
  if (act_order)
    std::stable_sort(order.begin(), order.end(), [&](int a, int b) {
      return H[static_cast<size_t>(a) * K + a] > H[static_cast<size_t>(b) * K + b];
    });
  if (perm)
    for (int t = 0; t < K; ++t) perm[t] = static_groups ? t : order[t];

  // U = upper Cholesky factor of (Hp + lam I)^-1 with Hp = H in quantization order
  std::vector<double> Hp(static_cast<size_t>(K) * K);
  for (int a = 0; a < K; ++a)
    for (int b = 0; b < K; ++b) Hp[static_cast<size_t>(a) * K + b] = H[static_cast<size_t>(order[a]) * K + order[b]];
  std::vector<double> A = damped(Hp.data(), K, damp);
  Hp.clear();
  Hp.shrink_to_fit();
  if (!spd_inverse(A, K) || !cholesky_lower(A, K))
    return fail(QLIN_EINVAL, std::string(fn) + ": H + lam I is not positive definite (raise damp)");
  std::vector<double> U(static_cast<size_t>(K) * K, 0.0);
  for (int i = 0; i < K; ++i)
    for (int j = 0; j <= i; ++j) U[static_cast<size_t>(j) * K + i] = A[static_cast<size_t>(i) * K + j];
  A.clear();
  A.shrink_to_fit();

  const int ng = K / G, nzw = (ng + 7) / 8;
  const int nbatch = (N + kRowBatch - 1) / kRowBatch;
  parallel_for(nbatch, static_cast<int64_t>(kRowBatch) * K * K / 2, [&](int64_t b) {
    const int r0 = static_cast<int>(b) * kRowBatch, nr = std::min(kRowBatch, N - r0);
    // current weights of the batch, in quantization order
    std::vector<double> Wc(static_cast<size_t>(nr) * K);
    for (int r = 0; r < nr; ++r)
      for (int t = 0; t < K; ++t) Wc[static_cast<size_t>(r) * K + t] = W[static_cast<size_t>(r0 + r) * K + order[t]];
    std::vector<double> E(static_cast<size_t>(nr) * kBlock);     // scaled errors of the current block
    std::vector<float> s(static_cast<size_t>(nr) * ng), z(static_cast<size_t>(nr) * ng), g32(G);
    for (int r = 0; r < nr; ++r) {
      std::fill(qweight + static_cast<size_t>(r0 + r) * (K / 8), qweight + static_cast<size_t>(r0 + r + 1) * (K / 8), 0u);
      std::fill(qzeros + static_cast<size_t>(r0 + r) * nzw, qzeros + static_cast<size_t>(r0 + r + 1) * nzw, 0u);
    }
    auto set_group = [&](int r, int g, const float* w) {
      uint16_t S;
      w4_group_stats(w, G, &S, &s[static_cast<size_t>(r) * ng + g], &z[static_cast<size_t>(r) * ng + g]);
      scales[static_cast<size_t>(r0 + r) * ng + g] = S;
      qzeros[static_cast<size_t>(r0 + r) * nzw + g / 8] |=
          static_cast<uint32_t>(z[static_cast<size_t>(r) * ng + g]) << (4 * (g % 8));
    };
    if (static_groups)
      for (int r = 0; r < nr; ++r)
        for (int g = 0; g < ng; ++g) set_group(r, g, W + static_cast<size_t>(r0 + r) * K + static_cast<size_t>(g) * G);
    for (int j0 = 0; j0 < K; j0 += kBlock) {
      const int j1 = std::min(K, j0 + kBlock);
      for (int j = j0; j < j1; ++j) {
        const double* uj = &U[static_cast<size_t>(j) * K];
        const int pos = static_groups ? order[j] : j;     // storage column of quantization step j
        const int g = pos / G;
        for (int r = 0; r < nr; ++r) {
          double* w = &Wc[static_cast<size_t>(r) * K];
          if (!static_groups && j % G == 0) {
            for (int i = 0; i < G; ++i) g32[i] = static_cast<float>(w[j + i]);
            set_group(r, g, g32.data());
          }
          const float sr = s[static_cast<size_t>(r) * ng + g], zr = z[static_cast<size_t>(r) * ng + g];
          const uint32_t q = w4_code(static_cast<float>(w[j]), sr, zr);
          qweight[static_cast<size_t>(r0 + r) * (K / 8) + pos / 8] |= q << (4 * (pos % 8));
          const double w_hat = static_cast<double>(sr) * (static_cast<double>(q) - static_cast<double>(zr));
          const double e = (w[j] - w_hat) / uj[j];
          E[static_cast<size_t>(r) * kBlock + (j - j0)] = e;
          for (int k = j + 1; k < j1; ++k) w[k] -= e * uj[k];      // inside the block: now
        }
      }
      // later blocks: the block's updates, applied in column order
      for (int r = 0; r < nr; ++r) {
        double* w = &Wc[static_cast<size_t>(r) * K];
        const double* e = &E[static_cast<size_t>(r) * kBlock];
        for (int j = j0; j < j1; ++j) {
          const double* uj = &U[static_cast<size_t>(j) * K];
          const double ej = e[j - j0];
          for (int k = j1; k < K; ++k) w[k] -= ej * uj[k];
        }
      }
    }
  });
  return QLIN_OK;
}

}  // namespace

extern "C" {

qlin_status qlin_hessian(const float* X, int n, int K, double* H) {
  clear_error();
  if (n <= 0 || K <= 0) return fail(QLIN_EINVAL, "qlin_hessian: n and K must be positive");
  if (!X || !H) return fail(QLIN_EINVAL, "qlin_hessian: NULL pointer");
  // columns of X as contiguous fp64 rows
  std::vector<double> Xt(static_cast<size_t>(K) * n);
  for (int m = 0; m < n; ++m)
    for (int k = 0; k < K; ++k) Xt[static_cast<size_t>(k) * n + m] = X[static_cast<size_t>(m) * K + k];
  const double f = 2.0 / n;
  parallel_for(K, static_cast<int64_t>(K) * n / 2, [&](int64_t ii) {
    const int i = static_cast<int>(ii);
    const double* xi = &Xt[static_cast<size_t>(i) * n];
    for (int j = 0; j <= i; ++j) {
      const double* xj = &Xt[static_cast<size_t>(j) * n];
      double v = 0.0;
      for (int m = 0; m < n; ++m) v += xi[m] * xj[m];
      H[static_cast<size_t>(i) * K + j] = f * v;
      H[static_cast<size_t>(j) * K + i] = f * v;
    }
  });
  return QLIN_OK;
}

qlin_status qlin_w4_pack_gptq(const float* W, int N, int K, int G, const double* H, double damp,
                              uint32_t* qweight, uint16_t* scales, uint32_t* qzeros) {
  return gptq_encode("qlin_w4_pack_gptq", W, N, K, G, H, damp, /*act_order=*/false, /*static_groups=*/false,
                     qweight, scales, qzeros, nullptr);
}

qlin_status qlin_w4_pack_gptq_actorder(const float* W, int N, int K, int G, const double* H, double damp,
                                       int static_groups, uint32_t* qweight, uint16_t* scales, uint32_t* qzeros,
                                       int32_t* perm) {
  if (!perm) return fail(QLIN_EINVAL, "qlin_w4_pack_gptq_actorder: NULL pointer");
  return gptq_encode("qlin_w4_pack_gptq_actorder", W, N, K, G, H, damp, /*act_order=*/true, static_groups != 0,
                     qweight, scales, qzeros, perm);
}

qlin_status spqr_pack_hessian(const float* W, int N, int K, double p, const double* H, double damp,
                              uint32_t* codes, uint32_t* stats1, uint16_t* stats2,
                              int32_t* row_ptr, int32_t* col_idx, uint16_t* vals,
                              int64_t nnz_cap, int64_t* nnz_out) {
  int64_t n_out = 0;
  qlin_status st = spqr_sizes(N, K, p, nullptr, nullptr, nullptr, &n_out);
  if (st != QLIN_OK) return st;
  if (!W || !H || !codes || !stats1 || !stats2 || !row_ptr)
    return fail(QLIN_EINVAL, "spqr_pack_hessian: NULL pointer");
  if (n_out > 0 && (!col_idx || !vals)) return fail(QLIN_EINVAL, "spqr_pack_hessian: NULL CSR arrays");
  if (nnz_cap < n_out) return fail(QLIN_EINVAL, "spqr_pack_hessian: nnz_cap smaller than the outlier count");
  if (!(damp >= 0.0) || !std::isfinite(damp)) return fail(QLIN_EINVAL, "spqr_pack_hessian: damp must be >= 0");
  if (!finite_and_symmetric(H, K)) return fail(QLIN_EINVAL, "spqr_pack_hessian: H must be finite and symmetric");

  const std::vector<double> A = damped(H, K, damp);
  std::vector<double> c(K);
  for (int k = 0; k < K; ++k) c[k] = A[static_cast<size_t>(k) * K + k];

  // leave-one-out sensitivity of every weight, per group of 16
  const size_t total = static_cast<size_t>(N) * K;
  std::vector<double> sens(total);
  parallel_for(N, static_cast<int64_t>(K) * 17 * 16 / 16, [&](int64_t nn) {
    const size_t base = static_cast<size_t>(nn) * K;
    double w[16], wo[15], co[15];
    for (int g = 0; g < K / 16; ++g) {
      for (int i = 0; i < 16; ++i) w[i] = W[base + 16 * g + i];
      const double* cg = &c[16 * g];
      const double full = group_error(w, cg, 16);
      for (int i = 0; i < 16; ++i) {
        int o = 0;
        for (int j = 0; j < 16; ++j)
          if (j != i) { wo[o] = w[j]; co[o] = cg[j]; ++o; }
        sens[base + 16 * g + i] = full - group_error(wo, co, 15);
      }
    }
  });
  const std::vector<uint8_t> mask = top_n_mask(sens.data(), total, n_out);
  sens.clear();
  sens.shrink_to_fit();
  spqr_encode_masked(W, N, K, mask.data(), codes, stats1, stats2, row_ptr, col_idx, vals, nnz_out);
  return QLIN_OK;
}

}  // extern "C"
