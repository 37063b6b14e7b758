// Host encoders (offline, untimed): W4 round-to-nearest, SpQR hybrid, SmoothQuant.
//
// Built with -ffp-contract=off and without fast-math: every expression below is
// evaluated in fp32 (or fp64 where stated) in the written order, so the output
// bytes are a deterministic function of the input.

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <numeric>
#include <vector>

#include "common.hpp"
#include "host_pack.hpp"

using namespace qlin;

namespace {

inline float rne(float x) { return std::nearbyint(x); }   // default mode: ties to even
inline float clampf(float x, float lo, float hi) { return std::min(std::max(x, lo), hi); }

// ---------------------------------------------------------------------------
// SpQR helpers

// Three-bit 3-field placement of a 32-code chunk into three words (the layout
// documented in qlin.h: for every word, field i of the low half and field i of
// the high half hold codes of the same group).
inline void spqr_pack_chunk(const uint8_t* a, const uint8_t* b, uint32_t* w) {
  auto fld = [](uint32_t v, int half, int i) { return v << (16 * half + 3 * i); };
  uint32_t w0 = 0, w1 = 0, w2 = 0;
  for (int i = 0; i < 5; ++i) w0 |= fld(a[i], 0, i) | fld(a[5 + i], 1, i);
  for (int i = 0; i < 3; ++i) w1 |= fld(a[10 + i], 0, i) | fld(a[13 + i], 1, i);
  for (int i = 0; i < 2; ++i) w1 |= fld(b[i], 0, 3 + i) | fld(b[2 + i], 1, 3 + i);
  for (int i = 0; i < 5; ++i) w2 |= fld(b[4 + i], 0, i) | fld(b[9 + i], 1, i);
  uint32_t* ws[3] = {&w0, &w1, &w2};
  for (int j = 0; j < 3; ++j) {
    *ws[j] |= ((static_cast<uint32_t>(b[14]) >> j) & 1u) << 15;
    *ws[j] |= ((static_cast<uint32_t>(b[15]) >> j) & 1u) << 31;
  }
  w[0] = w0; w[1] = w1; w[2] = w2;
}

// 3-bit min/max quantizer over 16 values (the second level of SpQR).
struct Level2 {
  uint16_t SS, ZS;   // fp16 bits
  uint8_t c[16];
  float vhat[16];
};

inline Level2 spqr_level2(const float* v) {
  Level2 r;
  float lo = v[0], hi = v[0];
  for (int i = 1; i < 16; ++i) { lo = std::min(lo, v[i]); hi = std::max(hi, v[i]); }
  uint16_t SS = host_f32_to_f16((hi - lo) / 7.0f);
  bool bad = (SS & 0x7FFFu) == 0;
  uint16_t ZS = 0;
  if (!bad) {
    ZS = host_f32_to_f16(-lo / host_f16_to_f32(SS));
    bad = !host_f16_is_finite(ZS);
  }
  if (bad) {
    SS = 0x3C00u;                          // fp16 1.0
    ZS = host_f32_to_f16(-lo / 1.0f);
  }
  const float ss = host_f16_to_f32(SS), zs = host_f16_to_f32(ZS);
  for (int i = 0; i < 16; ++i) {
    const float c = clampf(rne(v[i] / ss + zs), 0.0f, 7.0f);
    r.c[i] = static_cast<uint8_t>(c);
    r.vhat[i] = ss * (c - zs);
  }
  r.SS = SS;
  r.ZS = ZS;
  return r;
}

}  // namespace

namespace qlin {

// Mask of the n entries first in the order (-key, index).
template <typename T>
std::vector<uint8_t> top_n_mask(const T* key, size_t total, int64_t n) {
  std::vector<uint8_t> mask(total, 0);
  if (n <= 0) return mask;
  if (static_cast<size_t>(n) >= total) { std::fill(mask.begin(), mask.end(), 1); return mask; }
  std::vector<T> tmp(key, key + total);
  // threshold t = the n-th largest key
  std::nth_element(tmp.begin(), tmp.begin() + (n - 1), tmp.end(), std::greater<T>());
  const T t = tmp[n - 1];
  tmp.clear(); tmp.shrink_to_fit();
  int64_t taken = 0;
  for (size_t i = 0; i < total; ++i) if (key[i] > t) { mask[i] = 1; ++taken; }
  for (size_t i = 0; i < total && taken < n; ++i)
    if (key[i] == t) { mask[i] = 1; ++taken; }
  return mask;
}
template std::vector<uint8_t> top_n_mask<float>(const float*, size_t, int64_t);
template std::vector<uint8_t> top_n_mask<double>(const double*, size_t, int64_t);

void w4_group_stats(const float* w, int G, uint16_t* S, float* s, float* z) {
  float lo = 0.0f, hi = 0.0f;
  for (int i = 0; i < G; ++i) { lo = std::min(lo, w[i]); hi = std::max(hi, w[i]); }
  uint16_t Sh = host_f32_to_f16((hi - lo) / 15.0f);
  if ((Sh & 0x7FFFu) == 0) Sh = 0x3C00u;
  *S = Sh;
  *s = host_f16_to_f32(Sh);
  *z = clampf(rne(-lo / *s), 0.0f, 15.0f);
}

uint32_t w4_code(float w, float s, float z) {
  return static_cast<uint32_t>(clampf(rne(w / s) + z, 0.0f, 15.0f));
}

}  // namespace qlin

extern "C" {

// ===========================================================================
// W4

qlin_status qlin_w4_sizes(int N, int K, int G, size_t* qb, size_t* sb, size_t* zb) {
  clear_error();
  if (N <= 0 || K <= 0 || G <= 0) return fail(QLIN_EINVAL, "qlin_w4_sizes: N, K, G must be positive");
  if (G % 8 != 0 || K % G != 0) return fail(QLIN_EINVAL, "qlin_w4_sizes: need G % 8 == 0 and K % G == 0");
  const size_t ng = static_cast<size_t>(K / G);
  if (qb) *qb = static_cast<size_t>(N) * (K / 8) * 4;
  if (sb) *sb = static_cast<size_t>(N) * ng * 2;
  if (zb) *zb = static_cast<size_t>(N) * ((ng + 7) / 8) * 4;
  return QLIN_OK;
}

qlin_status qlin_w4_pack(const float* W, int N, int K, int G,
                         uint32_t* qweight, uint16_t* scales, uint32_t* qzeros) {
  qlin_status st = qlin_w4_sizes(N, K, G, nullptr, nullptr, nullptr);
  if (st != QLIN_OK) return st;
  if (!W || !qweight || !scales || !qzeros) return fail(QLIN_EINVAL, "qlin_w4_pack: NULL pointer");
  const int ng = K / G, nzw = (ng + 7) / 8;
  std::vector<uint8_t> q(G);
  for (int n = 0; n < N; ++n) {
    const float* row = W + static_cast<size_t>(n) * K;
    uint32_t* qrow = qweight + static_cast<size_t>(n) * (K / 8);
    uint32_t* zrow = qzeros + static_cast<size_t>(n) * nzw;
    std::fill(qrow, qrow + K / 8, 0u);
    std::fill(zrow, zrow + nzw, 0u);
    for (int g = 0; g < ng; ++g) {
      const float* w = row + static_cast<size_t>(g) * G;
      uint16_t S;
      float s, z;
      w4_group_stats(w, G, &S, &s, &z);
      for (int i = 0; i < G; ++i) {
        const uint32_t code = w4_code(w[i], s, z);
        const int k = g * G + i;
        qrow[k / 8] |= code << (4 * (k % 8));
      }
      scales[static_cast<size_t>(n) * ng + g] = S;
      zrow[g / 8] |= static_cast<uint32_t>(z) << (4 * (g % 8));
    }
  }
  return QLIN_OK;
}

// ===========================================================================
// SpQR

qlin_status spqr_sizes(int N, int K, double p, size_t* cb, size_t* s1b, size_t* s2b, int64_t* nnz) {
  clear_error();
  if (N <= 0 || K <= 0) return fail(QLIN_EINVAL, "spqr_sizes: N and K must be positive");
  if (K % 256 != 0) return fail(QLIN_EINVAL, "spqr_sizes: K must be a multiple of 256");
  if (!(p >= 0.0 && p < 1.0)) return fail(QLIN_EINVAL, "spqr_sizes: outlier_frac must lie in [0, 1)");
  const int64_t total = static_cast<int64_t>(N) * K;
  const int64_t n_out = static_cast<int64_t>(std::floor(p * static_cast<double>(total)));
  if (n_out > INT32_MAX) return fail(QLIN_EUNSUPPORTED, "spqr_sizes: more than 2^31-1 outliers");
  if (cb) *cb = static_cast<size_t>(N) * (K / 32) * 3 * 4;
  if (s1b) *s1b = static_cast<size_t>(N) * (K / 256) * 3 * 4;
  if (s2b) *s2b = static_cast<size_t>(N) * (K / 256) * 4 * 2;
  if (nnz) *nnz = n_out;
  return QLIN_OK;
}

qlin_status spqr_pack(const float* W, int N, int K, double p,
                      uint32_t* codes, uint32_t* stats1, uint16_t* stats2,
                      int32_t* row_ptr, int32_t* col_idx, uint16_t* vals,
                      int64_t nnz_cap, int64_t* nnz_out) {
  int64_t n_out = 0;
  qlin_status st = spqr_sizes(N, K, p, nullptr, nullptr, nullptr, &n_out);
  if (st != QLIN_OK) return st;
  if (!W || !codes || !stats1 || !stats2 || !row_ptr)
    return fail(QLIN_EINVAL, "spqr_pack: NULL pointer");
  if (n_out > 0 && (!col_idx || !vals)) return fail(QLIN_EINVAL, "spqr_pack: NULL CSR arrays");
  if (nnz_cap < n_out) return fail(QLIN_EINVAL, "spqr_pack: nnz_cap smaller than the outlier count");

  const size_t total = static_cast<size_t>(N) * K;
  std::vector<float> mag(total);
  for (size_t i = 0; i < total; ++i) mag[i] = std::fabs(W[i]);
  const std::vector<uint8_t> mask = top_n_mask(mag.data(), total, n_out);
  mag.clear(); mag.shrink_to_fit();
  spqr_encode_masked(W, N, K, mask.data(), codes, stats1, stats2, row_ptr, col_idx, vals, nnz_out);
  return QLIN_OK;
}

}  // extern "C"

namespace qlin {

void spqr_encode_masked(const float* W, int N, int K, const uint8_t* mask,
                        uint32_t* codes, uint32_t* stats1, uint16_t* stats2,
                        int32_t* row_ptr, int32_t* col_idx, uint16_t* vals, int64_t* nnz_out) {
  // CSR, rows = output channels, columns ascending
  int64_t nz = 0;
  row_ptr[0] = 0;
  for (int n = 0; n < N; ++n) {
    const size_t base = static_cast<size_t>(n) * K;
    for (int k = 0; k < K; ++k) {
      if (mask[base + k]) {
        col_idx[nz] = k;
        vals[nz] = host_f32_to_f16(W[base + k]);
        ++nz;
      }
    }
    row_ptr[n + 1] = static_cast<int32_t>(nz);
  }

  const int ng = K / 16, nb = K / 256;
  std::vector<float> R(K), s1(ng), z1(ng), sh(ng), zh(ng);
  std::vector<uint8_t> cs(ng), cz(ng), q(K);
  for (int n = 0; n < N; ++n) {
    const size_t base = static_cast<size_t>(n) * K;
    for (int k = 0; k < K; ++k) R[k] = mask[base + k] ? 0.0f : W[base + k];
    // first level
    for (int g = 0; g < ng; ++g) {
      float lo = R[16 * g], hi = R[16 * g];
      for (int i = 1; i < 16; ++i) { lo = std::min(lo, R[16 * g + i]); hi = std::max(hi, R[16 * g + i]); }
      if (hi == lo) { s1[g] = 1.0f; z1[g] = -lo; }
      else { s1[g] = (hi - lo) / 7.0f; z1[g] = -lo / s1[g]; }
    }
    // second level, per block of 16 groups
    for (int b = 0; b < nb; ++b) {
      const Level2 ls = spqr_level2(&s1[16 * b]);
      const Level2 lz = spqr_level2(&z1[16 * b]);
      uint16_t* s2 = stats2 + (static_cast<size_t>(n) * nb + b) * 4;
      s2[0] = ls.SS; s2[1] = ls.ZS; s2[2] = lz.SS; s2[3] = lz.ZS;
      uint32_t* w = stats1 + (static_cast<size_t>(n) * nb + b) * 3;
      w[0] = w[1] = w[2] = 0;
      for (int g = 0; g < 16; ++g) {
        cs[16 * b + g] = ls.c[g];
        cz[16 * b + g] = lz.c[g];
        sh[16 * b + g] = ls.vhat[g];
        zh[16 * b + g] = lz.vhat[g];
        const uint32_t f = static_cast<uint32_t>(ls.c[g]) | (static_cast<uint32_t>(lz.c[g]) << 3);
        const int bit = 6 * g, wi = bit / 32, off = bit % 32;
        w[wi] |= f << off;
        if (off > 26) w[wi + 1] |= f >> (32 - off);
      }
    }
    // codes against the decoded statistics
    for (int g = 0; g < ng; ++g) {
      for (int i = 0; i < 16; ++i) {
        const float t = (sh[g] == 0.0f) ? zh[g] : (R[16 * g + i] / sh[g] + zh[g]);
        q[16 * g + i] = static_cast<uint8_t>(clampf(rne(t), 0.0f, 7.0f));
      }
    }
    uint32_t* crow = codes + static_cast<size_t>(n) * (K / 32) * 3;
    for (int c = 0; c < K / 32; ++c) spqr_pack_chunk(&q[32 * c], &q[32 * c + 16], crow + 3 * c);
  }
  if (nnz_out) *nnz_out = nz;
}

}  // namespace qlin

extern "C" {

// ===========================================================================
// SmoothQuant (host side)

qlin_status sq_act_absmax(const uint16_t* Xcal, int Mcal, int K, float* amax) {
  clear_error();
  if (Mcal <= 0 || K <= 0) return fail(QLIN_EINVAL, "sq_act_absmax: Mcal and K must be positive");
  if (!Xcal || !amax) return fail(QLIN_EINVAL, "sq_act_absmax: NULL pointer");
  for (int j = 0; j < K; ++j) amax[j] = 0.0f;
  for (int m = 0; m < Mcal; ++m)
    for (int j = 0; j < K; ++j)
      amax[j] = std::max(amax[j], std::fabs(host_f16_to_f32(Xcal[static_cast<size_t>(m) * K + j])));
  return QLIN_OK;
}

qlin_status sq_compute_smoothing(const float* amax, const float* W, int N, int K,
                                 double alpha, float* s, float* inv_s) {
  clear_error();
  if (N <= 0 || K <= 0) return fail(QLIN_EINVAL, "sq_compute_smoothing: N and K must be positive");
  if (!amax || !W || !s || !inv_s) return fail(QLIN_EINVAL, "sq_compute_smoothing: NULL pointer");
  if (!(alpha >= 0.0 && alpha <= 1.0)) return fail(QLIN_EINVAL, "sq_compute_smoothing: alpha must lie in [0, 1]");
  std::vector<float> b(K, 0.0f);
  for (int n = 0; n < N; ++n)
    for (int j = 0; j < K; ++j) b[j] = std::max(b[j], std::fabs(W[static_cast<size_t>(n) * K + j]));
  for (int j = 0; j < K; ++j) {
    const double a = amax[j], bj = b[j];
    const double sj = (a == 0.0 || bj == 0.0) ? 1.0 : std::pow(a, alpha) / std::pow(bj, 1.0 - alpha);
    s[j] = static_cast<float>(sj);
    inv_s[j] = 1.0f / s[j];
  }
  return QLIN_OK;
}

qlin_status sq_pack_weight(const float* W, const float* s, int N, int K, int8_t* Wq, float* w_scale) {
  clear_error();
  if (N <= 0 || K <= 0) return fail(QLIN_EINVAL, "sq_pack_weight: N and K must be positive");
  if (!W || !s || !Wq || !w_scale) return fail(QLIN_EINVAL, "sq_pack_weight: NULL pointer");
  std::vector<float> wp(K);
  for (int n = 0; n < N; ++n) {
    const float* row = W + static_cast<size_t>(n) * K;
    float c = 0.0f;
    for (int j = 0; j < K; ++j) { wp[j] = row[j] * s[j]; c = std::max(c, std::fabs(wp[j])); }
    const float r = (c == 0.0f) ? 0.0f : 127.0f / c;
    int8_t* qrow = Wq + static_cast<size_t>(n) * K;
    for (int j = 0; j < K; ++j) qrow[j] = static_cast<int8_t>(clampf(rne(wp[j] * r), -127.0f, 127.0f));
    w_scale[n] = (c == 0.0f) ? 0.0f : c / 127.0f;
  }
  return QLIN_OK;
}

}  // extern "C"
