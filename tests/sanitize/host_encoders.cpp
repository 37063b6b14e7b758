// Driver for the sanitizer build of the host encoders (AddressSanitizer +
// UndefinedBehaviorSanitizer, every report fatal).  Runs each host encoder of
// the C ABI on small deterministic inputs, edge cases included (zero and
// constant rows and groups, no outliers, the largest fp16-range weights, both
// act-order variants), and every argument check that must refuse a call, then
// writes each input and output array as raw bytes into the directory given as
// argv[1] so the regular build's outputs can be compared byte for byte.
// Exit status 0 only if every call returned the expected status.

#include <cmath>
#include <cstdint>
#include <cstdio>
#include <string>
#include <vector>

#include "qlin.h"

namespace {

std::string g_dir;
int g_failures = 0;

// splitmix64: deterministic inputs without any library generator
uint64_t g_state = 0x5EED5EED12345678ull;
uint64_t next_u64() {
  uint64_t z = (g_state += 0x9E3779B97F4A7C15ull);
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}
double uniform() { return static_cast<double>(next_u64() >> 11) * (1.0 / 9007199254740992.0); }
float normal(float sigma) {
  const double u1 = uniform() + 1e-300, u2 = uniform();
  return static_cast<float>(sigma * std::sqrt(-2.0 * std::log(u1)) * std::cos(6.283185307179586 * u2));
}

template <typename T>
void put(const char* name, const std::vector<T>& v) {
  const std::string path = g_dir + "/" + name;
  FILE* f = std::fopen(path.c_str(), "wb");
  if (!f) {
    std::fprintf(stderr, "cannot write %s\n", path.c_str());
    ++g_failures;
    return;
  }
  if (!v.empty()) std::fwrite(v.data(), sizeof(T), v.size(), f);
  std::fclose(f);
}

void expect(const char* what, qlin_status got, qlin_status want) {
  if (got != want) {
    std::fprintf(stderr, "%s: status %d, expected %d (%s)\n", what, got, want, qlin_last_error());
    ++g_failures;
  }
}

std::vector<float> weights(int N, int K, float sigma) {
  std::vector<float> W(static_cast<size_t>(N) * K);
  for (auto& w : W) w = normal(sigma);
  return W;
}

// fp16 bits of x, for x = 0 or a multiple of 2^-4 with 2^-4 <= |x| < 2048 (exact)
uint16_t f16_bits(float x) {
  if (x == 0.0f) return 0;
  const uint16_t sign = x < 0 ? 0x8000u : 0u;
  int e = 0;
  const double f = std::frexp(std::fabs(static_cast<double>(x)), &e);    // |x| = f 2^e, f in [0.5, 1)
  const uint32_t mant = static_cast<uint32_t>(std::ldexp(f, 11)) & 0x3FFu; // 10 bits below the leading one
  return static_cast<uint16_t>(sign | (static_cast<uint32_t>(e - 1 + 15) << 10) | mant);
}

void w4_cases() {
  // 5 x 256, groups of 128: random; 3 x 64, groups of 32: a zero row, a constant
  // row and a row at the edge of the fp16 range
  {
    const int N = 5, K = 256, G = 128;
    std::vector<float> W = weights(N, K, 0.02f);
    size_t qb, sb, zb;
    expect("w4_sizes", qlin_w4_sizes(N, K, G, &qb, &sb, &zb), QLIN_OK);
    std::vector<uint32_t> qw(qb / 4), qz(zb / 4);
    std::vector<uint16_t> sc(sb / 2);
    expect("w4_pack random", qlin_w4_pack(W.data(), N, K, G, qw.data(), sc.data(), qz.data()), QLIN_OK);
    put("w4a_W", W);
    put("w4a_qweight", qw);
    put("w4a_scales", sc);
    put("w4a_qzeros", qz);
  }
  {
    const int N = 3, K = 64, G = 32;
    std::vector<float> W(static_cast<size_t>(N) * K, 0.0f);
    for (int k = 0; k < K; ++k) {
      W[K + k] = 0.75f;
      W[2 * K + k] = (k & 1) ? 60000.0f : -60000.0f * static_cast<float>(k % 5) / 4.0f;
    }
    size_t qb, sb, zb;
    expect("w4_sizes edge", qlin_w4_sizes(N, K, G, &qb, &sb, &zb), QLIN_OK);
    std::vector<uint32_t> qw(qb / 4), qz(zb / 4);
    std::vector<uint16_t> sc(sb / 2);
    expect("w4_pack edge", qlin_w4_pack(W.data(), N, K, G, qw.data(), sc.data(), qz.data()), QLIN_OK);
    put("w4b_W", W);
    put("w4b_qweight", qw);
    put("w4b_scales", sc);
    put("w4b_qzeros", qz);
    // refused: K not a multiple of G, NULL output
    expect("w4_pack K % G", qlin_w4_pack(W.data(), N, 48, G, qw.data(), sc.data(), qz.data()), QLIN_EINVAL);
    expect("w4_pack NULL", qlin_w4_pack(W.data(), N, K, G, nullptr, sc.data(), qz.data()), QLIN_EINVAL);
  }
}

void spqr_case(const char* tag, int N, int K, double p, std::vector<float> W) {
  size_t cb, s1b, s2b;
  int64_t nnz = 0;
  expect("spqr_sizes", spqr_sizes(N, K, p, &cb, &s1b, &s2b, &nnz), QLIN_OK);
  std::vector<uint32_t> codes(cb / 4), st1(s1b / 4);
  std::vector<uint16_t> st2(s2b / 2), vals(static_cast<size_t>(nnz));
  std::vector<int32_t> rp(N + 1), ci(static_cast<size_t>(nnz));
  int64_t got = -1;
  expect("spqr_pack", spqr_pack(W.data(), N, K, p, codes.data(), st1.data(), st2.data(), rp.data(), ci.data(),
                                vals.data(), nnz, &got), QLIN_OK);
  if (got != nnz) {
    std::fprintf(stderr, "spqr_pack %s: nnz %lld, expected %lld\n", tag, static_cast<long long>(got),
                 static_cast<long long>(nnz));
    ++g_failures;
  }
  const std::string t(tag);
  put((t + "_W").c_str(), W);
  put((t + "_codes").c_str(), codes);
  put((t + "_stats1").c_str(), st1);
  put((t + "_stats2").c_str(), st2);
  put((t + "_row_ptr").c_str(), rp);
  put((t + "_col_idx").c_str(), ci);
  put((t + "_val").c_str(), vals);
  if (nnz > 0)
    expect("spqr_pack small capacity", spqr_pack(W.data(), N, K, p, codes.data(), st1.data(), st2.data(), rp.data(),
                                                 ci.data(), vals.data(), nnz - 1, &got), QLIN_EINVAL);
}

void spqr_cases() {
  spqr_case("spqra", 7, 256, 0.0, weights(7, 256, 0.02f));
  std::vector<float> W = weights(4, 512, 0.02f);
  for (int k = 0; k < 16; ++k) W[k] = 0.5f;                 // a constant group
  for (int k = 16; k < 32; ++k) W[k] = 0.0f;                // a zero group
  spqr_case("spqrb", 4, 512, 0.05, W);
  std::vector<float> bad(256);
  expect("spqr_pack K % 256", spqr_pack(bad.data(), 1, 200, 0.0, nullptr, nullptr, nullptr, nullptr, nullptr,
                                        nullptr, 0, nullptr), QLIN_EINVAL);
}

void sq_cases() {
  const int M = 9, N = 6, K = 128;
  std::vector<uint16_t> X(static_cast<size_t>(M) * K);
  for (int m = 0; m < M; ++m)
    for (int k = 0; k < K; ++k) {
      const float v = k == 7 ? 0.0f : (k % 13 == 0 ? 100.0f : 1.0f) * std::round(normal(4.0f)) * 0.5f;
      X[static_cast<size_t>(m) * K + k] = f16_bits(v);
    }
  std::vector<float> amax(K), s(K), inv(K);
  expect("sq_act_absmax", sq_act_absmax(X.data(), M, K, amax.data()), QLIN_OK);
  std::vector<float> W = weights(N, K, 0.02f);
  for (int k = 0; k < K; ++k) W[static_cast<size_t>(2) * K + k] = 0.0f;   // a zero output row
  for (int n = 0; n < N; ++n) W[static_cast<size_t>(n) * K + 9] = 0.0f;   // a zero input column
  expect("sq_compute_smoothing", sq_compute_smoothing(amax.data(), W.data(), N, K, 0.85, s.data(), inv.data()),
         QLIN_OK);
  std::vector<int8_t> Wq(static_cast<size_t>(N) * K);
  std::vector<float> wsc(N);
  expect("sq_pack_weight", sq_pack_weight(W.data(), s.data(), N, K, Wq.data(), wsc.data()), QLIN_OK);
  expect("sq_compute_smoothing alpha", sq_compute_smoothing(amax.data(), W.data(), N, K, 1.5, s.data(), inv.data()),
         QLIN_EINVAL);
  put("sq_X", X);
  put("sq_W", W);
  put("sq_amax", amax);
  put("sq_s", s);
  put("sq_inv", inv);
  put("sq_Wq", Wq);
  put("sq_wscale", wsc);
}

void second_order_cases() {
  const int n = 16, K = 128;
  std::vector<float> X(static_cast<size_t>(n) * K);
  for (auto& x : X) x = normal(1.0f);
  std::vector<double> H(static_cast<size_t>(K) * K);
  expect("qlin_hessian", qlin_hessian(X.data(), n, K, H.data()), QLIN_OK);
  put("so_X", X);
  put("so_H", H);
  {
    const int N = 6, G = 64;
    std::vector<float> W = weights(N, K, 0.02f);
    size_t qb, sb, zb;
    qlin_w4_sizes(N, K, G, &qb, &sb, &zb);
    std::vector<uint32_t> qw(qb / 4), qz(zb / 4);
    std::vector<uint16_t> sc(sb / 2);
    expect("w4_pack_gptq", qlin_w4_pack_gptq(W.data(), N, K, G, H.data(), 0.01, qw.data(), sc.data(), qz.data()),
           QLIN_OK);
    put("gq_W", W);
    put("gq_qweight", qw);
    put("gq_scales", sc);
    put("gq_qzeros", qz);
    std::vector<double> Hbad = H;
    Hbad[1] += 1.0;                                          // not symmetric
    expect("w4_pack_gptq asymmetric H",
           qlin_w4_pack_gptq(W.data(), N, K, G, Hbad.data(), 0.01, qw.data(), sc.data(), qz.data()), QLIN_EINVAL);
  }
  for (int sg = 0; sg < 2; ++sg) {
    const int N = 5, G = 32;
    std::vector<float> W = weights(N, K, 0.02f);
    size_t qb, sb, zb;
    qlin_w4_sizes(N, K, G, &qb, &sb, &zb);
    std::vector<uint32_t> qw(qb / 4), qz(zb / 4);
    std::vector<uint16_t> sc(sb / 2);
    std::vector<int32_t> perm(K);
    expect("w4_pack_gptq_actorder", qlin_w4_pack_gptq_actorder(W.data(), N, K, G, H.data(), 0.01, sg, qw.data(),
                                                               sc.data(), qz.data(), perm.data()), QLIN_OK);
    const std::string t = sg ? "ao_static" : "ao_dynamic";
    put((t + "_W").c_str(), W);
    put((t + "_qweight").c_str(), qw);
    put((t + "_scales").c_str(), sc);
    put((t + "_qzeros").c_str(), qz);
    put((t + "_perm").c_str(), perm);
  }
  {
    const int N = 5, K2 = 256;
    std::vector<float> X2(static_cast<size_t>(n) * K2);
    for (auto& x : X2) x = normal(1.0f);
    std::vector<double> H2(static_cast<size_t>(K2) * K2);
    expect("qlin_hessian 256", qlin_hessian(X2.data(), n, K2, H2.data()), QLIN_OK);
    std::vector<float> W = weights(N, K2, 0.02f);
    size_t cb, s1b, s2b;
    int64_t nnz = 0;
    spqr_sizes(N, K2, 0.02, &cb, &s1b, &s2b, &nnz);
    std::vector<uint32_t> codes(cb / 4), st1(s1b / 4);
    std::vector<uint16_t> st2(s2b / 2), vals(static_cast<size_t>(nnz));
    std::vector<int32_t> rp(N + 1), ci(static_cast<size_t>(nnz));
    int64_t got = -1;
    expect("spqr_pack_hessian", spqr_pack_hessian(W.data(), N, K2, 0.02, H2.data(), 0.01, codes.data(), st1.data(),
                                                  st2.data(), rp.data(), ci.data(), vals.data(), nnz, &got),
           QLIN_OK);
    put("sh_X", X2);
    put("sh_W", W);
    put("sh_codes", codes);
    put("sh_stats1", st1);
    put("sh_stats2", st2);
    put("sh_row_ptr", rp);
    put("sh_col_idx", ci);
    put("sh_val", vals);
  }
}

}  // namespace

int main(int argc, char** argv) {
  if (argc != 2) {
    std::fprintf(stderr, "usage: %s OUTPUT_DIR\n", argv[0]);
    return 2;
  }
  g_dir = argv[1];
  w4_cases();
  spqr_cases();
  sq_cases();
  second_order_cases();
  if (g_failures) {
    std::fprintf(stderr, "%d unexpected results\n", g_failures);
    return 1;
  }
  std::printf("host encoders OK\n");
  return 0;
}
