// Plain C++17 oracle forwards of the packed quantized linear layer
//   Y[m][n] = sum_k X[m][k] * W_hat[n][k]
// for the three weight encodings.
//
// TEST INFRASTRUCTURE ONLY: the test-suite, the package smoke check and the
// benchmark's CPU-baseline leg load this; the library never does, and this
// file shares no code, header or table with it (it is compiled on its own by
// the host C++ compiler, never by the GPU toolchain).
//
// It is slow on purpose: one output row n at a time (OpenMP splits the rows),
// the row's weights decoded to fp64 from the stored bits, then plain fp64 dot
// products in index order.  No blocking, no vector intrinsics.
//
// Sources (three "Makale Bülteni" newsletter pages):
//   GPTQ bulletin, lead and "İddia ve Gerçeklik": 4-bit weights quantized in
//     groups (of 128) along the input dimension; weight-only, activations stay
//     16-bit.  Storage: codes 8 per uint32 (code k in bits 4(k%8) of word
//     k/8), fp16 scale S and 4-bit zero z per group (zero of group g in bits
//     4(g%8) of word g/8 of the row's zero words); w_hat = S (q - z).
//   SpQR bulletin, "İddia ve Gerçeklik": a dense 3-bit part in groups of 16
//     with statistics that are themselves quantized (per 16 groups), plus a
//     sparse fp16 matrix of about 1% outliers; both are applied to the same
//     output.  Decoding: s_hat = SS_s (c_s - ZS_s), z_hat = SS_z (c_z - ZS_z),
//     w_hat = s_hat (q - z_hat) + (the CSR value at (n, k), if any).
//   SmoothQuant bulletin, "İddia ve Gerçeklik" and its equation
//     Y = (X diag(s)^-1)(diag(s) W): per-token int8 activations with scale
//     dX_m, per-channel int8 weights with scale dW_n, integer accumulation:
//     acc = sum_k Xq Wq (exact, int64 here), Y = dX_m dW_n acc in fp64.
//
// The byte layouts are this library's readings where the pages are silent;
// they are written out again below from their definitions.

#include <omp.h>

#include <cmath>
#include <cstdint>
#include <cstring>
#include <vector>

namespace {

// IEEE binary16 bits -> double (exact).
double half_to_double(uint16_t h) {
  const int sign = (h >> 15) & 1;
  const int e = (h >> 10) & 0x1F;
  const int m = h & 0x3FF;
  double v;
  if (e == 0) {
    v = std::ldexp(static_cast<double>(m), -24);                 // zero or subnormal
  } else if (e == 31) {
    v = m == 0 ? INFINITY : NAN;
  } else {
    v = std::ldexp(static_cast<double>(1024 + m), e - 25);       // (1 + m/1024) 2^(e-15)
  }
  return sign ? -v : v;
}

// bfloat16 bits -> double (exact): the top half of a binary32.
double bf16_to_double(uint16_t b) {
  const uint32_t u = static_cast<uint32_t>(b) << 16;
  float f;
  std::memcpy(&f, &u, 4);
  return static_cast<double>(f);
}

// Activations as fp64, [M][K].
std::vector<double> decode_x(const uint16_t* X, int is_bf16, int M, int K) {
  std::vector<double> x(static_cast<size_t>(M) * K);
  for (size_t i = 0; i < x.size(); ++i) x[i] = is_bf16 ? bf16_to_double(X[i]) : half_to_double(X[i]);
  return x;
}

void set_threads(int threads) {
  if (threads > 0) omp_set_num_threads(threads);
}

// ---------------------------------------------------------------------------
// SpQR chunk layout: bit b of code c (0..31) of a 32-code chunk lives at
// bit chunk_bit[c][b] of the chunk's 96-bit little-endian stream (word =
// bit / 32).  Codes 0..15 are group 2i (a0..a15), 16..31 group 2i+1 (b0..b15).
// Each word is two 16-bit halves with five 3-bit fields (field f of half h at
// bit 16h + 3f):
//   word 0: a0..a4 | a5..a9
//   word 1: a10 a11 a12 b0 b1 | a13 a14 a15 b2 b3
//   word 2: b4..b8 | b9..b13
// and b14 / b15 keep bit j at bit 15 / bit 31 of word j.
struct ChunkLayout {
  int bit[32][3];
  ChunkLayout() {
    auto field = [&](int code, int word, int half, int f) {
      for (int b = 0; b < 3; ++b) bit[code][b] = 32 * word + 16 * half + 3 * f + b;
    };
    for (int f = 0; f < 5; ++f) {
      field(f, 0, 0, f);            // a0..a4
      field(5 + f, 0, 1, f);        // a5..a9
      field(20 + f, 2, 0, f);       // b4..b8
      field(25 + f, 2, 1, f);       // b9..b13
    }
    for (int f = 0; f < 3; ++f) {
      field(10 + f, 1, 0, f);       // a10..a12
      field(13 + f, 1, 1, f);       // a13..a15
    }
    for (int f = 0; f < 2; ++f) {
      field(16 + f, 1, 0, 3 + f);   // b0 b1
      field(18 + f, 1, 1, 3 + f);   // b2 b3
    }
    for (int j = 0; j < 3; ++j) {
      bit[30][j] = 32 * j + 15;     // b14
      bit[31][j] = 32 * j + 31;     // b15
    }
  }
};

const ChunkLayout& chunk_layout() {
  static const ChunkLayout L;
  return L;
}

}  // namespace

extern "C" {

int oracle_max_threads(void) { return omp_get_max_threads(); }

// W4 forward: Y [M][N] fp64.  X [M][K] fp16 (or bf16 when x_is_bf16) bits.
void oracle_w4_forward(const uint16_t* X, int x_is_bf16, int M, int K, const uint32_t* qweight,
                       const uint16_t* scales, const uint32_t* qzeros, int N, int G, double* Y, int threads) {
  set_threads(threads);
  const std::vector<double> x = decode_x(X, x_is_bf16, M, K);
  const int ng = K / G;
  const int nzw = (ng + 7) / 8;
#pragma omp parallel
  {
    std::vector<double> w(K);
#pragma omp for schedule(static)
    for (int n = 0; n < N; ++n) {
      // decode row n: w_hat[k] = S[g] (q[k] - z[g]), exact in fp64
      for (int k = 0; k < K; ++k) {
        const int g = k / G;
        const uint32_t q = (qweight[static_cast<size_t>(n) * (K / 8) + k / 8] >> (4 * (k % 8))) & 15u;
        const uint32_t z = (qzeros[static_cast<size_t>(n) * nzw + g / 8] >> (4 * (g % 8))) & 15u;
        const double S = half_to_double(scales[static_cast<size_t>(n) * ng + g]);
        w[k] = S * (static_cast<double>(q) - static_cast<double>(z));
      }
      for (int m = 0; m < M; ++m) {
        const double* xm = x.data() + static_cast<size_t>(m) * K;
        double acc = 0.0;
        for (int k = 0; k < K; ++k) acc += xm[k] * w[k];
        Y[static_cast<size_t>(m) * N + n] = acc;
      }
    }
  }
}

// SpQR forward: Y [M][N] fp64 = X . W_dense^T + X . W_sparse^T.  X fp16 [M][K].
void oracle_spqr_forward(const uint16_t* X, int M, int K, const uint32_t* codes, const uint32_t* stats1,
                         const uint16_t* stats2, const int32_t* row_ptr, const int32_t* col_idx,
                         const uint16_t* vals, int N, double* Y, int threads) {
  set_threads(threads);
  const std::vector<double> x = decode_x(X, 0, M, K);
  const ChunkLayout& L = chunk_layout();
  const int nchunk = K / 32;        // 32 codes per 3 words
  const int nblock = K / 256;       // 16 groups of 16 per statistics block
#pragma omp parallel
  {
    std::vector<double> w(K);
#pragma omp for schedule(static)
    for (int n = 0; n < N; ++n) {
      const uint32_t* crow = codes + static_cast<size_t>(n) * nchunk * 3;
      const uint32_t* s1row = stats1 + static_cast<size_t>(n) * nblock * 3;
      const uint16_t* s2row = stats2 + static_cast<size_t>(n) * nblock * 4;
      for (int k = 0; k < K; ++k) {
        // 3-bit code of k
        const uint32_t* cw = crow + 3 * (k / 32);
        uint32_t q = 0;
        for (int b = 0; b < 3; ++b) {
          const int pos = L.bit[k % 32][b];
          q |= ((cw[pos / 32] >> (pos % 32)) & 1u) << b;
        }
        // statistic codes of group g = k / 16: 6-bit field (g % 16) of its block,
        // at bit 6 (g % 16) of the block's 96-bit stream, c_s = low 3 bits, c_z = high 3
        const int blk = k / 256, gi = (k / 16) % 16;
        const uint32_t* sw = s1row + 3 * blk;
        uint32_t f = 0;
        for (int b = 0; b < 6; ++b) {
          const int pos = 6 * gi + b;
          f |= ((sw[pos / 32] >> (pos % 32)) & 1u) << b;
        }
        const double cs = static_cast<double>(f & 7u), cz = static_cast<double>(f >> 3);
        const uint16_t* st = s2row + 4 * blk;    // SS_s, ZS_s, SS_z, ZS_z
        const double s_hat = half_to_double(st[0]) * (cs - half_to_double(st[1]));
        const double z_hat = half_to_double(st[2]) * (cz - half_to_double(st[3]));
        w[k] = s_hat * (static_cast<double>(q) - z_hat);
      }
      // outliers of row n: added to the dense weight at their columns
      for (int j = row_ptr[n]; j < row_ptr[n + 1]; ++j) w[col_idx[j]] += half_to_double(vals[j]);
      for (int m = 0; m < M; ++m) {
        const double* xm = x.data() + static_cast<size_t>(m) * K;
        double acc = 0.0;
        for (int k = 0; k < K; ++k) acc += xm[k] * w[k];
        Y[static_cast<size_t>(m) * N + n] = acc;
      }
    }
  }
}

// W8A8 integer product and rescale: acc [M][N] (int64, exact) and, if Y is not
// NULL, Y [M][N] = (dX_m * dW_n) * acc in fp64.
void oracle_sq_forward(const int8_t* Xq, const float* x_scale, const int8_t* Wq, const float* w_scale, int M,
                       int N, int K, int64_t* acc, double* Y, int threads) {
  set_threads(threads);
#pragma omp parallel for schedule(static)
  for (int n = 0; n < N; ++n) {
    const int8_t* wn = Wq + static_cast<size_t>(n) * K;
    for (int m = 0; m < M; ++m) {
      const int8_t* xm = Xq + static_cast<size_t>(m) * K;
      int64_t s = 0;
      for (int k = 0; k < K; ++k) s += static_cast<int64_t>(xm[k]) * static_cast<int64_t>(wn[k]);
      acc[static_cast<size_t>(m) * N + n] = s;
      if (Y)
        Y[static_cast<size_t>(m) * N + n] =
            static_cast<double>(x_scale[m]) * static_cast<double>(w_scale[n]) * static_cast<double>(s);
    }
  }
}

}  // extern "C"
