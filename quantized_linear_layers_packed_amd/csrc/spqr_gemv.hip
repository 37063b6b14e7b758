// SpQR GEMV / skinny GEMM (M <= 16) with the CSR outliers fused, gfx950.
//
// Y[m][n] = sum_k x[m][k] * s_hat(q - z_hat)  +  sum_{(n,k,v) in CSR} x[m][k] * v
//
// The SpQR bulletin ("İddia ve Gerçeklik") describes inference as decompressing
// the dense 3-bit weights while the sparse fp16 product runs beside it, and
// warns that mixing the irregular sparse part with dense blocks costs register
// pressure and divergence.  Here both parts feed ONE fp32 accumulator per
// (row, batch entry) in the same pass:
//   * 16 lanes share an output row (4 rows per wavefront); lane j of a row reads
//     the 32-code chunks j, j+16, ... (three 32-bit words each);
//   * the chunk layout places two codes of the same group in field i of the low
//     and high 16-bit halves of a word, so one shift + and-or yields an fp16 pair
//     1024 + 8c exactly, ready for v_dot2 against activation pairs staged in LDS
//     in the matching order;
//   * the two first-level statistics of the chunk's groups are decoded from
//     their 3-bit codes and the block's fp16 second-level values
//     (s_hat = SS_s (c_s - ZS_s), z_hat = SS_z (c_z - ZS_z)) in fp32;
//   * then the same 16 lanes walk the row's CSR segment (entry e goes to lane
//     e mod 16), gather x from LDS and add x * v into the same accumulators,
//     before the one 16-lane reduction that produces Y.  No second pass, no
//     atomics.
// Activations are staged in K-slices when M*K does not fit the LDS budget.

#include "common.hpp"
#include "device.hpp"
#include "launch.hpp"

namespace qlin {

namespace {

constexpr int kThreads = 256;
constexpr int kLPR = 16;                 // lanes per output row
constexpr int kRowsPerWG = kThreads / kLPR;
constexpr size_t kLdsBudget = 48 * 1024;

// fp16 pair (1024 + 8 c_lo, 1024 + 8 c_hi) from field i of both halves of w.
__device__ __forceinline__ uint32_t field_pair(uint32_t w, int i) {
  constexpr uint32_t MASK = 0x00380038u, MAGIC = 0x64006400u;
  switch (i) {
    case 0: return ((w << 3) & MASK) | MAGIC;
    case 1: return (w & MASK) | MAGIC;
    case 2: return ((w >> 3) & MASK) | MAGIC;
    case 3: return ((w >> 6) & MASK) | MAGIC;
    default: return ((w >> 9) & MASK) | MAGIC;
  }
}

// The sixteen pairs of a chunk, pairs 0..7 from group 2c, 8..15 from group 2c+1.
__device__ __forceinline__ void unpack_chunk(uint32_t w0, uint32_t w1, uint32_t w2, uint32_t p[16]) {
#pragma unroll
  for (int i = 0; i < 5; ++i) {
    p[i] = field_pair(w0, i);
    p[5 + i] = field_pair(w1, i);
    p[10 + i] = field_pair(w2, i);
  }
  p[15] = ((w0 >> 12) & 0x00080008u) | ((w1 >> 11) & 0x00100010u) | ((w2 >> 10) & 0x00200020u) | 0x64006400u;
}

// Within-chunk offsets (k % 32) of the two codes of pair p.
__host__ __device__ constexpr int pair_lo(int p) {
  return p < 5 ? p : p < 8 ? p + 5 : p == 8 ? 16 : p == 9 ? 17 : p < 15 ? p + 10 : 30;
}
__host__ __device__ constexpr int pair_hi(int p) {
  return p < 5 ? p + 5 : p < 8 ? p + 8 : p == 8 ? 18 : p == 9 ? 19 : p < 15 ? p + 15 : 31;
}

// Inverse: (pair << 1 | half) of within-chunk offset o.
__device__ __forceinline__ int pair_slot(int o) {
  if (o < 16) {
    if (o < 5) return o << 1;
    if (o < 10) return ((o - 5) << 1) | 1;
    if (o < 13) return (o - 5) << 1;
    return ((o - 8) << 1) | 1;
  }
  const int b = o - 16;
  if (b < 2) return (8 + b) << 1;
  if (b < 4) return ((6 + b) << 1) | 1;
  if (b < 9) return (6 + b) << 1;
  if (b < 14) return ((1 + b) << 1) | 1;
  return (15 << 1) | (b - 14);
}

__device__ __forceinline__ uint32_t half_of(const uint32_t u[16], int o) {
  return (u[o >> 1] >> (16 * (o & 1))) & 0xFFFFu;
}

template <int MT, int OUTK>
__global__ __launch_bounds__(kThreads) void spqr_gemv_kernel(
    const uint16_t* __restrict__ X, int M, int K, int KS,
    const uint32_t* __restrict__ codes, const uint32_t* __restrict__ stats1,
    const uint16_t* __restrict__ stats2, const int32_t* __restrict__ row_ptr,
    const int32_t* __restrict__ col_idx, const uint16_t* __restrict__ vals,
    int N, void* __restrict__ Y) {
  extern __shared__ uint4 smem[];
  const int CS = KS >> 5;                             // chunks per slice
  uint4* xl = smem;                                   // [MT][4][CS] pair quads
  float* xs = reinterpret_cast<float*>(smem + static_cast<size_t>(MT) * 4 * CS);   // [MT][2*CS]

  const int lane = threadIdx.x & 63;
  const int sub = lane & (kLPR - 1);
  const int n = blockIdx.x * kRowsPerWG + (threadIdx.x >> 4);
  const bool row_ok = n < N;
  const int nb = K >> 8;
  const size_t nrow = static_cast<size_t>(row_ok ? n : 0);
  const uint32_t* crow = codes + nrow * (K >> 5) * 3;
  const uint32_t* s1row = stats1 + nrow * nb * 3;
  const uint2* s2row = reinterpret_cast<const uint2*>(stats2) + nrow * nb;
  const int e0 = row_ok ? row_ptr[n] : 0;
  const int e1 = row_ok ? row_ptr[n + 1] : 0;

  float res[MT];
#pragma unroll
  for (int m = 0; m < MT; ++m) res[m] = 0.0f;

  for (int k0 = 0; k0 < K; k0 += KS) {
    const int ks = min(KS, K - k0);
    const int cs = ks >> 5;
    // ---- stage the activation slice as pairs + per-group sums
    __syncthreads();
    for (int it = threadIdx.x; it < M * cs; it += kThreads) {
      const int m = it / cs, c = it - m * cs;
      const uint4* src = reinterpret_cast<const uint4*>(X + static_cast<size_t>(m) * K + k0) + 4 * c;
      uint32_t u[16];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint4 v = src[i];
        u[4 * i] = v.x; u[4 * i + 1] = v.y; u[4 * i + 2] = v.z; u[4 * i + 3] = v.w;
      }
      uint32_t P[16];
#pragma unroll
      for (int p = 0; p < 16; ++p) P[p] = half_of(u, pair_lo(p)) | (half_of(u, pair_hi(p)) << 16);
#pragma unroll
      for (int q = 0; q < 4; ++q)
        xl[(static_cast<size_t>(m) * 4 + q) * CS + c] = make_uint4(P[4 * q], P[4 * q + 1], P[4 * q + 2], P[4 * q + 3]);
      float sa = 0.0f, sb = 0.0f;
#pragma unroll
      for (int o = 0; o < 16; ++o) {
        sa += f16_bits_to_f32(static_cast<uint16_t>(half_of(u, o)));
        sb += f16_bits_to_f32(static_cast<uint16_t>(half_of(u, 16 + o)));
      }
      xs[m * 2 * CS + 2 * c] = sa;
      xs[m * 2 * CS + 2 * c + 1] = sb;
    }
    __syncthreads();
    if (!row_ok) continue;

    // ---- dense 3-bit part over this slice
    const int cbase = k0 >> 5;
    for (int c = sub; c < cs; c += kLPR) {
      const int cg = cbase + c;                       // global chunk index
      const uint32_t* cw = crow + 3 * cg;
      const uint32_t w0 = __builtin_nontemporal_load(cw);
      const uint32_t w1 = __builtin_nontemporal_load(cw + 1);
      const uint32_t w2 = __builtin_nontemporal_load(cw + 2);
      const int b = cg >> 3, j = cg & 7;
      const uint32_t* sw = s1row + 3 * b;
      const uint64_t lo64 = static_cast<uint64_t>(sw[0]) | (static_cast<uint64_t>(sw[1]) << 32);
      const uint64_t hi64 = static_cast<uint64_t>(sw[1]) | (static_cast<uint64_t>(sw[2]) << 32);
      const int off = 12 * j;
      const uint32_t f = static_cast<uint32_t>((off <= 52 ? (lo64 >> off) : (hi64 >> (off - 32))) & 0xFFFu);
      const uint2 s2 = s2row[b];
      const float SSs = f16_bits_to_f32(static_cast<uint16_t>(s2.x));
      const float ZSs = f16_bits_to_f32(static_cast<uint16_t>(s2.x >> 16));
      const float SSz = f16_bits_to_f32(static_cast<uint16_t>(s2.y));
      const float ZSz = f16_bits_to_f32(static_cast<uint16_t>(s2.y >> 16));
      const float sA = SSs * (static_cast<float>(f & 7u) - ZSs);
      const float zA = SSz * (static_cast<float>((f >> 3) & 7u) - ZSz);
      const float sB = SSs * (static_cast<float>((f >> 6) & 7u) - ZSs);
      const float zB = SSz * (static_cast<float>((f >> 9) & 7u) - ZSz);

      uint32_t p[16];
      unpack_chunk(w0, w1, w2, p);
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        if (m < M) {
          float aA = 0.0f, aB = 0.0f;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const uint4 xp = xl[(static_cast<size_t>(m) * 4 + q) * CS + c];
            if (q < 2) {
              aA = dot2_f16(p[4 * q], xp.x, aA);
              aA = dot2_f16(p[4 * q + 1], xp.y, aA);
              aA = dot2_f16(p[4 * q + 2], xp.z, aA);
              aA = dot2_f16(p[4 * q + 3], xp.w, aA);
            } else {
              aB = dot2_f16(p[4 * q], xp.x, aB);
              aB = dot2_f16(p[4 * q + 1], xp.y, aB);
              aB = dot2_f16(p[4 * q + 2], xp.z, aB);
              aB = dot2_f16(p[4 * q + 3], xp.w, aB);
            }
          }
          // sum x (c - z_hat) = acc / 8 - (128 + z_hat) * sum(x)
          const float xa = xs[m * 2 * CS + 2 * c], xb = xs[m * 2 * CS + 2 * c + 1];
          const float tA = fmaf(aA, 0.125f, -(128.0f + zA) * xa);
          const float tB = fmaf(aB, 0.125f, -(128.0f + zB) * xb);
          res[m] = fmaf(sA, tA, res[m]);
          res[m] = fmaf(sB, tB, res[m]);
        }
      }
    }

    // ---- CSR outliers of this row whose column falls in the slice
    for (int e = e0 + sub; e < e1; e += kLPR) {
      const int col = col_idx[e] - k0;
      if (col < 0 || col >= ks) continue;
      const float v = f16_bits_to_f32(vals[e]);
      const int c = col >> 5, slot = pair_slot(col & 31);
      const int q = slot >> 3, wi = (slot >> 1) & 3, hh = slot & 1;
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        if (m < M) {
          const uint32_t* quad = reinterpret_cast<const uint32_t*>(xl + (static_cast<size_t>(m) * 4 + q) * CS + c);
          const uint16_t xh = static_cast<uint16_t>(quad[wi] >> (16 * hh));
          res[m] = fmaf(f16_bits_to_f32(xh), v, res[m]);
        }
      }
    }
  }

  // ---- 16-lane reduction and store
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    float r = res[m];
    r += __shfl_xor(r, 8, 64);
    r += __shfl_xor(r, 4, 64);
    r += __shfl_xor(r, 2, 64);
    r += __shfl_xor(r, 1, 64);
    if (m < M && row_ok && sub == 0) store_out<OUTK>(Y, static_cast<size_t>(m) * N + n, r);
  }
}

template <int MT>
void launch_m(const SpqrArgs& a, hipStream_t stream) {
  // slice length: a multiple of 512 whose activation pairs + sums fit the budget
  // bytes per k: MT * 2 (fp16 pairs) + MT * 4 / 16 (one fp32 sum per group of 16)
  int KS = static_cast<int>(kLdsBudget * 4 / (static_cast<size_t>(MT) * 9)) / 512 * 512;
  if (KS < 512) KS = 512;
  if (KS > a.K) KS = a.K;
  const int CS = KS / 32;
  const size_t lds = static_cast<size_t>(MT) * 4 * CS * 16 + static_cast<size_t>(MT) * 2 * CS * 4;
  const int grid = (a.N + kRowsPerWG - 1) / kRowsPerWG;
  if (a.y_dtype == QLIN_F32)
    hipLaunchKernelGGL((spqr_gemv_kernel<MT, OUT_F32>), dim3(grid), dim3(kThreads), lds, stream,
                       a.X, a.M, a.K, KS, a.codes, a.stats1, a.stats2, a.row_ptr, a.col_idx, a.vals, a.N, a.Y);
  else
    hipLaunchKernelGGL((spqr_gemv_kernel<MT, OUT_F16>), dim3(grid), dim3(kThreads), lds, stream,
                       a.X, a.M, a.K, KS, a.codes, a.stats1, a.stats2, a.row_ptr, a.col_idx, a.vals, a.N, a.Y);
}

// Debug: dense codes and first-level statistic codes via the forward's routines.
__global__ void spqr_unpack_kernel(const uint32_t* __restrict__ codes, const uint32_t* __restrict__ stats1,
                                   int N, int K, uint8_t* __restrict__ q, uint8_t* __restrict__ cs,
                                   uint8_t* __restrict__ cz) {
  const size_t chunks = static_cast<size_t>(N) * (K >> 5);
  for (size_t i = blockIdx.x * static_cast<size_t>(blockDim.x) + threadIdx.x; i < chunks;
       i += static_cast<size_t>(gridDim.x) * blockDim.x) {
    uint32_t p[16];
    unpack_chunk(codes[3 * i], codes[3 * i + 1], codes[3 * i + 2], p);
    uint8_t* dst = q + 32 * i;
#pragma unroll
    for (int pp = 0; pp < 16; ++pp) {
      dst[pair_lo(pp)] = static_cast<uint8_t>((p[pp] >> 3) & 7u);
      dst[pair_hi(pp)] = static_cast<uint8_t>((p[pp] >> 19) & 7u);
    }
    // the two groups of this chunk: same field extraction as the forward kernel
    const size_t nrow = i / (K >> 5);
    const int cg = static_cast<int>(i - nrow * (K >> 5));
    const int b = cg >> 3, j = cg & 7;
    const uint32_t* sw = stats1 + (nrow * (K >> 8) + b) * 3;
    const uint64_t lo64 = static_cast<uint64_t>(sw[0]) | (static_cast<uint64_t>(sw[1]) << 32);
    const uint64_t hi64 = static_cast<uint64_t>(sw[1]) | (static_cast<uint64_t>(sw[2]) << 32);
    const int off = 12 * j;
    const uint32_t f = static_cast<uint32_t>((off <= 52 ? (lo64 >> off) : (hi64 >> (off - 32))) & 0xFFFu);
    cs[2 * i] = static_cast<uint8_t>(f & 7u);
    cz[2 * i] = static_cast<uint8_t>((f >> 3) & 7u);
    cs[2 * i + 1] = static_cast<uint8_t>((f >> 6) & 7u);
    cz[2 * i + 1] = static_cast<uint8_t>((f >> 9) & 7u);
  }
}

}  // namespace

void spqr_gemv_launch(const SpqrArgs& a, hipStream_t stream) {
  if (a.M <= 1) launch_m<1>(a, stream);
  else if (a.M <= 2) launch_m<2>(a, stream);
  else if (a.M <= 4) launch_m<4>(a, stream);
  else if (a.M <= 8) launch_m<8>(a, stream);
  else launch_m<16>(a, stream);
}

void spqr_unpack_launch(const uint32_t* codes, const uint32_t* stats1, int N, int K,
                        uint8_t* q, uint8_t* cs, uint8_t* cz, hipStream_t stream) {
  hipLaunchKernelGGL(spqr_unpack_kernel, dim3(1024), dim3(256), 0, stream, codes, stats1, N, K, q, cs, cz);
}

}  // namespace qlin
