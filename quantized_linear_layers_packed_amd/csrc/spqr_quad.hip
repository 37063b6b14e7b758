// SpQR GEMV for batches of 1 .. 8 tokens on the 4 x 4 x 4 matrix instruction
// with the CSR outliers fused, gfx950.
//
// Y[m][n] = sum_k x[m][k] * s_hat(q - z_hat)  +  sum_{(n,k,v) in CSR} x[m][k] * v
//
// The single-token GEMV (spqr_gemv.hip) spends one v_dot2 per two weights and
// token; from two tokens those products and their LDS operand reads dominate
// its instruction stream.  Here they go to v_mfma_f32_4x4x4_16b_f16, whose
// sixteen independent 4 x 4 x 4 blocks fit the GEMV's chunk layout as it is:
//   * a wave serves four rows; at each step lane 4 b + j holds chunk b of the
//     step's 16 consecutive chunks of row j (its B operand: the codes as fp16
//     1024 + 8 c, exact) and the activations of token j at the same chunk (its
//     A operand, from the LDS staging), so block b forms the 4 tokens x 4 rows
//     products of its chunk: two code pairs (4 weights) per instruction, four
//     instructions per group of 16 codes with the accumulator chained;
//   * lane 4 b + j then holds the group's sums for the four tokens of row j
//     and applies the group statistics in fp32 as the GEMV does:
//     s_hat * (acc / 8 - (128 + z_hat) * sum x), sum x from the staging;
//   * five to eight tokens run two token groups on the same codes; a single
//     token (routed here on long rows, where the GEMV's 64-chunk blocks leave
//     lanes idle) has one group-sum pair and one accumulator per chunk and
//     takes rows of up to 18432 in one K slice;
//   * the row's statistics are staged per workgroup, the row's CSR entries are
//     walked by the 16 lanes of the row in each of its waves and added into the
//     same accumulators, and the lanes' and waves' parts are summed in a fixed
//     order (no atomics).
// Rows are split over KSW = 4 waves (each a contiguous run of the K slice's
// chunks); activations are staged in K slices when M * K exceeds the LDS
// budget, as in the GEMV.  A workgroup serves one or two groups of 8 rows (two
// where a row of up to 4 tokens is one slice: one staging for 16 rows).  The
// load order matters as much as the arithmetic: the code stream is issued
// before anything waits for row_ptr (first slice peeled off the slice loop, a
// scheduling barrier after the code loads) and the CSR preloads are
// unconditional, so every wait the compiler inserts counts exactly the loads
// it needs.

#include <type_traits>

#include "common.hpp"
#include "device.hpp"
#include "launch.hpp"
#include "spqr_chunk.hpp"

namespace qlin {

namespace {

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kKsw = 4;                          // waves per row quad
constexpr int kRows = 4 * (kWaves / kKsw);       // rows per workgroup

typedef _Float16 h4_t __attribute__((ext_vector_type(4)));

// Largest K slice in statistic blocks of 256: 32 (8192 values); 72 (18432)
// for a single token, whose staging is small enough to take a 17920-wide row
// in one slice.
constexpr int max_blocks(int MT) { return MT == 1 ? 72 : 32; }

// 16 blocks of D (4 x 4) += A (4 x 4) B (4 x 4): lane 4 b + i supplies row i of
// A_b and column i of B_b (4 fp16 each, element e of both at the same k) and
// receives column i of D_b (rows 0..3).
__device__ __forceinline__ f32x4_t mfma4(uint32_t a0, uint32_t a1, uint32_t b0, uint32_t b1, f32x4_t c) {
  const h4_t A = bitcast<h4_t>(make_uint2(a0, a1));
  const h4_t B = bitcast<h4_t>(make_uint2(b0, b1));
  return __builtin_amdgcn_mfma_f32_4x4x4f16(A, B, c, 0, 0, 0);
}

// Per K slice, in this order:
//   1. the activation loads of the LDS staging (one 32-value piece per thread),
//   2. the slice's statistics of the workgroup's rows (4-byte pieces, up to
//      three and two per thread), the wave's code chunks of the first row
//      group for all its steps and, on the first slice, the first CSR entries
//      of each row,
//   3. the staging (pairs in the unpack order, the per-chunk group sums) and
//      the statistics into LDS,
//   4. after the barrier, per row group: per step unpack, statistics decode,
//      the matrix instructions and the rescale; then the next group's codes
//      are issued into the same registers, and the group's CSR entries are
//      added while they arrive.
// A workgroup serves R groups of 8 rows: one activation staging and one pass
// of barriers for all of them.
template <int MT, int S, int R, int OUTK>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(4))) void spqr_quad_kernel(
    const uint16_t* X, int M, int K, int KS,
    const uint32_t* codes, const uint32_t* stats1,
    const uint16_t* stats2, const int32_t* row_ptr,
    const int32_t* col_idx, const uint16_t* vals,
    int N, void* Y) {
  constexpr int kCsr = R == 1 ? 4 : 1;                // CSR entries per lane and row held in registers
  constexpr int NG = (MT + 3) / 4;                    // token groups of 4 (a single token fills one)
  constexpr int TG = MT < 4 ? MT : 4;                 // tokens used per group
  constexpr int ROWS = R * kRows;                     // rows of the workgroup
  constexpr int NR1 = (ROWS * max_blocks(MT) * 3 + kThreads - 1) / kThreads;   // statistic piece rounds
  constexpr int NR2 = (ROWS * max_blocks(MT) * 2 + kThreads - 1) / kThreads;
  extern __shared__ uint4 smem[];
  __shared__ float red[kWaves][R][MT][4];
  const int CS = KS >> 5;                             // chunks per slice
  const int BS = KS >> 8;                             // statistic blocks per slice
  // staged pair quads: chunk c of token m at 16-byte unit m T + 4 c + c / 4 (its
  // four quads contiguous): one spare unit after every 4 chunks and one per
  // token row (T odd), so the staging stores of 16 consecutive chunks and the
  // step's reads of 4 chunks x 4 tokens each meet 16 distinct bank groups
  const int T = 4 * CS + (CS >> 2) + 1;
  uint4* xl = smem;                                                                    // [MT][T] pair quads
  float2* xs = reinterpret_cast<float2*>(smem + static_cast<size_t>(MT) * T);          // [CS][MT] group sums
  float4* ls2f = reinterpret_cast<float4*>(xs + static_cast<size_t>(CS) * MT);          // [rows][bs] combined second level
  uint32_t* ls1 = reinterpret_cast<uint32_t*>(ls2f + static_cast<size_t>(ROWS) * BS);   // [rows][bs][3] first-level words
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int part = wv % kKsw;
  const int b = lane >> 2, j = lane & 3;              // chunk slot of the step; row of the quad and token of the group
  const int n0 = blockIdx.x * ROWS;
  const int C = K >> 5, nb = K >> 8;
  int rowl[R], n[R], p0[R], p1[R];                    // row of group r within the workgroup, its index, row_ptr of its row
  int e0[R], e1[R];                                   // its CSR range (empty past N), set on the first slice
  bool nok[R];
  const uint32_t* crow[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    rowl[r] = r * kRows + 4 * (wv / kKsw) + j;
    n[r] = n0 + rowl[r];
    nok[r] = n[r] < N;
    const int nc = min(n[r], N - 1);
    crow[r] = codes + static_cast<size_t>(nc) * C * 3;
    p0[r] = row_ptr[nc];                              // unconditional: a select here would wait for the load
    p1[r] = row_ptr[nc + 1];
    e0[r] = 0;
    e1[r] = 0;
  }
  int tok[NG];                                        // this lane's A-operand token per group (rows past M re-read M - 1)
#pragma unroll
  for (int g = 0; g < NG; ++g) tok[g] = min(4 * g + j, M - 1);

  // CSR entries of each row held by this lane: e0 + 16 (KSW i + part) + b,
  // loaded on the first slice behind the dense stream, kept as raw bits; bit
  // r kCsr + i of cvalid flags a loaded entry
  int ccol[R][kCsr];
  uint32_t cbits[R][kCsr];
  uint32_t cvalid = 0u;

  float res[R][MT];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int m = 0; m < MT; ++m) res[r][m] = 0.0f;

  // one K slice; the first is peeled off the loop (straight-line code, so the
  // row_ptr values are waited for where the CSR preload uses them, after the
  // stream is issued, not hoisted ahead of it)
  auto slice = [&](const int k0, auto first_c) {
    constexpr bool kFirst = decltype(first_c)::value;
    const int ks = min(KS, K - k0);
    const int cs = ks >> 5, bs = ks >> 8;
    const int cbase = k0 >> 5, bbase = k0 >> 8;
    const int cp = ((cs + kKsw - 1) / kKsw + 3) & ~3;  // chunks per wave of the row, a multiple of 4
    const int c0 = part * cp, c1 = min(cs, c0 + cp);

    // ---- 1. the staging pieces of this thread (items tid and tid + 512,
    //      at most 2 * 512 >= 8 * 112 and 4 * 224; the second only in waves
    //      that have one; clamped).  An item's token is floor(it / cs), taken
    //      as (it + 1/2) times the hardware reciprocal (exact for it < 2048, cs <= 1024)
    const int items = M * cs;
    const int wfirst = 64 * wv;
    const float invcs = __builtin_amdgcn_rcpf(static_cast<float>(cs));
    uint4 xv[2][4];
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      if (r == 0 || wfirst + kThreads < items) {
        const int it = min(tid + kThreads * r, items - 1);
        const int m = static_cast<int>((static_cast<float>(it) + 0.5f) * invcs), c = it - m * cs;
        const uint4* src = reinterpret_cast<const uint4*>(X + static_cast<size_t>(m) * K + k0) + 4 * c;
#pragma unroll
        for (int i = 0; i < 4; ++i) xv[r][i] = src[i];
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) xv[r][i] = make_uint4(0u, 0u, 0u, 0u);
      }
    }
    // ---- 2. statistics of the workgroup's rows in the slice (a row's blocks
    //      are contiguous: 4-byte pieces, only waves holding pieces load, rows
    //      past N read row N - 1; piece i's row is floor(i / (w bs)), w = 3 or
    //      2, taken as (i + 1/2) times the hardware reciprocal (within 1 ulp),
    //      exact for i < 2048 and w bs <= 96), then the codes
    const int it1 = ROWS * bs * 3, it2 = ROWS * bs * 2;
    const float inv1 = __builtin_amdgcn_rcpf(static_cast<float>(bs * 3));
    const float inv2 = __builtin_amdgcn_rcpf(static_cast<float>(bs * 2));
    uint32_t v1[NR1], v2[NR2];
#pragma unroll
    for (int q = 0; q < NR1; ++q) {
      if (wfirst + kThreads * q < it1) {
        const int i = min(tid + kThreads * q, it1 - 1);
        const int row = static_cast<int>((static_cast<float>(i) + 0.5f) * inv1);
        const int wi = i - row * (bs * 3);
        v1[q] = stats1[static_cast<size_t>(min(n0 + row, N - 1)) * nb * 3 + bbase * 3 + wi];
      } else {
        v1[q] = 0u;
      }
    }
#pragma unroll
    for (int q = 0; q < NR2; ++q) {
      if (wfirst + kThreads * q < it2) {
        const int i = min(tid + kThreads * q, it2 - 1);
        const int row = static_cast<int>((static_cast<float>(i) + 0.5f) * inv2);
        const int wi = i - row * (bs * 2);
        v2[q] = reinterpret_cast<const uint32_t*>(stats2)[static_cast<size_t>(min(n0 + row, N - 1)) * nb * 2 +
                                                           bbase * 2 + wi];
      } else {
        v2[q] = 0u;
      }
    }
    uint3 w[S];
#pragma unroll
    for (int s = 0; s < S; ++s) {
      const int c = min(c0 + 16 * s + b, cs - 1);
      w[s] = *reinterpret_cast<const uint3*>(crow[0] + 3 * (cbase + c));
    }
    __builtin_amdgcn_sched_barrier(0);               // the whole code stream is issued before anything below
    if constexpr (kFirst) {
      // the row_ptr values pass through an empty asm after the stream is
      // issued, so that nothing using them is scheduled ahead of it
#pragma unroll
      for (int r = 0; r < R; ++r) {
        asm volatile("" : "+v"(p0[r]), "+v"(p1[r]));
        e0[r] = nok[r] ? p0[r] : 0;
        e1[r] = nok[r] ? p1[r] : 0;
      }
#pragma unroll
      for (int r = 0; r < R; ++r)
#pragma unroll
        for (int i = 0; i < kCsr; ++i) {
          // unconditional (a conditional load here is followed by a wait for
          // it): entries past the row re-read one inside the arrays, which are
          // never empty (with no outliers the entry point passes row_ptr)
          const int e = e0[r] + 16 * (kKsw * i + part) + b;
          const int ec = max(min(e, p1[r] - 1), 0);
          ccol[r][i] = col_idx[ec];
          cbits[r][i] = vals[ec];
          cvalid |= e < e1[r] ? 1u << (r * kCsr + i) : 0u;
        }
    }
    // ---- 3. staging (after a barrier from the second slice on: the previous
    //      slice's readers must be done)
    if constexpr (!kFirst) __syncthreads();
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int it = tid + kThreads * r;
      if (it >= items) break;
      const int m = static_cast<int>((static_cast<float>(it) + 0.5f) * invcs), c = it - m * cs;
      uint32_t u[16];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        u[4 * i] = xv[r][i].x; u[4 * i + 1] = xv[r][i].y; u[4 * i + 2] = xv[r][i].z; u[4 * i + 3] = xv[r][i].w;
      }
      uint32_t P[16];
#pragma unroll
      for (int q = 0; q < 16; ++q) P[q] = half_of(u, pair_lo(q)) | (half_of(u, pair_hi(q)) << 16);
      uint4* dst = xl + static_cast<size_t>(m) * T + 4 * c + (c >> 2);
#pragma unroll
      for (int q = 0; q < 4; ++q) dst[q] = make_uint4(P[4 * q], P[4 * q + 1], P[4 * q + 2], P[4 * q + 3]);
      // group sums by dot products with (1, 1): pairs 0..7 hold group 2c, 8..15 group 2c+1
      float sa = 0.0f, sb = 0.0f;
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        sa = dot2_f16(P[q], 0x3C003C00u, sa);
        sb = dot2_f16(P[8 + q], 0x3C003C00u, sb);
      }
      xs[static_cast<size_t>(c) * MT + m] = make_float2(sa, sb);
    }
#pragma unroll
    for (int q = 0; q < NR1; ++q)
      if (tid + kThreads * q < it1) ls1[tid + kThreads * q] = v1[q];
    // second-level pairs go to LDS already combined into what a chunk's decode
    // needs, per (row, block): scale pair (SS, ZS) -> SS, -SS ZS and zero pair
    // -> -SS, SS ZS - 128, so that s_hat = SS c + (-SS ZS) and -(128 + z_hat)
    // = (-SS) c + (SS ZS - 128) are one fma each (piece i -> floats 2i, 2i + 1)
#pragma unroll
    for (int q = 0; q < NR2; ++q) {
      const int i = tid + kThreads * q;
      if (i < it2) {
        const float S2 = f16_bits_to_f32(static_cast<uint16_t>(v2[q]));
        const float Z2 = f16_bits_to_f32(static_cast<uint16_t>(v2[q] >> 16));
        reinterpret_cast<float2*>(ls2f)[i] =
            (i & 1) ? make_float2(-S2, fmaf(S2, Z2, -128.0f)) : make_float2(S2, -(S2 * Z2));
      }
    }
    __syncthreads();

    // ---- 4. per row group: the dense 3-bit part (16 chunks of 4 rows per
    //      step), the next group's codes, the group's CSR outliers
#pragma unroll
    for (int r = 0; r < R; ++r) {
#pragma unroll
      for (int s = 0; s < S; ++s) {
        if (c0 + 16 * s < c1) {                        // wave-uniform: the matrix instructions run with every lane
          const int c = c0 + 16 * s + b;
          const int cc = min(c, cs - 1);
          uint32_t pk[16];
          unpack_chunk(w[s].x, w[s].y, w[s].z, pk);
          const int blk = cc >> 3, jj = cc & 7;        // block within the slice; chunk within the block
          const uint32_t* r1 = ls1 + (rowl[r] * bs + blk) * 3;
          const float4 d = ls2f[rowl[r] * bs + blk];
          const uint32_t sw0 = r1[0], sw1 = r1[1], sw2 = r1[2];
          const int off = 12 * jj;                     // bit offset of the chunk's two 6-bit fields
          const uint32_t lo = off < 32 ? sw0 : (off < 64 ? sw1 : sw2);
          const uint32_t hi = off < 32 ? sw1 : sw2;
          const uint32_t f = static_cast<uint32_t>(((static_cast<uint64_t>(hi) << 32) | lo) >> (off & 31)) & 0xFFFu;
          // s_hat and -(128 + z_hat) of the chunk's two groups; slots past the
          // wave's run hold clamped codes: their scale is zeroed
          const bool act = c < c1;
          const float sA = act ? fmaf(d.x, static_cast<float>(f & 7u), d.y) : 0.0f;
          const float cA = fmaf(d.z, static_cast<float>((f >> 3) & 7u), d.w);
          const float sB = act ? fmaf(d.x, static_cast<float>((f >> 6) & 7u), d.y) : 0.0f;
          const float cB = fmaf(d.z, static_cast<float>((f >> 9) & 7u), d.w);
#pragma unroll
          for (int g = 0; g < NG; ++g) {
            const uint4* xa = xl + static_cast<size_t>(tok[g]) * T + 4 * cc + (cc >> 2);
            const uint4 a0 = xa[0], a1 = xa[1], a2 = xa[2], a3 = xa[3];
            const f32x4_t zero = {0.0f, 0.0f, 0.0f, 0.0f};
            f32x4_t dA = mfma4(a0.x, a0.y, pk[0], pk[1], zero);
            f32x4_t dB = mfma4(a2.x, a2.y, pk[8], pk[9], zero);
            dA = mfma4(a0.z, a0.w, pk[2], pk[3], dA);
            dB = mfma4(a2.z, a2.w, pk[10], pk[11], dB);
            dA = mfma4(a1.x, a1.y, pk[4], pk[5], dA);
            dB = mfma4(a3.x, a3.y, pk[12], pk[13], dB);
            dA = mfma4(a1.z, a1.w, pk[6], pk[7], dA);
            dB = mfma4(a3.z, a3.w, pk[14], pk[15], dB);
            // the group sums of tokens 4 g .. 4 g + 3 at this chunk: (A, B) per token
            float xA[4], xB[4];
            if constexpr (TG == 4) {
              const float4* xq = reinterpret_cast<const float4*>(xs + static_cast<size_t>(cc) * MT + 4 * g);
              const float4 s01 = xq[0], s23 = xq[1];
              xA[0] = s01.x; xA[1] = s01.z; xA[2] = s23.x; xA[3] = s23.z;
              xB[0] = s01.y; xB[1] = s01.w; xB[2] = s23.y; xB[3] = s23.w;
            } else {
              const float2 s0 = xs[static_cast<size_t>(cc) * MT];
              xA[0] = s0.x;
              xB[0] = s0.y;
            }
#pragma unroll
            for (int t = 0; t < TG; ++t) {
              // sum x (c - z_hat) = acc / 8 - (128 + z_hat) * sum(x)
              res[r][4 * g + t] = fmaf(sA, fmaf(dA[t], 0.125f, cA * xA[t]), res[r][4 * g + t]);
              res[r][4 * g + t] = fmaf(sB, fmaf(dB[t], 0.125f, cB * xB[t]), res[r][4 * g + t]);
            }
          }
        }
      }
      if (r + 1 < R) {
#pragma unroll
        for (int s = 0; s < S; ++s) {
          const int c = min(c0 + 16 * s + b, cs - 1);
          w[s] = *reinterpret_cast<const uint3*>(crow[r + 1] + 3 * (cbase + c));
        }
      }
      // CSR outliers of the lane's row of this group whose column falls in the slice
      auto outlier = [&](int colg, float v) {
        const int col = colg - k0;
        if (col < 0 || col >= ks) return;
        const int c = col >> 5, slot = pair_slot(col & 31);
        const int q = slot >> 3, wi = (slot >> 1) & 3, hh = slot & 1;
#pragma unroll
        for (int m = 0; m < MT; ++m) {
          if (m < M) {
            const uint32_t* quad = reinterpret_cast<const uint32_t*>(xl + static_cast<size_t>(m) * T + 4 * c + (c >> 2) + q);
            const uint16_t xh = static_cast<uint16_t>(quad[wi] >> (16 * hh));
            res[r][m] = fmaf(f16_bits_to_f32(xh), v, res[r][m]);
          }
        }
      };
#pragma unroll
      for (int i = 0; i < kCsr; ++i)
        if ((cvalid >> (r * kCsr + i)) & 1u) outlier(ccol[r][i], f16_bits_to_f32(static_cast<uint16_t>(cbits[r][i])));
      for (int e = e0[r] + 16 * (kKsw * kCsr + part) + b; e < e1[r]; e += 16 * kKsw)
        outlier(col_idx[e], f16_bits_to_f32(vals[e]));
    }
  };
  slice(0, std::true_type{});
  for (int k0 = KS; k0 < K; k0 += KS) slice(k0, std::false_type{});

  // ---- sum over the 16 lanes of each row (lanes j, j + 4, ..., j + 60), then
  //      over the row's waves in a fixed order through LDS (rotations by 8 and
  //      4 within each row of 16 lanes leave every lane with the sum of its
  //      row's lanes of the same j; two cross-row exchanges finish)
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      float v = res[r][m];
      v += bitcast<float>(__builtin_amdgcn_update_dpp(0, bitcast<int>(v), 0x128, 0xF, 0xF, false));   // row_ror:8
      v += bitcast<float>(__builtin_amdgcn_update_dpp(0, bitcast<int>(v), 0x124, 0xF, 0xF, false));   // row_ror:4
      v += __shfl_xor(v, 16, 64);
      v += __shfl_xor(v, 32, 64);
      if (b == 0) red[wv][r][m][j] = v;
    }
  __syncthreads();
  if (part == 0 && b == 0) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      if (nok[r]) {
#pragma unroll
        for (int m = 0; m < MT; ++m) {
          if (m < M) {
            float v = red[wv][r][m][j];
#pragma unroll
            for (int q = 1; q < kKsw; ++q) v += red[wv + q][r][m][j];
            store_out<OUTK>(Y, static_cast<size_t>(m) * N + n[r], v);
          }
        }
      }
    }
  }
}

// LDS budget per workgroup: two workgroups per CU (160 KB) with the static
// reduction array beside it.
constexpr size_t lds_budget(int R) { return R == 1 ? 72 * 1024 : 77 * 1024; }

template <int MT, int S, int R>
void launch_k(const SpqrArgs& a, int KS, hipStream_t stream) {
  constexpr int ROWS = R * kRows;
  const int CS = KS / 32, BS = KS / 256;
  const size_t lds = static_cast<size_t>(MT) * (4 * CS + CS / 4 + 1) * 16 + static_cast<size_t>(CS) * MT * 8 +
                     static_cast<size_t>(ROWS) * BS * 28;
  const int grid = (a.N + ROWS - 1) / ROWS;
  // more than 64 KB of dynamic LDS must be allowed per kernel (once per process,
  // thread-safe initialisation of function-local statics)
  static const bool lds_f32 = (hipFuncSetAttribute(reinterpret_cast<const void*>(spqr_quad_kernel<MT, S, R, OUT_F32>),
                                                   hipFuncAttributeMaxDynamicSharedMemorySize,
                                                   static_cast<int>(lds_budget(R) + 1024)) == hipSuccess);
  static const bool lds_f16 = (hipFuncSetAttribute(reinterpret_cast<const void*>(spqr_quad_kernel<MT, S, R, OUT_F16>),
                                                   hipFuncAttributeMaxDynamicSharedMemorySize,
                                                   static_cast<int>(lds_budget(R) + 1024)) == hipSuccess);
  (void)lds_f32;
  (void)lds_f16;
  if (a.y_dtype == QLIN_F32)
    hipLaunchKernelGGL((spqr_quad_kernel<MT, S, R, OUT_F32>), dim3(grid), dim3(kThreads), lds, stream,
                       a.X, a.M, a.K, KS, a.codes, a.stats1, a.stats2, a.row_ptr, a.col_idx, a.vals, a.N, a.Y);
  else
    hipLaunchKernelGGL((spqr_quad_kernel<MT, S, R, OUT_F16>), dim3(grid), dim3(kThreads), lds, stream,
                       a.X, a.M, a.K, KS, a.codes, a.stats1, a.stats2, a.row_ptr, a.col_idx, a.vals, a.N, a.Y);
}

// K slice (multiple of 256): staged activations (2.375 bytes per value and
// token with the bank skew, plus 16 per token) and the rows' statistics (28
// bytes per 256 values and row) within the LDS budget, at most max_blocks
// statistic blocks (which sizes the statistic piece rounds), in slices of
// equal size.
template <int MT, int R>
int slice_k(int K) {
  const double per_k = 2.375 * MT + 28.0 * R * kRows / 256.0;
  int KS = static_cast<int>(static_cast<double>(lds_budget(R) - 16 * MT) / per_k);
  if (KS > 256 * max_blocks(MT)) KS = 256 * max_blocks(MT);
  KS = KS / 256 * 256;
  if (KS < 256) KS = 256;
  if (KS > K) KS = K;
  const int nslices = (K + KS - 1) / KS;
  return (K / 256 + nslices - 1) / nslices * 256;
}

template <int MT, int R>
void launch_r(const SpqrArgs& a, hipStream_t stream) {
  const int KS = slice_k<MT, R>(a.K);
  // steps of 16 chunks per wave: the wave's run of ceil(cs / 4) chunks rounded
  // up to a multiple of 4, as in the kernel
  const int cs = KS / 32;
  const int steps = ((((cs + kKsw - 1) / kKsw + 3) & ~3) + 15) / 16;
  if (steps <= 1) launch_k<MT, 1, R>(a, KS, stream);
  else if (steps == 2) launch_k<MT, 2, R>(a, KS, stream);
  else if (steps == 3) launch_k<MT, 3, R>(a, KS, stream);
  else if (steps == 4 || MT > 1) launch_k<MT, 4, R>(a, KS, stream);
  else if constexpr (MT == 1) {
    if (steps <= 6) launch_k<MT, 6, R>(a, KS, stream);
    else launch_k<MT, 9, R>(a, KS, stream);
  }
}

// Two row groups per workgroup where a row is one K slice (up to 4 tokens):
// 33B-shaped layers at M = 4, one group vs two (us): 6656 x 6656 16.7-17.2
// vs 14.9, 17920 x 6656 35.2 vs 34.8; with three slices (6656 x 17920) the
// second group gained nothing at M = 2..4 and lost 1 us at M = 1.  Five to
// eight tokens, and single tokens (whose rows of up to 18432 take 9 steps),
// keep one group: two would spill registers.
template <int MT>
void launch_m(const SpqrArgs& a, hipStream_t stream) {
  if constexpr (MT == 4) {
    if (slice_k<MT, 2>(a.K) == a.K) {
      launch_r<MT, 2>(a, stream);
      return;
    }
  }
  launch_r<MT, 1>(a, stream);
}

}  // namespace

void spqr_quad_launch(const SpqrArgs& a, hipStream_t stream) {
  if (a.M == 1) launch_m<1>(a, stream);
  else if (a.M <= 4) launch_m<4>(a, stream);
  else launch_m<8>(a, stream);
}

}  // namespace qlin
