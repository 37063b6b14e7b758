// W4 fused unpack-dequant GEMV for small batches (M <= 16), gfx950.
//
// Y[m][n] = sum_g S[n][g] * sum_{k in g} x[m][k] * (q[n][k] - z[n][g])
//
// Weight-only 4-bit inference at small batch is bound by memory bandwidth
// (GPTQ bulletin, "İddia ve Gerçeklik"), so this kernel streams the packed words
// exactly once with 128-bit loads and keeps the per-code work at a few VALU
// operations:
//   * the activations of the whole batch are staged once per workgroup in LDS,
//     already arranged as the (x_j, x_{j+4}) pairs the code unpack produces,
//     together with two per-chunk sums (a chunk = 32 codes = one uint4);
//   * each wavefront owns whole output rows (or, for long rows, one of KS
//     contiguous K parts of a row); its lanes stride over the row's chunks
//     (64 lanes x 16 B contiguous per load instruction), and the whole part is
//     loaded before any arithmetic;
//   * codes become exact 16-bit floats by and-or into the mantissa of 1024:
//     the low nibble of a byte gives 1024 + q, the high nibble 1024 + 16 q
//     without a shift (the activations paired with those registers are staged
//     pre-divided by 16), and v_dot2 accumulates against the pairs in fp32;
//     the magic offsets and the group's zero point then fold into one fused
//     multiply-add with the chunk's sums;
//   * the per-group fp16 scale multiplies that chunk result in fp32; a DPP
//     row reduction (and, for split rows, a fixed-order sum of the parts in
//     LDS) finishes the row.

#include "common.hpp"
#include "device.hpp"
#include "launch.hpp"

namespace qlin {

namespace {

constexpr int kWaves = 8;                 // waves (= output rows) per workgroup
constexpr int kThreads = 64 * kWaves;

// Value of lane `src` of v (ds_bpermute through the LDS crossbar).
__device__ __forceinline__ uint32_t lane_value(uint32_t v, int src) {
  return static_cast<uint32_t>(__builtin_amdgcn_ds_bpermute(src << 2, static_cast<int>(v)));
}

// Sum over each group of LPR lanes (16, 32 or 64) with DPP: the group's total
// ends up in its last lane.
template <int LPR>
__device__ __forceinline__ float group_sum(float v) {
  auto dpp = [](float x, int ctrl, int row_mask) -> float {
    switch (ctrl) {   // the control must be a constant expression
      case 0xB1: return bitcast<float>(__builtin_amdgcn_update_dpp(0, bitcast<int>(x), 0xB1, 0xF, 0xF, true));
      case 0x4E: return bitcast<float>(__builtin_amdgcn_update_dpp(0, bitcast<int>(x), 0x4E, 0xF, 0xF, true));
      case 0x141: return bitcast<float>(__builtin_amdgcn_update_dpp(0, bitcast<int>(x), 0x141, 0xF, 0xF, true));
      case 0x140: return bitcast<float>(__builtin_amdgcn_update_dpp(0, bitcast<int>(x), 0x140, 0xF, 0xF, true));
      case 0x142: return bitcast<float>(__builtin_amdgcn_update_dpp(0, bitcast<int>(x), 0x142, 0xA, 0xF, false));
      default: return bitcast<float>(__builtin_amdgcn_update_dpp(0, bitcast<int>(x), 0x143, 0xC, 0xF, false));
    }
    (void)row_mask;
  };
  v += dpp(v, 0xB1, 0xF);      // quad_perm [1,0,3,2]: pairs
  v += dpp(v, 0x4E, 0xF);      // quad_perm [2,3,0,1]: quads
  v += dpp(v, 0x141, 0xF);     // row_half_mirror: groups of 8
  v += dpp(v, 0x140, 0xF);     // row_mirror: rows of 16 (every lane of the row)
  if constexpr (LPR >= 32) v += dpp(v, 0x142, 0xA);   // row_bcast:15 into rows 1 and 3
  if constexpr (LPR >= 64) v += dpp(v, 0x143, 0xC);   // row_bcast:31 into rows 2 and 3
  return v;
}

// A wave serves RPW = 64 / LPR output rows; the LPR lanes of a row read chunks
// l, l + LPR, ... so every load instruction covers LPR x 16 contiguous bytes
// of each of its rows.  Per row the lanes load its scales and zero words once,
// coalesced (lane i of the row holds scale i + LPR t and zero word i); each
// chunk then picks its group's values with a cross-lane read instead of two
// more memory instructions.  The activation loads for the LDS staging are
// issued before the weight loads (vector loads return in order) so the staging
// overlaps the weight stream.  Per chunk the staging stores the 16 activation
// pairs and two sums (Codec::sums); a chunk's sum of x (q - z) is then
// acc - (E + z S) with the chunk's (E, S), acc the dot products with the
// unpacked codes.
template <int MT, int LPR, int KS, int BPL, typename Codec, int OUTK>
__global__ __launch_bounds__(kThreads) void w4_gemv_kernel(
    const uint16_t* __restrict__ X, int M, int K,
    const uint32_t* __restrict__ qweight, const uint16_t* __restrict__ scales,
    const uint32_t* __restrict__ qzeros, int N, int gshift, void* __restrict__ Y) {
  constexpr int RPW = 64 / LPR;
  static_assert(KS == 1 || LPR == 64, "K split across waves needs whole-wave rows");
  // With three or more blocks per lane the codes are unpacked after the
  // barrier, block by block: unpacked early they hold 16 registers per block
  // (74 / 93 VGPRs at 3 / 4 blocks, 6 / 5 waves per SIMD), late the kernel fits
  // 8 waves per SIMD, and the 4096 x 11008 layer measured 8.5 -> 8.15 us.
  // With one or two blocks the early unpack, overlapping the staging, is
  // faster.
  constexpr bool kLateUnpack = BPL >= 3;
  extern __shared__ uint4 smem[];
  __shared__ float red[kWaves][MT];            // per-wave partial sums (K split)
  constexpr int ROWS = kWaves / KS * RPW;      // output rows of the workgroup
  const int C = K >> 5;                        // chunks per row
  uint4* xl = smem;                            // [MT][4][C] activation pairs
  float2* xs = reinterpret_cast<float2*>(smem + MT * 4 * C);   // [MT][C] (E, S)

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int sub = lane / LPR, sl = lane % LPR;
  const int wv = tid >> 6;
  const int part = wv % KS;                    // this wave's share of the row's chunks
  const int n = (blockIdx.x * (kWaves / KS) + wv / KS) * RPW + sub;
  const bool nok = n < N;
  const int ng = K >> gshift, nzw = (ng + 7) >> 3;
  uint32_t* lz = reinterpret_cast<uint32_t*>(xs + MT * C);       // [ROWS][nzw] zero words
  uint16_t* ls = reinterpret_cast<uint16_t*>(lz + ROWS * nzw);   // [ROWS][ng] scales
  const int cshift = gshift - 5;               // chunk -> group

  // ---- 1. activation loads for the staging of batch rows 0 and 1, coalesced:
  //      thread tid loads the 16-byte pieces tid + 512 r (r < RX) of the row,
  //      so each instruction covers 1 KB contiguous and the four pieces of a
  //      32-code chunk land in four adjacent lanes.  Every load up to the
  //      staging is unconditional (pieces past the row re-read its last one,
  //      lanes past it the last valid address), so the count of loads issued
  //      after these is fixed and the staging waits for the activations alone,
  //      not for the weight stream behind them.
  constexpr int XR = MT < 2 ? MT : 2;          // batch rows staged from these registers (M >= XR)
  constexpr int RX = (KS * BPL + 1) / 2;       // rounds: a row has 4 C <= 256 KS BPL pieces
  const int P4 = 4 * C;
  uint4 xv[XR][RX];
#pragma unroll
  for (int m = 0; m < XR; ++m) {
    const uint4* src = reinterpret_cast<const uint4*>(X + m * K);
#pragma unroll
    for (int r = 0; r < RX; ++r) xv[m][r] = src[min(tid + 512 * r, P4 - 1)];
  }

  // ---- 2. the scales and zero words of the workgroup's rows (contiguous in
  //      memory: one 2- / 4-byte piece per thread, only waves holding pieces
  //      load, indices clamped into the arrays), staged in LDS with the
  //      activations; issued before the weights so that the staging waits
  //      never wait for the weight stream.  Then the weights (rows past N read
  //      row N - 1).
  constexpr int RS = (ROWS * 64 * KS * BPL + kThreads - 1) / kThreads;   // rounds for up to one group per chunk
  const int n0 = blockIdx.x * ROWS;
  const int ns = ROWS * ng, nz = ROWS * nzw;
  const int wfirst = __builtin_amdgcn_readfirstlane(64 * wv);      // wave-uniform: whole waves skip
  const size_t slast = static_cast<size_t>(N) * ng - 1, zlast = static_cast<size_t>(N) * nzw - 1;
  uint32_t lsv[RS];
#pragma unroll
  for (int r = 0; r < RS; ++r)
    lsv[r] = wfirst + kThreads * r < ns
                 ? static_cast<uint32_t>(scales[min(static_cast<size_t>(n0) * ng + tid + kThreads * r, slast)])
                 : 0u;
  const uint32_t lzv = wfirst < nz ? qzeros[min(static_cast<size_t>(n0) * nzw + tid, zlast)] : 0u;
  const size_t nn = static_cast<size_t>(min(n, N - 1));
  const uint4* qrow = reinterpret_cast<const uint4*>(qweight + nn * (K >> 3));
  // chunk of block b: LPR (KS b + part) + sl (the KS waves of a row interleave
  // their blocks of LPR chunks)
  uint4 w[BPL];
#pragma unroll
  for (int b = 0; b < BPL; ++b) {
    const int c = LPR * (KS * b + part) + sl;
    w[b] = load_stream16(qrow + min(c, C - 1));
  }

  // ---- 3. staging.  Rows 0 and 1 from the registers above: each lane pairs
  //      its piece, the quad adds the chunk's two sums (the same values as a
  //      sequential sum up to the order of four fp32 additions).  Further rows
  //      (batches of three or more): chunk tid per thread, loaded here.
  auto quad_sum = [](float v) {
    v += bitcast<float>(__builtin_amdgcn_update_dpp(0, bitcast<int>(v), 0xB1, 0xF, 0xF, true));   // pairs
    v += bitcast<float>(__builtin_amdgcn_update_dpp(0, bitcast<int>(v), 0x4E, 0xF, 0xF, true));   // quads
    return v;
  };
#pragma unroll
  for (int m = 0; m < XR; ++m)
#pragma unroll
    for (int r = 0; r < RX; ++r) {
      const int piece = tid + 512 * r;
      const uint32_t u[4] = {xv[m][r].x, xv[m][r].y, xv[m][r].z, xv[m][r].w};
      uint32_t P[4];
      pair_up(u, P);
      float2 es = make_float2(0.0f, 0.0f);
      Codec::stage(P, es);
      es.x = quad_sum(es.x);
      es.y = quad_sum(es.y);
      if (piece < P4) {                          // whole quads: P4 and 512 r are multiples of 4
        xl[(m * 4 + (piece & 3)) * C + (piece >> 2)] = make_uint4(P[0], P[1], P[2], P[3]);
        if ((piece & 3) == 0) xs[m * C + (piece >> 2)] = Codec::sums(es);
      }
    }
  if (tid < C) {
    for (int m = XR; m < MT && m < M; ++m) {
      const uint4* src = reinterpret_cast<const uint4*>(X + m * K) + 4 * tid;
      float2 es = make_float2(0.0f, 0.0f);
      uint4 pq[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint4 v = src[i];
        const uint32_t u[4] = {v.x, v.y, v.z, v.w};
        uint32_t P[4];
        pair_up(u, P);
        Codec::stage(P, es);
        pq[i] = make_uint4(P[0], P[1], P[2], P[3]);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) xl[(m * 4 + i) * C + tid] = pq[i];
      xs[m * C + tid] = Codec::sums(es);
    }
  }
#pragma unroll
  for (int r = 0; r < RS; ++r)
    if (tid + kThreads * r < ns) ls[tid + kThreads * r] = static_cast<uint16_t>(lsv[r]);
  if (tid < nz) lz[tid] = lzv;
  // ---- 4. unpack the codes and look up the groups' scales and zero points
  //      while the activation staging is still in flight (this needs only the
  //      weights), then the dot products once the staged activations are visible
  const int rowl = (wv / KS) * RPW + sub;     // this row within the workgroup
  uint32_t p[BPL][4][4];
#pragma unroll
  for (int b = 0; b < BPL; ++b) {
    const int c = LPR * (KS * b + part) + sl;
    if constexpr (!kLateUnpack) {
      if (c < C) {
        Codec::unpack(w[b].x, p[b][0]);
        Codec::unpack(w[b].y, p[b][1]);
        Codec::unpack(w[b].z, p[b][2]);
        Codec::unpack(w[b].w, p[b][3]);
      }
    }
  }
  __syncthreads();                             // staged activations and statistics visible
  float s[BPL], zf[BPL];
#pragma unroll
  for (int b = 0; b < BPL; ++b) {               // lanes past the row end read its last group, discarded
    const int g = min(LPR * (KS * b + part) + sl, C - 1) >> cshift;
    s[b] = f16_bits_to_f32(ls[rowl * ng + g]);
    zf[b] = static_cast<float>((lz[rowl * nzw + (g >> 3)] >> (4 * (g & 7))) & 15u);
  }

  float res[MT];
#pragma unroll
  for (int m = 0; m < MT; ++m) res[m] = 0.0f;
#pragma unroll
  for (int b = 0; b < BPL; ++b) {
    const int c = LPR * (KS * b + part) + sl;
    if (c < C) {
      if constexpr (kLateUnpack) {
        Codec::unpack(w[b].x, p[b][0]);
        Codec::unpack(w[b].y, p[b][1]);
        Codec::unpack(w[b].z, p[b][2]);
        Codec::unpack(w[b].w, p[b][3]);
      }
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        if (m < M) {
          float acc = 0.0f;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const uint4 xp = xl[(m * 4 + i) * C + c];
            acc = Codec::dot(p[b][i][0], xp.x, acc);
            acc = Codec::dot(p[b][i][1], xp.y, acc);
            acc = Codec::dot(p[b][i][2], xp.z, acc);
            acc = Codec::dot(p[b][i][3], xp.w, acc);
          }
          res[m] = fmaf(s[b], Codec::finish(acc, xs[m * C + c], zf[b]), res[m]);
        }
      }
    }
  }
  // ---- 5. reduce over each row's lanes (the row's last lane holds the sum),
  //      then over the KS waves of the row in a fixed order, and store
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    if (m < M) {
      const float v = group_sum<LPR>(res[m]);
      if constexpr (KS == 1) {
        if (sl == LPR - 1 && nok) store_out<OUTK>(Y, static_cast<size_t>(m) * N + n, v);
      } else {
        if (lane == 63) red[wv][m] = v;
      }
    }
  }
  if constexpr (KS > 1) {
    __syncthreads();
    if (part == 0 && lane == 63 && nok) {
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        if (m < M) {
          float v = red[wv][m];
#pragma unroll
          for (int q = 1; q < KS; ++q) v += red[wv + q][m];
          store_out<OUTK>(Y, static_cast<size_t>(m) * N + n, v);
        }
      }
    }
  }
}

template <int MT, int LPR, int KS, int BPL, typename Codec, int OUTK>
void launch_t(const W4Args& a, hipStream_t stream) {
  constexpr int RPW = 64 / LPR;
  constexpr int ROWS = kWaves / KS * RPW;      // output rows per workgroup
  const int C = a.K >> 5;
  const int ng = a.K / a.G, nzw = (ng + 7) / 8;
  const size_t lds = static_cast<size_t>(MT) * 4 * C * 16 + static_cast<size_t>(MT) * C * 8 +
                     static_cast<size_t>(ROWS) * (4 * nzw + 2 * ng);
  const int grid = (a.N + ROWS - 1) / ROWS;
  const int gshift = __builtin_ctz(static_cast<unsigned>(a.G));
  hipLaunchKernelGGL((w4_gemv_kernel<MT, LPR, KS, BPL, Codec, OUTK>), dim3(grid), dim3(kThreads), lds, stream,
                     static_cast<const uint16_t*>(a.X), a.M, a.K, a.qweight, a.scales, a.qzeros, a.N, gshift, a.Y);
}

template <int MT, int LPR, int KS, int BPL>
void launch_b(const W4Args& a, hipStream_t stream) {
  const bool bf = a.x_dtype == QLIN_BF16;
  const int ok = a.y_dtype == QLIN_F16 ? OUT_F16 : (a.y_dtype == QLIN_BF16 ? OUT_BF16 : OUT_F32);
  if (!bf) {
    if (ok == OUT_F16) launch_t<MT, LPR, KS, BPL, W4F16, OUT_F16>(a, stream);
    else if (ok == OUT_BF16) launch_t<MT, LPR, KS, BPL, W4F16, OUT_BF16>(a, stream);
    else launch_t<MT, LPR, KS, BPL, W4F16, OUT_F32>(a, stream);
  } else {
    if (ok == OUT_F16) launch_t<MT, LPR, KS, BPL, W4BF16, OUT_F16>(a, stream);
    else if (ok == OUT_BF16) launch_t<MT, LPR, KS, BPL, W4BF16, OUT_BF16>(a, stream);
    else launch_t<MT, LPR, KS, BPL, W4BF16, OUT_F32>(a, stream);
  }
}

template <int MT>
void launch_m(const W4Args& a, hipStream_t stream) {
  // One row per wave, 64 lanes; rows with more than two blocks of 64 chunks are
  // split over KS waves (at most 4 blocks per wave, so the unpacked codes of the
  // wave fit in registers and the per-wave tail after the activations arrive
  // stays short).  Rows per wave, fewer lanes per row and 16-wave workgroups
  // were measured slower, and so were two waves per row on 4096-long rows
  // (11008 x 4096: 8.3 against 7.0 us; 4096 x 4096: 4.8 against 4.2-4.6).
  const int blocks = ((a.K >> 5) + 63) / 64;
  if (blocks <= 1) launch_b<MT, 64, 1, 1>(a, stream);
  else if (blocks <= 2) launch_b<MT, 64, 1, 2>(a, stream);
  else if (blocks <= 4) launch_b<MT, 64, 2, 2>(a, stream);
  else if (blocks <= 6) launch_b<MT, 64, 2, 3>(a, stream);
  else launch_b<MT, 64, 2, 4>(a, stream);
}

// Debug: codes recovered from the same and-or unpack the GEMV uses (the pair
// (n_j, n_{j+4}) of register j), zeros from the same nibble extraction.
__global__ void w4_unpack_kernel(const uint32_t* __restrict__ qweight, const uint32_t* __restrict__ qzeros,
                                 int N, int K, int G, uint8_t* __restrict__ codes, uint8_t* __restrict__ zeros) {
  const size_t words = static_cast<size_t>(N) * (K >> 3);
  for (size_t i = blockIdx.x * static_cast<size_t>(blockDim.x) + threadIdx.x; i < words;
       i += static_cast<size_t>(gridDim.x) * blockDim.x) {
    uint32_t p[4];
    W4F16::unpack(qweight[i], p);
    uint8_t* dst = codes + i * 8;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      dst[j] = static_cast<uint8_t>(W4F16::code_of(j, static_cast<uint16_t>(p[j])));
      dst[j + 4] = static_cast<uint8_t>(W4F16::code_of(j, static_cast<uint16_t>(p[j] >> 16)));
    }
  }
  const int ng = K / G, nzw = (ng + 7) >> 3;
  const size_t nz = static_cast<size_t>(N) * ng;
  for (size_t i = blockIdx.x * static_cast<size_t>(blockDim.x) + threadIdx.x; i < nz;
       i += static_cast<size_t>(gridDim.x) * blockDim.x) {
    const size_t n = i / ng;
    const int g = static_cast<int>(i - n * ng);
    zeros[i] = static_cast<uint8_t>((qzeros[n * nzw + (g >> 3)] >> (4 * (g & 7))) & 15u);
  }
}

}  // namespace

void w4_unpack_launch(const uint32_t* qweight, const uint32_t* qzeros, int N, int K, int G,
                      uint8_t* codes, uint8_t* zeros, hipStream_t stream) {
  hipLaunchKernelGGL(w4_unpack_kernel, dim3(1024), dim3(256), 0, stream, qweight, qzeros, N, K, G, codes, zeros);
}

size_t w4_gemv_lds_bytes(int M, int K) {
  const size_t MT = M <= 1 ? 1 : M <= 2 ? 2 : M <= 4 ? 4 : M <= 8 ? 8 : 16;
  const size_t C = static_cast<size_t>(K) / 32;
  // activations and their sums, and the statistics of up to 8 rows at one
  // group per chunk (the smallest group size)
  return MT * 4 * C * 16 + MT * C * 8 + 8 * (4 * ((C + 7) / 8) + 2 * C);
}

bool w4_gemv_supported(int M, int K, int G) {
  // one pass holds at most 8 blocks of 64 chunks per row (K <= 16384)
  return M <= 16 && K <= 16384 && w4_gemv_lds_bytes(M, K) <= 64 * 1024 && G >= 32;
}

void w4_gemv_launch(const W4Args& a, hipStream_t stream) {
  if (a.M <= 1) launch_m<1>(a, stream);
  else if (a.M <= 2) launch_m<2>(a, stream);
  else if (a.M <= 4) launch_m<4>(a, stream);
  else if (a.M <= 8) launch_m<8>(a, stream);
  else launch_m<16>(a, stream);
}

}  // namespace qlin
