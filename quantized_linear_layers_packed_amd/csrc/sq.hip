// SmoothQuant W8A8 on gfx950: per-token smooth + int8 quantize, then an int8
// MFMA GEMM with a per-token x per-channel rescale epilogue.
//
// SmoothQuant bulletin ("İddia ve Gerçeklik" and its equation
// Y = (X diag(s)^-1)(diag(s) W)): s is folded into the weights offline; online,
// the activations are divided by s per channel, quantized per token to int8 and
// multiplied against per-channel int8 weights on the INT8 matrix units.
//
// Activation kernel: one workgroup per token row.  x~ = fp32(x) * inv_s,
// a = max |x~| (wave shuffle, then LDS across the four waves),
// scale = a / 127, q = clamp(rint(x~ * (127 / a)), -127, 127) with correctly
// rounded fp32 divisions and round-half-even, so the int8 codes and scales
// equal the host definition bit for bit.
//
// GEMM kernels: v_mfma_i32_32x32x32_i8, exact int32 accumulation
// (|acc| <= K * 127^2 < 2^31 for K <= 131072).  The token tile of Xq and the
// weight rows stream from HBM straight into a multi-stage LDS ring several K
// steps ahead.  Epilogue: float(acc) * x_scale[m] * w_scale[n], rounded once.
// Up to 2 tokens a GEMV with v_dot4; up to 32 a small-batch kernel with the K
// split inside the workgroup (v_mfma_i32_16x16x64_i8); larger batches a grid of
// eight waves with tiles of up to 256 x 128, whose operands are re-read from L2
// half as often per multiply-add; tiles of 32 TM x 128 (one wave per 32
// columns) where K is not a multiple of 128.

#include <algorithm>

#include "common.hpp"
#include "device.hpp"
#include "launch.hpp"
#include "splitk.hpp"
#include "tile_gemm.hpp"
#include "workspace.hpp"

namespace qlin {

namespace {

constexpr int kActThreads = 256;
constexpr int kActKeep = 4;           // groups of 8 values per thread kept in registers between the passes

__global__ __launch_bounds__(kActThreads) void sq_act_kernel(const uint16_t* __restrict__ X,
                                                             const float* __restrict__ inv_s, int K,
                                                             int8_t* __restrict__ Xq, float* __restrict__ x_scale) {
  __shared__ float red[kActThreads / 64];
  const int m = blockIdx.x;
  const uint4* xr = reinterpret_cast<const uint4*>(X + static_cast<size_t>(m) * K);
  const int nv = K >> 3;                      // groups of 8 values
  // x~ = x * inv_s for group i; the first kActKeep groups of each thread stay
  // in registers for the quantize pass (rows up to 8 * 4 * 256 = 8192 values
  // are read once), later groups are read again
  auto scaled = [&](int i, float (&t)[8]) {
    const uint4 v = xr[i];
    const uint32_t u[4] = {v.x, v.y, v.z, v.w};
    const float4 s0 = reinterpret_cast<const float4*>(inv_s)[2 * i];
    const float4 s1 = reinterpret_cast<const float4*>(inv_s)[2 * i + 1];
    const float sv[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
#pragma unroll
    for (int j = 0; j < 8; ++j) t[j] = f16_bits_to_f32(static_cast<uint16_t>(u[j >> 1] >> (16 * (j & 1)))) * sv[j];
  };
  float keep[kActKeep][8];
  float amax = 0.0f;
#pragma unroll
  for (int c = 0; c < kActKeep; ++c) {
    const int i = threadIdx.x + c * kActThreads;
    if (i < nv) {
      scaled(i, keep[c]);
#pragma unroll
      for (int j = 0; j < 8; ++j) amax = fmaxf(amax, fabsf(keep[c][j]));
    }
  }
  for (int i = threadIdx.x + kActKeep * kActThreads; i < nv; i += kActThreads) {
    float t[8];
    scaled(i, t);
#pragma unroll
    for (int j = 0; j < 8; ++j) amax = fmaxf(amax, fabsf(t[j]));
  }
  amax = wave_max(amax);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = amax;
  __syncthreads();
  float a = red[0];
#pragma unroll
  for (int w = 1; w < kActThreads / 64; ++w) a = fmaxf(a, red[w]);
  const float r = (a == 0.0f) ? 0.0f : __fdiv_rn(127.0f, a);
  if (threadIdx.x == 0) x_scale[m] = (a == 0.0f) ? 0.0f : __fdiv_rn(a, 127.0f);

  uint2* qr = reinterpret_cast<uint2*>(Xq + static_cast<size_t>(m) * K);
  auto quantize = [&](int i, const float (&t)[8]) {
    uint32_t packed[2] = {0u, 0u};
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float q = fminf(fmaxf(rintf(__fmul_rn(t[j], r)), -127.0f), 127.0f);
      const uint32_t b = static_cast<uint32_t>(static_cast<int32_t>(q)) & 0xFFu;
      packed[j >> 2] |= b << (8 * (j & 3));
    }
    qr[i] = make_uint2(packed[0], packed[1]);
  };
#pragma unroll
  for (int c = 0; c < kActKeep; ++c) {
    const int i = threadIdx.x + c * kActThreads;
    if (i < nv) quantize(i, keep[c]);
  }
  for (int i = threadIdx.x + kActKeep * kActThreads; i < nv; i += kActThreads) {
    float t[8];
    scaled(i, t);
    quantize(i, t);
  }
}

// GEMV for batches of at most 2 tokens (4 where K is not a multiple of 128),
// where the product is bound by the
// weight stream: each output row is served by KS waves (KS contiguous blocks
// of 64 lanes x 16 bytes interleaved, so every load instruction covers 1 KB of
// the row); all of a lane's weight chunks are loaded first, then the matching
// 16-byte activation chunks (shared by every row of the workgroup, so they come
// from cache) feed v_dot4 (exact int32); lane sums, then the KS waves' sums in a
// fixed order, then the same epilogue as the GEMM.
constexpr int kGemvWaves = 8;

template <int MT, int KS, int BPL, int OUTK>
__global__ __launch_bounds__(64 * kGemvWaves) void sq_gemv_kernel(
    const int8_t* __restrict__ Xq, const float* __restrict__ x_scale, const int8_t* __restrict__ Wq,
    const float* __restrict__ w_scale, int M, int N, int K, void* __restrict__ Y, int32_t* __restrict__ acc_out) {
  __shared__ int red[kGemvWaves][MT];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int part = wv % KS;
  const int n = blockIdx.x * (kGemvWaves / KS) + wv / KS;
  const int C = K >> 4;                                           // 16-byte chunks per row
  const uint4* wrow = reinterpret_cast<const uint4*>(Wq + static_cast<size_t>(min(n, N - 1)) * K);
  // Every load is issued before any arithmetic and none is conditional (chunks
  // past the row end re-read its last chunk, batch rows past M the last row),
  // so the waits before the dot products count exactly: the activation chunks
  // (cache hits behind the weight stream) are never fetched one at a time.
  // A chunk past the row end gets a zero weight, adding exactly nothing; the
  // launch shape keeps such chunks to less than one block per row.
  uint4 w[BPL];
#pragma unroll
  for (int b = 0; b < BPL; ++b) {
    const int c = 64 * (KS * b + part) + lane;
    w[b] = load_stream16(wrow + min(c, C - 1));
  }
  uint4 x[BPL][MT];
#pragma unroll
  for (int b = 0; b < BPL; ++b) {
    const int c = min(64 * (KS * b + part) + lane, C - 1);
#pragma unroll
    for (int m = 0; m < MT; ++m) x[b][m] = reinterpret_cast<const uint4*>(Xq + static_cast<size_t>(min(m, M - 1)) * K)[c];
  }
  int acc[MT];
#pragma unroll
  for (int m = 0; m < MT; ++m) acc[m] = 0;
#pragma unroll
  for (int b = 0; b < BPL; ++b) {
    const bool inrow = 64 * (KS * b + part) + lane < C;
    const uint4 wb = inrow ? w[b] : make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      acc[m] = __builtin_amdgcn_sdot4(static_cast<int>(wb.x), static_cast<int>(x[b][m].x), acc[m], false);
      acc[m] = __builtin_amdgcn_sdot4(static_cast<int>(wb.y), static_cast<int>(x[b][m].y), acc[m], false);
      acc[m] = __builtin_amdgcn_sdot4(static_cast<int>(wb.z), static_cast<int>(x[b][m].z), acc[m], false);
      acc[m] = __builtin_amdgcn_sdot4(static_cast<int>(wb.w), static_cast<int>(x[b][m].w), acc[m], false);
    }
  }
#pragma unroll
  for (int m = 0; m < MT; ++m) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) acc[m] += __shfl_xor(acc[m], off);
  }
  if constexpr (KS > 1) {
    if (lane == 0) {
#pragma unroll
      for (int m = 0; m < MT; ++m) red[wv][m] = acc[m];
    }
    __syncthreads();
  }
  if (part == 0 && lane == 0 && n < N) {
    const float wsc = w_scale[n];
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      if (m < M) {
        int a = acc[m];
        if constexpr (KS > 1) {
          a = red[wv][m];
#pragma unroll
          for (int q = 1; q < KS; ++q) a += red[wv + q][m];
        }
        const size_t idx = static_cast<size_t>(m) * N + n;
        store_out<OUTK>(Y, idx, static_cast<float>(a) * x_scale[m] * wsc);
        if (acc_out) acc_out[idx] = a;
      }
    }
  }
}

template <int MT, int KS, int BPL, int OUTK>
void gemv_t(const int8_t* Xq, const float* xsc, const int8_t* Wq, const float* wsc, int M, int N, int K, void* Y,
            int32_t* acc_out, hipStream_t stream) {
  constexpr int rows = kGemvWaves / KS;
  hipLaunchKernelGGL((sq_gemv_kernel<MT, KS, BPL, OUTK>), dim3((N + rows - 1) / rows), dim3(64 * kGemvWaves), 0,
                     stream, Xq, xsc, Wq, wsc, M, N, K, Y, acc_out);
}

template <int MT, int OUTK>
void gemv_k(const int8_t* Xq, const float* xsc, const int8_t* Wq, const float* wsc, int M, int N, int K, void* Y,
            int32_t* acc_out, hipStream_t stream) {
  // blocks of 64 chunks (1 KB) per row, at most 4 per lane: 1, 2, 4 or 8 waves
  // per row, each with the fewest blocks that cover the row (every block is
  // loaded, so a block past the row end would be wasted work)
  const int blocks = ((K >> 4) + 63) / 64;
  if (blocks <= 1) gemv_t<MT, 1, 1, OUTK>(Xq, xsc, Wq, wsc, M, N, K, Y, acc_out, stream);
  else if (blocks <= 2) gemv_t<MT, 1, 2, OUTK>(Xq, xsc, Wq, wsc, M, N, K, Y, acc_out, stream);
  else if (blocks <= 3) gemv_t<MT, 1, 3, OUTK>(Xq, xsc, Wq, wsc, M, N, K, Y, acc_out, stream);
  else if (blocks <= 4) gemv_t<MT, 1, 4, OUTK>(Xq, xsc, Wq, wsc, M, N, K, Y, acc_out, stream);
  else if (blocks <= 6) gemv_t<MT, 2, 3, OUTK>(Xq, xsc, Wq, wsc, M, N, K, Y, acc_out, stream);
  else if (blocks <= 8) gemv_t<MT, 2, 4, OUTK>(Xq, xsc, Wq, wsc, M, N, K, Y, acc_out, stream);
  else if (blocks <= 12) gemv_t<MT, 4, 3, OUTK>(Xq, xsc, Wq, wsc, M, N, K, Y, acc_out, stream);
  else if (blocks <= 16) gemv_t<MT, 4, 4, OUTK>(Xq, xsc, Wq, wsc, M, N, K, Y, acc_out, stream);
  else if (blocks <= 24) gemv_t<MT, 8, 3, OUTK>(Xq, xsc, Wq, wsc, M, N, K, Y, acc_out, stream);
  else gemv_t<MT, 8, 4, OUTK>(Xq, xsc, Wq, wsc, M, N, K, Y, acc_out, stream);
}

template <int MT>
void gemv_o(const int8_t* Xq, const float* xsc, const int8_t* Wq, const float* wsc, int M, int N, int K, void* Y,
            int y_dtype, int32_t* acc_out, hipStream_t stream) {
  if (y_dtype == QLIN_F32) gemv_k<MT, OUT_F32>(Xq, xsc, Wq, wsc, M, N, K, Y, acc_out, stream);
  else gemv_k<MT, OUT_F16>(Xq, xsc, Wq, wsc, M, N, K, Y, acc_out, stream);
}

// Small batches (5 .. 32 tokens): CT tiles of 16 output columns per workgroup
// of NWV waves that split K (128-byte blocks) among themselves, each wave
// accumulating 16 x 16 int32 tiles (TM of them along the batch) with
// v_mfma_i32_16x16x64_i8; the waves' tiles are added in wave order through LDS
// (exact, no workspace, no hand-off between workgroups), then the GEMM's
// epilogue.  Weights and activations go straight from memory into D-deep
// register rings (unconditional, clamped loads); lane quarter h of an MFMA
// takes bytes 64 s + 16 h .. + 15 of block s of both operands.
template <int NWV, int TM, int D, int CT, int OUTK>
__global__ __launch_bounds__(64 * NWV) void sq_skinny_kernel(
    const int8_t* __restrict__ Xq, const float* __restrict__ x_scale, const int8_t* __restrict__ Wq,
    const float* __restrict__ w_scale, int M, int N, int K, void* __restrict__ Y, int32_t* __restrict__ acc_out) {
  __shared__ i32x4_t red[NWV][CT * TM][64];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 15, h = lane >> 4;
  const int n0 = blockIdx.x * (16 * CT);
  const int nb = K >> 7;                                          // 128-byte K blocks
  const int b0 = (wv * nb) / NWV, b1 = ((wv + 1) * nb) / NWV;
  const int8_t* wrow[CT];
  const int8_t* xrow[TM];
#pragma unroll
  for (int c = 0; c < CT; ++c) wrow[c] = Wq + static_cast<size_t>(min(n0 + 16 * c + col, N - 1)) * K + 16 * h;
#pragma unroll
  for (int t = 0; t < TM; ++t) xrow[t] = Xq + static_cast<size_t>(min(16 * t + col, M - 1)) * K + 16 * h;

  i32x4_t acc[CT][TM];
#pragma unroll
  for (int c = 0; c < CT; ++c)
#pragma unroll
    for (int t = 0; t < TM; ++t) acc[c][t] = i32x4_t{};

  if (b0 < b1) {
    const int blast = b1 - 1;
    uint4 wq[D][CT][2];
    uint4 av[D][TM][2];
    auto load = [&](int b, uint4 (&w)[CT][2], uint4 (&a)[TM][2]) {
#pragma unroll
      for (int c = 0; c < CT; ++c)
#pragma unroll
        for (int q = 0; q < 2; ++q) w[c][q] = *reinterpret_cast<const uint4*>(wrow[c] + 128 * b + 64 * q);
#pragma unroll
      for (int t = 0; t < TM; ++t)
#pragma unroll
        for (int q = 0; q < 2; ++q) a[t][q] = *reinterpret_cast<const uint4*>(xrow[t] + 128 * b + 64 * q);
    };
    auto compute = [&](const uint4 (&w)[CT][2], const uint4 (&a)[TM][2]) {
#pragma unroll
      for (int q = 0; q < 2; ++q)
#pragma unroll
        for (int c = 0; c < CT; ++c)
#pragma unroll
          for (int t = 0; t < TM; ++t)
            acc[c][t] = __builtin_amdgcn_mfma_i32_16x16x64_i8(bitcast<i32x4_t>(a[t][q]), bitcast<i32x4_t>(w[c][q]),
                                                             acc[c][t], 0, 0, 0);
    };
#pragma unroll
    for (int j = 0; j < D - 1; ++j) load(min(b0 + j, blast), wq[j], av[j]);
    auto step = [&](auto slot_c, int b) {
      constexpr int S = decltype(slot_c)::value;
      constexpr int SF = (S + D - 1) % D;
      load(min(b + D - 1, blast), wq[SF], av[SF]);
      __builtin_amdgcn_sched_barrier(0);     // keep the prefetch issued ahead of the math
      compute(wq[S], av[S]);
    };
    // The one-tile, 16-row kernel runs whole ring groups in an exit-free loop
    // (4096 x 4096: 7.6 -> 6.4 us at M = 8, 8.3 -> 7.1 at M = 16, with the ring
    // 3 deep instead of 4); the others keep an exit after every step, whose
    // batched prefetches measured faster for them (11008 x 4096: 14.2 vs 15.0
    // us at M = 8, 18.8 vs 20.1 at M = 32).
    if constexpr (CT == 1 && TM == 1) {
      sk_ring_steps<D>(step, b0, b1);
    } else {
      int b = b0;
      while (sk_run_steps<0, D>(step, b, b1)) {
      }
    }
  }

  // fixed-order sum of the waves' tiles; lane l of a tile holds column l % 16,
  // rows 4 (l / 16) + r; wave c TM + t sums tile (c, t) and stores it
#pragma unroll
  for (int c = 0; c < CT; ++c)
#pragma unroll
    for (int t = 0; t < TM; ++t) red[wv][c * TM + t][lane] = acc[c][t];
  __syncthreads();
  if (wv < CT * TM) {
    const int t = wv % TM;
    const int n = n0 + 16 * (wv / TM) + col;
    i32x4_t tot = red[0][wv][lane];
#pragma unroll
    for (int w = 1; w < NWV; ++w) tot += red[w][wv][lane];
    if (n < N) {
      const float wsc = w_scale[n];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = 16 * t + 4 * h + r;
        if (m < M) {
          const size_t idx = static_cast<size_t>(m) * N + n;
          store_out<OUTK>(Y, idx, static_cast<float>(tot[r]) * x_scale[m] * wsc);
          if (acc_out) acc_out[idx] = tot[r];
        }
      }
    }
  }
}

template <int NWV, int TM, int D, int CT>
void skinny_o(const int8_t* Xq, const float* xsc, const int8_t* Wq, const float* wsc, int M, int N, int K, void* Y,
              int y_dtype, int32_t* acc_out, hipStream_t stream) {
  static_assert(CT * TM <= NWV, "one summing wave per output tile");
  const dim3 grid((N + 16 * CT - 1) / (16 * CT));
  if (y_dtype == QLIN_F32)
    hipLaunchKernelGGL((sq_skinny_kernel<NWV, TM, D, CT, OUT_F32>), grid, dim3(64 * NWV), 0, stream, Xq, xsc, Wq, wsc,
                       M, N, K, Y, acc_out);
  else
    hipLaunchKernelGGL((sq_skinny_kernel<NWV, TM, D, CT, OUT_F16>), grid, dim3(64 * NWV), 0, stream, Xq, xsc, Wq, wsc,
                       M, N, K, Y, acc_out);
}

constexpr int kGemmThreads = 256;   // 4 waves side by side along N
constexpr int kBN = 128;            // output columns per tile
constexpr int kBK = 128;            // K bytes per step (4 MFMA steps of 32)

// Tiles of BM = 32 TM rows x 128 columns; a wave owns all BM rows and 32
// columns.  Within one 128-byte K step, MFMA step st and lane half h use bytes
// 64h + 16st .. +15 of both operands (a fixed permutation of k, identical for A
// and B).  Both operands stream from HBM straight into an NS-stage LDS ring
// (direct-to-LDS loads, NS - 1 steps ahead, no registers involved); each
// 128-byte row is stored with its 16-byte chunks XOR-swizzled by row / 2, which
// the direct loads realise by choosing which global chunk each lane fetches, so
// the 32 rows an MFMA reads fall in distinct banks.  One explicit vmcnt wait and
// one barrier per step.  The (tile, K step) space is split evenly over the
// workgroups (stream-K); shared tiles are summed (int32, exact) by the last
// workgroup to finish them.
template <int TM, int NS, int OUTK>
__global__ __launch_bounds__(kGemmThreads) void sq_gemm_sk_kernel(
    const int8_t* __restrict__ Xq, const float* __restrict__ x_scale, const int8_t* __restrict__ Wq,
    const float* __restrict__ w_scale, int M, int N, int K, int tiles_n, SkPlan plan, void* __restrict__ Y,
    int32_t* __restrict__ acc_out, int* __restrict__ ws, int* __restrict__ counters) {
  constexpr int BM = 32 * TM;
  constexpr int A_PIECES = BM * 8, B_PIECES = kBN * 8;         // 16-byte pieces per stage
  constexpr int STAGE = A_PIECES + B_PIECES;
  constexpr int DMA_PER_STAGE = TM + 4;                         // direct loads per wave per stage
  extern __shared__ uint4 smem[];
  __shared__ int s_last;

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int col = lane & 31, h = lane >> 5;
  const int swz = (col >> 1) & 7;                               // swizzle of every row this lane reads
  const int lrow = lane >> 3, lpos = lane & 7;                  // this lane's piece in a direct load

  const int p = xcd_tile(blockIdx.x, gridDim.x);
  long long u = sk_begin(plan, p);
  const long long u_end = sk_begin(plan, p + 1);

  while (u < u_end) {
    const int t = static_cast<int>(u / plan.ksteps);
    const int k0 = static_cast<int>(u - static_cast<long long>(t) * plan.ksteps);
    const int k1 = static_cast<int>(std::min<long long>(plan.ksteps, k0 + (u_end - u)));
    const int klast = k1 - 1;
    const int m0 = (t / tiles_n) * BM;
    const int nt0 = (t % tiles_n) * kBN;
    const int n = nt0 + 32 * wv + col;
    const bool nok = n < N;

    // Direct loads for ring position j (slot j % NS) of the data of step s =
    // min(j, klast).  Wave wv loads A row blocks wv*TM .. and B row blocks wv*4 ..
    // (8 rows of 128 bytes per instruction).  Rows past M / N read the last row
    // (their results are never stored); positions past the range re-read its last
    // step into slots no step of the range reads again; chunks past K (half step)
    // read the row's last chunk and meet zeroed activations.
    auto issue = [&](int j) {
      const int s = min(j, klast);
      uint4* slot = smem + static_cast<size_t>(j % NS) * STAGE;
#pragma unroll
      for (int j = 0; j < TM; ++j) {
        const int rb = wv * TM + j;
        const int row = 8 * rb + lrow;
        const int c = lpos ^ ((row >> 1) & 7);
        const int m = min(m0 + row, M - 1);
        dma16(Xq + static_cast<size_t>(m) * K + min(s * kBK + 16 * c, K - 16), slot + 64 * rb);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int rb = wv * 4 + j;
        const int row = 8 * rb + lrow;
        const int c = lpos ^ ((row >> 1) & 7);
        const int nn = min(nt0 + row, N - 1);
        dma16(Wq + static_cast<size_t>(nn) * K + min(s * kBK + 16 * c, K - 16), slot + A_PIECES + 64 * rb);
      }
    };

    i32x16_t acc[TM];
#pragma unroll
    for (int i = 0; i < TM; ++i) acc[i] = i32x16_t{};

#pragma unroll
    for (int j = 0; j < NS - 1; ++j) issue(k0 + j);

    for (int kk = k0; kk < k1; ++kk) {
      wait_vmcnt<(NS - 2) * DMA_PER_STAGE>();                   // this wave's loads of step kk
      barrier_raw();                                            // everyone's; step kk - 1 finished
      const uint4* slot = smem + static_cast<size_t>(kk % NS) * STAGE;
      if (kk * kBK + kBK > K) {                                 // half step: zero A chunks past K
        uint4* a = const_cast<uint4*>(slot);
        for (int q = tid; q < BM * 4; q += kGemmThreads) {
          const int row = q >> 2, c = 4 + (q & 3);
          a[row * 8 + (c ^ ((row >> 1) & 7))] = make_uint4(0u, 0u, 0u, 0u);
        }
        __syncthreads();
      }
      issue(kk + NS - 1);
      const uint4* As = slot;
      const uint4* Bs = slot + A_PIECES + (32 * wv + col) * 8;
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        const int c = 4 * h + st;
        const i32x4_t b = bitcast<i32x4_t>(Bs[c ^ swz]);
#pragma unroll
        for (int i = 0; i < TM; ++i) {
          const i32x4_t a = bitcast<i32x4_t>(As[(32 * i + col) * 8 + (c ^ swz)]);
          acc[i] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, acc[i], 0, 0, 0);
        }
      }
    }
    wait_vmcnt<0>();                                            // loads past the range end
    __syncthreads();

    // ---- finish the tile: lane holds column n, rows 8*(r/4) + 4*h + r%4 of each 32-row block
    bool write = true;
    if (k0 != 0 || k1 != plan.ksteps) {
      const int first = sk_owner(plan, static_cast<long long>(t) * plan.ksteps);
      const int last = sk_owner(plan, static_cast<long long>(t + 1) * plan.ksteps - 1);
      int* mine = ws + static_cast<size_t>(sk_slot(plan, p, t)) * (BM * kBN);
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) sk_store(mine + ((wv * TM + i) * 16 + r) * 64 + lane, acc[i][r]);
      write = sk_arrive_last(&counters[first], last - first, &s_last);
      if (write) {
        for (int q = first; q <= last; ++q) {
          if (q == p) continue;
          const int* other = ws + static_cast<size_t>(sk_slot(plan, q, t)) * (BM * kBN);
          int part[TM][16];                     // issue all loads, then add (one wait)
#pragma unroll
          for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r) part[i][r] = sk_load(other + ((wv * TM + i) * 16 + r) * 64 + lane);
#pragma unroll
          for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][r] += part[i][r];
        }
        if (tid == 0) sk_reset(&counters[first]);
      }
    }
    if (write && nok) {
      const float wsc = w_scale[n];
      float xsc[TM][16];                        // row scales first (clamped rows, no branches)
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) xsc[i][r] = x_scale[min(m0 + 32 * i + 8 * (r >> 2) + 4 * h + (r & 3), M - 1)];
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int m = m0 + 32 * i + 8 * (r >> 2) + 4 * h + (r & 3);
          if (m < M) {
            const size_t idx = static_cast<size_t>(m) * N + n;
            store_out<OUTK>(Y, idx, static_cast<float>(acc[i][r]) * xsc[i][r] * wsc);
            if (acc_out) acc_out[idx] = acc[i][r];
          }
        }
    }
    u += k1 - k0;
  }
}

// Large tiles for large batches (tile_gemm.hpp): a WM x WN grid of waves,
// each owning 32 TM rows x 32 TN columns, v_mfma_i32_32x32x32_i8 on rows of K
// bytes, exact int32 split-K fix-up; epilogue as above.
struct SqI8Op {
  using acc_t = i32x16_t;
  using part_t = int;
  static constexpr bool kExact = true;
  const float* x_scale;
  const float* w_scale;
  int32_t* acc_out;
  __device__ __forceinline__ static acc_t mfma(i32x4_t a, i32x4_t b, acc_t c) {
    return __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c, 0, 0, 0);
  }
  // one 32 x 32 block's column n, rows mb + 8 (r / 4) + r % 4
  template <int OUTK>
  __device__ __forceinline__ void store(void* Y, int M, int N, int mb, int n, const acc_t& acc) const {
    const float wsc = w_scale[n];
    float xsc[16];                              // row scales first (clamped rows, no branches)
#pragma unroll
    for (int r = 0; r < 16; ++r) xsc[r] = x_scale[min(mb + 8 * (r >> 2) + (r & 3), M - 1)];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int m = mb + 8 * (r >> 2) + (r & 3);
      if (m < M) {
        const size_t idx = static_cast<size_t>(m) * N + n;
        store_out<OUTK>(Y, idx, static_cast<float>(acc[r]) * xsc[r] * wsc);
        if (acc_out) acc_out[idx] = acc[r];
      }
    }
  }
};

template <int TM, int NS, int OUTK>
qlin_status gemm_t(const int8_t* Xq, const float* xsc, const int8_t* Wq, const float* wsc, int M, int N, int K,
                   void* Y, int32_t* acc_out, WsView ws, size_t* need, hipStream_t stream) {
  constexpr int BM = 32 * TM;
  constexpr size_t lds = static_cast<size_t>(NS) * (BM + kBN) * 8 * sizeof(uint4);
  // resident workgroups per CU, queried once per process (thread-safe
  // initialisation of a function-local static), after raising the dynamic LDS limit
  static const int occ = [] {
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(sq_gemm_sk_kernel<TM, NS, OUTK>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
    int o = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&o, sq_gemm_sk_kernel<TM, NS, OUTK>, kGemmThreads, lds) !=
            hipSuccess || o <= 0)
      o = 1;
    return std::min(o, 2);
  }();
  const int tiles_m = (M + BM - 1) / BM;
  const int tiles_n = (N + kBN - 1) / kBN;
  const long long tiles = static_cast<long long>(tiles_m) * tiles_n;
  SkPlan plan;
  plan.ksteps = (K + kBK - 1) / kBK;
  plan.units = tiles * plan.ksteps;
  plan.P = static_cast<int>(std::min<long long>(
      std::min<long long>(static_cast<long long>(occ) * device_cus(), kCounterSlots), plan.units));
  const size_t partial_bytes = static_cast<size_t>(2) * plan.P * BM * kBN * sizeof(int);
  if (need) {
    *need = partial_bytes;
    return QLIN_OK;
  }
  if (ws.bytes < kCounterBytes + partial_bytes)
    return fail(QLIN_EINVAL, "sq_int8_gemm: workspace too small for the split-K GEMM");
  hipLaunchKernelGGL((sq_gemm_sk_kernel<TM, NS, OUTK>), dim3(plan.P), dim3(kGemmThreads), lds, stream, Xq, xsc, Wq,
                     wsc, M, N, K, tiles_n, plan, Y, acc_out, static_cast<int*>(ws.partials()), ws.counters());
  return QLIN_OK;
}

template <int WM, int WN, int TM, int TN, int BK, int NS, int WPE = WM * WN / 4>
qlin_status gemm_big_o(const int8_t* Xq, const float* xsc, const int8_t* Wq, const float* wsc, int M, int N, int K,
                       void* Y, int y_dtype, int32_t* acc_out, WsView ws, size_t* need, hipStream_t stream) {
  const SqI8Op op{xsc, wsc, acc_out};
  return y_dtype == QLIN_F32
             ? tile_gemm_launch<SqI8Op, WM, WN, TM, TN, BK, NS, OUT_F32, WPE>("sq_int8_gemm", Xq, Wq, M, N, K, op, Y,
                                                                               ws, need, stream)
             : tile_gemm_launch<SqI8Op, WM, WN, TM, TN, BK, NS, OUT_F16, WPE>("sq_int8_gemm", Xq, Wq, M, N, K, op, Y,
                                                                               ws, need, stream);
}

template <int TM, int NS>
qlin_status gemm_o(const int8_t* Xq, const float* xsc, const int8_t* Wq, const float* wsc, int M, int N, int K,
                   void* Y, int y_dtype, int32_t* acc_out, WsView ws, size_t* need, hipStream_t stream) {
  return y_dtype == QLIN_F32 ? gemm_t<TM, NS, OUT_F32>(Xq, xsc, Wq, wsc, M, N, K, Y, acc_out, ws, need, stream)
                             : gemm_t<TM, NS, OUT_F16>(Xq, xsc, Wq, wsc, M, N, K, Y, acc_out, ws, need, stream);
}

}  // namespace

void sq_act_launch(const uint16_t* X, const float* inv_s, int M, int K, int8_t* Xq, float* x_scale,
                   hipStream_t stream) {
  hipLaunchKernelGGL(sq_act_kernel, dim3(M), dim3(kActThreads), 0, stream, X, inv_s, K, Xq, x_scale);
}

qlin_status sq_gemm_launch(const int8_t* Xq, const float* x_scale, const int8_t* Wq, const float* w_scale,
                           int M, int N, int K, void* Y, int y_dtype, int32_t* acc_out, WsView ws, size_t* need,
                           hipStream_t stream) {
  // Up to 2 tokens (rows up to 32768): the GEMV, bound by the weight stream;
  // then up to 32 tokens (K a multiple of 128) the small-batch MFMA kernel.
  // Larger batches (K a multiple of 128): eight waves, two per SIMD.  Above 64
  // tokens a 4 x 2 wave grid and the largest tile of 256 x 128 (64 x 64 per
  // wave), 128 x 128 (32 x 64) or 128 x 64 (32 x 32) that still gives at least
  // 160 tiles (the smallest one otherwise): bigger tiles re-read fewer operand
  // bytes per multiply-add, enough tiles keep the K splits to fix up few; 33 to
  // 64 tokens a 2 x 4 grid of 32 x 32 wave tiles (64 x 128).  Batches of at most
  // 32 use the 32 TM x 128 kernel, whose ring depth stays within 160 KB of LDS:
  // stage = (32 TM + 128) rows x 128 bytes.
  if (need) *need = 0;                 // the kernels without a K split need no workspace
  if (M <= 2 && K <= 32768) {
    if (need) return QLIN_OK;
    if (M == 1) gemv_o<1>(Xq, x_scale, Wq, w_scale, M, N, K, Y, y_dtype, acc_out, stream);
    else gemv_o<2>(Xq, x_scale, Wq, w_scale, M, N, K, Y, y_dtype, acc_out, stream);
    return QLIN_OK;
  }
  if (M <= 32 && K % 128 == 0) {
    if (need) return QLIN_OK;
    // small batches: 16-column tiles, 4, 2 or 1 per workgroup while at least
    // 300 workgroups remain (with two 16-token tiles: 2 while at least 160)
    const long long wg4 = (N + 63) / 64, wg2 = (N + 31) / 32;
    if (M <= 16) {
      if (wg4 >= 300) skinny_o<4, 1, 3, 4>(Xq, x_scale, Wq, w_scale, M, N, K, Y, y_dtype, acc_out, stream);
      else if (wg2 >= 300) skinny_o<4, 1, 3, 2>(Xq, x_scale, Wq, w_scale, M, N, K, Y, y_dtype, acc_out, stream);
      else skinny_o<4, 1, 3, 1>(Xq, x_scale, Wq, w_scale, M, N, K, Y, y_dtype, acc_out, stream);
    } else {
      if (wg2 >= 160) skinny_o<4, 2, 3, 2>(Xq, x_scale, Wq, w_scale, M, N, K, Y, y_dtype, acc_out, stream);
      else skinny_o<4, 2, 3, 1>(Xq, x_scale, Wq, w_scale, M, N, K, Y, y_dtype, acc_out, stream);
    }
    return QLIN_OK;
  }
  if (M <= 4 && K <= 32768) {          // K not a multiple of 128
    if (need) return QLIN_OK;
    gemv_o<4>(Xq, x_scale, Wq, w_scale, M, N, K, Y, y_dtype, acc_out, stream);
    return QLIN_OK;
  }
  if (M > 32 && M <= 64 && K % 128 == 0)
    return gemm_big_o<2, 4, 1, 1, 128, 6>(Xq, x_scale, Wq, w_scale, M, N, K, Y, y_dtype, acc_out, ws, need, stream);
  if (M > 64 && K % 128 == 0) {
    auto tiles = [&](int bm, int bn) { return static_cast<long long>((M + bm - 1) / bm) * ((N + bn - 1) / bn); };
    if (tiles(256, 128) >= 160)
      return gemm_big_o<4, 2, 2, 2, 128, 3>(Xq, x_scale, Wq, w_scale, M, N, K, Y, y_dtype, acc_out, ws, need, stream);
    if (tiles(128, 128) >= 160)
      return gemm_big_o<4, 2, 1, 2, 128, 4>(Xq, x_scale, Wq, w_scale, M, N, K, Y, y_dtype, acc_out, ws, need, stream);
    return gemm_big_o<4, 2, 1, 1, 128, 6>(Xq, x_scale, Wq, w_scale, M, N, K, Y, y_dtype, acc_out, ws, need, stream);
  }
  if (M <= 32) return gemm_o<1, 6>(Xq, x_scale, Wq, w_scale, M, N, K, Y, y_dtype, acc_out, ws, need, stream);
  if (M <= 64) return gemm_o<2, 6>(Xq, x_scale, Wq, w_scale, M, N, K, Y, y_dtype, acc_out, ws, need, stream);
  return gemm_o<4, 4>(Xq, x_scale, Wq, w_scale, M, N, K, Y, y_dtype, acc_out, ws, need, stream);
}

}  // namespace qlin
