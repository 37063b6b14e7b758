// SpQR GEMV / skinny GEMM (M <= 16) with the CSR outliers fused, gfx950.
//
// Y[m][n] = sum_k x[m][k] * s_hat(q - z_hat)  +  sum_{(n,k,v) in CSR} x[m][k] * v
//
// The SpQR bulletin ("İddia ve Gerçeklik") describes inference as decompressing
// the dense 3-bit weights while the sparse fp16 product runs beside it, and
// warns that mixing the irregular sparse part with dense blocks costs register
// pressure and divergence.  Here both parts feed ONE fp32 accumulator per
// (row, batch entry) in the same pass:
//   * a row is served by one wave (two for long rows, each taking half of its
//     chunks); lane j of a wave reads the 32-code chunks j, j+64, ... of its
//     part (three 32-bit words each);
//   * the chunk layout places two codes of the same group in field i of the low
//     and high 16-bit halves of a word, so one shift + and-or yields an fp16 pair
//     1024 + 8c exactly, ready for v_dot2 against activation pairs staged in LDS
//     in the matching order;
//   * the two first-level statistics of the chunk's groups are decoded from
//     their 3-bit codes and the block's fp16 second-level values
//     (s_hat = SS_s (c_s - ZS_s), z_hat = SS_z (c_z - ZS_z)) in fp32;
//   * then the same lanes walk the row's CSR segment (entry e goes to lane
//     e mod 64 of one of the row's waves), gather x from LDS and add x * v into
//     the same accumulators, before one DPP reduction per row (and a
//     fixed-order sum of its waves' parts).  No second pass, no atomics.
// Activations are staged in K-slices when M*K does not fit the LDS budget.

#include <type_traits>

#include "common.hpp"
#include "device.hpp"
#include "launch.hpp"
#include "spqr_chunk.hpp"

namespace qlin {

namespace {

constexpr int kWaves = 8;                // output rows (one per wavefront) per workgroup
constexpr int kThreads = 64 * kWaves;
// LDS for one K slice: two workgroups still fit a CU's 160 KB, and a 6656-wide row is one slice up
// to 4 batch rows
constexpr size_t kLdsBudget = 72 * 1024;

// Sum over the 64 lanes of a wave with DPP row operations and row broadcasts;
// the total ends up in lane 63.
__device__ __forceinline__ float row_sum64(float v) {
  auto dpp = [](float x, auto ctrl_c) -> float {
    constexpr int C = decltype(ctrl_c)::value;
    constexpr int RM = C == 0x142 ? 0xA : C == 0x143 ? 0xC : 0xF;
    constexpr bool BC = C != 0x142 && C != 0x143;
    return bitcast<float>(__builtin_amdgcn_update_dpp(0, bitcast<int>(x), C, RM, 0xF, BC));
  };
  v += dpp(v, std::integral_constant<int, 0xB1>{});    // quad_perm [1,0,3,2]: pairs
  v += dpp(v, std::integral_constant<int, 0x4E>{});    // quad_perm [2,3,0,1]: quads
  v += dpp(v, std::integral_constant<int, 0x141>{});   // row_half_mirror: groups of 8
  v += dpp(v, std::integral_constant<int, 0x140>{});   // row_mirror: rows of 16
  v += dpp(v, std::integral_constant<int, 0x142>{});   // row_bcast:15 into rows 1 and 3
  v += dpp(v, std::integral_constant<int, 0x143>{});   // row_bcast:31 into rows 2 and 3
  return v;
}

// A row is served by KSW waves, each taking a contiguous run of the slice's
// chunks (a multiple of 8 chunks, so a wave's statistic blocks are its own);
// lane l of a wave reads its chunks l, l + 64, ... (12 bytes each, 768
// contiguous bytes per load instruction).  Per slice, in this order:
//   1. the activation loads for the LDS staging (one 32-value piece per
//      thread; vector loads return in order, so these arrive first),
//   2. everything else the workgroup needs from HBM: the statistics of its
//      rows' blocks in the slice (one 4-byte piece per thread: a row's blocks
//      are contiguous, so this takes a few wide requests per workgroup rather
//      than gathers by every wave), the wave's chunks and, on the first slice,
//      up to 4 CSR entries per lane (no load waits for another before the
//      stream is issued),
//   3. the staging (pairs in the unpack order + two per-chunk sums), then
//      the statistic pieces into LDS,
//   4. the code unpack, while other waves' staging may still be in flight,
//   5. after the barrier, the dot products, then the row's CSR entries of the
//      slice into the same accumulators.
// One DPP reduction per row and batch entry; the KSW parts are added in a
// fixed order through LDS.  All loads are unconditional (clamped addresses).
template <int MT, int KSW, int BPL, int OUTK>
__global__ __launch_bounds__(kThreads) void spqr_gemv_kernel(
    const uint16_t* X, int M, int K, int KS,
    const uint32_t* codes, const uint32_t* stats1,
    const uint16_t* stats2, const int32_t* row_ptr,
    const int32_t* col_idx, const uint16_t* vals,
    int N, void* Y) {
  constexpr int kCsr = 4;                             // CSR entries per lane held in registers
  extern __shared__ uint4 smem[];
  __shared__ float red[kWaves][MT];
  const int CS = KS >> 5;                             // chunks per slice
  const int BS = KS >> 8;                             // statistic blocks per slice
  uint4* xl = smem;                                   // [MT][4][CS] pair quads
  float* xs = reinterpret_cast<float*>(smem + static_cast<size_t>(MT) * 4 * CS);   // [MT][2*CS]
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int part = wv % KSW;
  // the slice's statistics of the workgroup's rows: [ROWS][bs][3] first-level
  // words, then [ROWS][bs][2] second-level words
  constexpr int ROWS = kWaves / KSW;
  float4* ls2f = reinterpret_cast<float4*>(xs + static_cast<size_t>(MT) * 2 * CS);   // [ROWS][bs] combined second level
  uint32_t* ls1 = reinterpret_cast<uint32_t*>(ls2f + static_cast<size_t>(ROWS) * BS);  // [ROWS][bs][3] first-level words

  const int n = blockIdx.x * (kWaves / KSW) + wv / KSW;
  const int rowl = wv / KSW;                          // this row within the workgroup
  const bool nok = n < N;
  const int C = K >> 5, nb = K >> 8;
  const size_t nrow = static_cast<size_t>(min(n, N - 1));
  const uint32_t* crow = codes + nrow * C * 3;
  int p0 = row_ptr[nrow];                            // unconditional: a select here would wait for the load
  int p1 = row_ptr[nrow + 1];
  int e0 = 0, e1 = 0;                                 // this row's CSR range (empty past N), set on the first slice

  // CSR entries of this row held by this lane: e0 + 64 (KSW i + part) + lane,
  // loaded on the first slice behind the dense stream and kept as raw fp16
  // bits until used (a conversion here would make the wave wait for each
  // load); bit i of cvalid flags a real entry
  int ccol[kCsr];
  uint32_t cbits[kCsr];
  uint32_t cvalid = 0u;

  float res[MT];
#pragma unroll
  for (int m = 0; m < MT; ++m) res[m] = 0.0f;

  // one K slice; the first is peeled off the loop (straight-line code, so the
  // row_ptr values are waited for where the CSR preload uses them, after the
  // stream is issued, not hoisted ahead of it)
  auto slice = [&](const int k0, auto first_c) {
    constexpr bool kFirst = decltype(first_c)::value;
    const int ks = min(KS, K - k0);
    const int cs = ks >> 5, bs = ks >> 8;
    const int cbase = k0 >> 5, bbase = k0 >> 8;
    const int cp = ((cs + KSW - 1) / KSW + 7) & ~7;   // chunks per part, a multiple of 8
    const int c0 = part * cp, c1 = min(cs, c0 + cp);

    // ---- 1. first staging piece of this thread (item it = tid; clamped; its
    //      token floor(it / cs) taken as (it + 1/2) times the hardware
    //      reciprocal, exact for it < 2048 and cs <= 1024 as above)
    const int items = M * cs;
    const float invcs = __builtin_amdgcn_rcpf(static_cast<float>(cs));
    uint4 xv[4];
    {
      const int it = min(tid, items - 1);
      const int m = static_cast<int>((static_cast<float>(it) + 0.5f) * invcs), c = it - m * cs;
      const uint4* src = reinterpret_cast<const uint4*>(X + static_cast<size_t>(m) * K + k0) + 4 * c;
#pragma unroll
      for (int i = 0; i < 4; ++i) xv[i] = src[i];
    }
    // ---- 2. the slice's statistics of the workgroup's rows (contiguous per
    //      row: one 4-byte piece per thread, 768 and 512 at most, only waves
    //      holding pieces load, rows past N read row N - 1), issued before the
    //      chunks so that the staging stores never wait for the chunk stream;
    //      then this wave's chunks (clamped into the row)
    //      (the row of piece i is floor(i / (w bs)), w = 3 or 2, taken as
    //      (i + 1/2) times the hardware reciprocal, which is within 1 ulp: i <
    //      1024 and w bs <= 384 keep the quotient at least 1 / 768 from an
    //      integer while the error moves it by less than 1024 * 2^-21; a host
    //      check over every reachable size with the reciprocal moved by up to
    //      2 ulp either way finds no mismatch)
    const int n0 = blockIdx.x * ROWS;
    const int it1 = ROWS * bs * 3, it2 = ROWS * bs * 2;
    const float inv1 = __builtin_amdgcn_rcpf(static_cast<float>(bs * 3));
    const float inv2 = __builtin_amdgcn_rcpf(static_cast<float>(bs * 2));
    const int wfirst = 64 * wv;
    uint32_t v1[2], v2;
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      if (wfirst + kThreads * r < it1) {
        const int i = min(tid + kThreads * r, it1 - 1);
        const int row = static_cast<int>((static_cast<float>(i) + 0.5f) * inv1);
        const int wi = i - row * (bs * 3);
        v1[r] = stats1[static_cast<size_t>(min(n0 + row, N - 1)) * nb * 3 + bbase * 3 + wi];
      } else {
        v1[r] = 0u;
      }
    }
    if (wfirst < it2) {
      const int i = min(tid, it2 - 1);
      const int row = static_cast<int>((static_cast<float>(i) + 0.5f) * inv2);
      const int wi = i - row * (bs * 2);
      v2 = reinterpret_cast<const uint32_t*>(stats2)[static_cast<size_t>(min(n0 + row, N - 1)) * nb * 2 + bbase * 2 + wi];
    } else {
      v2 = 0u;
    }
    uint3 w[BPL];
#pragma unroll
    for (int b = 0; b < BPL; ++b) {
      const int c = min(c0 + 64 * b + lane, cs - 1);
      w[b] = *reinterpret_cast<const uint3*>(crow + 3 * (cbase + c));
    }
    __builtin_amdgcn_sched_barrier(0);               // the whole code stream is issued before anything below
    if constexpr (kFirst) {
      // the row_ptr values pass through an empty asm after the stream is
      // issued, so that nothing using them is scheduled ahead of it
      asm volatile("" : "+v"(p0), "+v"(p1));
      e0 = nok ? p0 : 0;
      e1 = nok ? p1 : 0;
#pragma unroll
      for (int i = 0; i < kCsr; ++i) {
        // unconditional (a conditional load here is followed by a wait for
        // it): entries past the row re-read one inside the arrays, which are
        // never empty (with no outliers the entry point passes row_ptr)
        const int e = e0 + 64 * (KSW * i + part) + lane;
        const int ec = max(min(e, p1 - 1), 0);
        ccol[i] = col_idx[ec];
        cbits[i] = vals[ec];
        cvalid |= e < e1 ? 1u << i : 0u;
      }
    }
    // ---- 3. staging (after a barrier from the second slice on: the previous
    //      slice's readers must be done); the activations first: they were
    //      loaded first, so this VALU work overlaps the weight loads still in
    //      flight
    if constexpr (!kFirst) __syncthreads();
    for (int it = tid; it < items; it += kThreads) {
      const int m = static_cast<int>((static_cast<float>(it) + 0.5f) * invcs), c = it - m * cs;
      uint32_t u[16];
      if (it == tid) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          u[4 * i] = xv[i].x; u[4 * i + 1] = xv[i].y; u[4 * i + 2] = xv[i].z; u[4 * i + 3] = xv[i].w;
        }
      } else {
        const uint4* src = reinterpret_cast<const uint4*>(X + static_cast<size_t>(m) * K + k0) + 4 * c;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint4 v = src[i];
          u[4 * i] = v.x; u[4 * i + 1] = v.y; u[4 * i + 2] = v.z; u[4 * i + 3] = v.w;
        }
      }
      uint32_t P[16];
#pragma unroll
      for (int q = 0; q < 16; ++q) P[q] = half_of(u, pair_lo(q)) | (half_of(u, pair_hi(q)) << 16);
#pragma unroll
      for (int q = 0; q < 4; ++q)
        xl[(static_cast<size_t>(m) * 4 + q) * CS + c] = make_uint4(P[4 * q], P[4 * q + 1], P[4 * q + 2], P[4 * q + 3]);
      // group sums by dot products with (1, 1): pairs 0..7 hold group 2c, 8..15 group 2c+1
      float sa = 0.0f, sb = 0.0f;
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        sa = dot2_f16(P[q], 0x3C003C00u, sa);
        sb = dot2_f16(P[8 + q], 0x3C003C00u, sb);
      }
      xs[m * 2 * CS + 2 * c] = sa;
      xs[m * 2 * CS + 2 * c + 1] = sb;
    }
#pragma unroll
    for (int r = 0; r < 2; ++r)
      if (tid + kThreads * r < it1) ls1[tid + kThreads * r] = v1[r];
    // second-level pairs go to LDS already combined into what a chunk's decode
    // needs, per (row, block): scale pair (SS, ZS) -> SS, -SS ZS and zero pair
    // -> -SS, SS ZS - 128, so that s_hat = SS c + (-SS ZS) and -(128 + z_hat)
    // = (-SS) c + (SS ZS - 128) are one fma each (piece i -> floats 2i, 2i + 1)
    if (tid < it2) {
      const float S2 = f16_bits_to_f32(static_cast<uint16_t>(v2));
      const float Z2 = f16_bits_to_f32(static_cast<uint16_t>(v2 >> 16));
      reinterpret_cast<float2*>(ls2f)[tid] =
          (tid & 1) ? make_float2(-S2, fmaf(S2, Z2, -128.0f)) : make_float2(S2, -(S2 * Z2));
    }
    // ---- 4. unpack this wave's chunks while the staging completes
    uint32_t pk[BPL][16];
#pragma unroll
    for (int b = 0; b < BPL; ++b) unpack_chunk(w[b].x, w[b].y, w[b].z, pk[b]);
    __syncthreads();

    // ---- 5. dense 3-bit part
#pragma unroll
    for (int b = 0; b < BPL; ++b) {
      const int c = c0 + 64 * b + lane;
      if (nok && c < c1) {
        const int blk = c >> 3, j = c & 7;             // block within the slice; chunk within the block
        const uint32_t* r1 = ls1 + (rowl * bs + blk) * 3;
        const float4 d = ls2f[rowl * bs + blk];
        const int off = 12 * j;                         // bit offset of the chunk's two 6-bit fields
        const uint32_t lo = off < 32 ? r1[0] : (off < 64 ? r1[1] : r1[2]);
        const uint32_t hi = off < 32 ? r1[1] : r1[2];
        const uint32_t f = static_cast<uint32_t>(((static_cast<uint64_t>(hi) << 32) | lo) >> (off & 31)) & 0xFFFu;
        // s_hat and -(128 + z_hat) of the chunk's two groups
        const float sA = fmaf(d.x, static_cast<float>(f & 7u), d.y);
        const float cA = fmaf(d.z, static_cast<float>((f >> 3) & 7u), d.w);
        const float sB = fmaf(d.x, static_cast<float>((f >> 6) & 7u), d.y);
        const float cB = fmaf(d.z, static_cast<float>((f >> 9) & 7u), d.w);
#pragma unroll
        for (int m = 0; m < MT; ++m) {
          if (m < M) {
            float aA = 0.0f, aB = 0.0f;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const uint4 xp = xl[(static_cast<size_t>(m) * 4 + q) * CS + c];
              if (q < 2) {
                aA = dot2_f16(pk[b][4 * q], xp.x, aA);
                aA = dot2_f16(pk[b][4 * q + 1], xp.y, aA);
                aA = dot2_f16(pk[b][4 * q + 2], xp.z, aA);
                aA = dot2_f16(pk[b][4 * q + 3], xp.w, aA);
              } else {
                aB = dot2_f16(pk[b][4 * q], xp.x, aB);
                aB = dot2_f16(pk[b][4 * q + 1], xp.y, aB);
                aB = dot2_f16(pk[b][4 * q + 2], xp.z, aB);
                aB = dot2_f16(pk[b][4 * q + 3], xp.w, aB);
              }
            }
            // sum x (c - z_hat) = acc / 8 - (128 + z_hat) * sum(x)
            const float2 xab = reinterpret_cast<const float2*>(xs)[static_cast<size_t>(m) * CS + c];
            const float tA = fmaf(aA, 0.125f, cA * xab.x);
            const float tB = fmaf(aB, 0.125f, cB * xab.y);
            res[m] = fmaf(sA, tA, res[m]);
            res[m] = fmaf(sB, tB, res[m]);
          }
        }
      }
    }

    // ---- CSR outliers of this row whose column falls in the slice
    auto outlier = [&](int colg, float v) {
      const int col = colg - k0;
      if (col < 0 || col >= ks) return;
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
    };
    if (nok) {
#pragma unroll
      for (int i = 0; i < kCsr; ++i)
        if ((cvalid >> i) & 1u) outlier(ccol[i], f16_bits_to_f32(static_cast<uint16_t>(cbits[i])));
      for (int e = e0 + 64 * (KSW * kCsr + part) + lane; e < e1; e += 64 * KSW)
        outlier(col_idx[e], f16_bits_to_f32(vals[e]));
    }
  };
  slice(0, std::true_type{});
  for (int k0 = KS; k0 < K; k0 += KS) slice(k0, std::false_type{});

  // ---- reduction over the row's lanes, then over its KSW waves in a fixed order
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    if (m < M) {
      const float r = row_sum64(res[m]);
      if constexpr (KSW == 1) {
        if (nok && lane == 63) store_out<OUTK>(Y, static_cast<size_t>(m) * N + n, r);
      } else {
        if (lane == 63) red[wv][m] = r;
      }
    }
  }
  if constexpr (KSW > 1) {
    __syncthreads();
    if (part == 0 && lane == 63 && nok) {
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        if (m < M) {
          float v = red[wv][m];
#pragma unroll
          for (int q = 1; q < KSW; ++q) v += red[wv + q][m];
          store_out<OUTK>(Y, static_cast<size_t>(m) * N + n, v);
        }
      }
    }
  }
}

template <int MT, int KSW, int BPL>
void launch_k(const SpqrArgs& a, int KS, hipStream_t stream) {
  const int CS = KS / 32, BS = KS / 256;
  const size_t lds = static_cast<size_t>(MT) * 4 * CS * 16 + static_cast<size_t>(MT) * 2 * CS * 4 +
                     static_cast<size_t>(kWaves / KSW) * BS * 28;
  const int rows = kWaves / KSW;
  const int grid = (a.N + rows - 1) / rows;
  // more than 64 KB of dynamic LDS must be allowed per kernel (once per process,
  // thread-safe initialisation of function-local statics)
  static const bool lds_f32 = (hipFuncSetAttribute(reinterpret_cast<const void*>(spqr_gemv_kernel<MT, KSW, BPL, OUT_F32>),
                                                   hipFuncAttributeMaxDynamicSharedMemorySize,
                                                   static_cast<int>(kLdsBudget + 1024)) == hipSuccess);
  static const bool lds_f16 = (hipFuncSetAttribute(reinterpret_cast<const void*>(spqr_gemv_kernel<MT, KSW, BPL, OUT_F16>),
                                                   hipFuncAttributeMaxDynamicSharedMemorySize,
                                                   static_cast<int>(kLdsBudget + 1024)) == hipSuccess);
  (void)lds_f32;
  (void)lds_f16;
  if (a.y_dtype == QLIN_F32)
    hipLaunchKernelGGL((spqr_gemv_kernel<MT, KSW, BPL, OUT_F32>), dim3(grid), dim3(kThreads), lds, stream,
                       a.X, a.M, a.K, KS, a.codes, a.stats1, a.stats2, a.row_ptr, a.col_idx, a.vals, a.N, a.Y);
  else
    hipLaunchKernelGGL((spqr_gemv_kernel<MT, KSW, BPL, OUT_F16>), dim3(grid), dim3(kThreads), lds, stream,
                       a.X, a.M, a.K, KS, a.codes, a.stats1, a.stats2, a.row_ptr, a.col_idx, a.vals, a.N, a.Y);
}

template <int MT>
void launch_m(const SpqrArgs& a, hipStream_t stream) {
  // K slice (multiple of 256): staged activations (2.25 bytes per value and batch
  // row) plus the rows' statistics (28 bytes per 256 values and row, priced at
  // one row per wave) within the LDS budget, at most 32768 values (with the
  // split below a workgroup's rows then hold at most 768 first-level and 512
  // second-level statistic words per slice: 8 rows x 32 blocks, 4 x 64 or 2 x
  // 128, two and one pieces per thread)
  const double per_k = 2.25 * MT + 28.0 * kWaves / 256.0;
  int KS = static_cast<int>(static_cast<double>(kLdsBudget) / per_k);
  if (KS > 32768) KS = 32768;
  KS = KS / 256 * 256;
  if (KS < 256) KS = 256;
  if (KS > a.K) KS = a.K;
  // as many slices as that needs, of equal size (a short last slice would pay a
  // whole pass of staging, barriers and load latency for little work); K and
  // the largest slice are multiples of 256, so this size stays within the budget
  const int nslices = (a.K + KS - 1) / KS;
  KS = (a.K / 256 + nslices - 1) / nslices * 256;
  // split a row over KSW waves so that each wave has at most 4 chunks per lane
  // (its unpacked codes then stay in registers), and give each wave the fewest
  // 64-chunk blocks that cover its part (every block is loaded and unpacked)
  const int cs = KS / 32;
  const int ksw = cs <= 256 ? 1 : cs <= 512 ? 2 : 4;
  const int cp = ((cs + ksw - 1) / ksw + 7) & ~7;          // chunks per wave, as in the kernel
  const int bpl = (cp + 63) / 64;
  if (ksw == 1) {
    if (bpl <= 1) launch_k<MT, 1, 1>(a, KS, stream);
    else if (bpl == 2) launch_k<MT, 1, 2>(a, KS, stream);
    else if (bpl == 3) launch_k<MT, 1, 3>(a, KS, stream);
    else launch_k<MT, 1, 4>(a, KS, stream);
  } else if (ksw == 2) {
    if (bpl <= 3) launch_k<MT, 2, 3>(a, KS, stream);
    else launch_k<MT, 2, 4>(a, KS, stream);
  } else {
    if (bpl <= 3) launch_k<MT, 4, 3>(a, KS, stream);
    else launch_k<MT, 4, 4>(a, KS, stream);
  }
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
  // single tokens only: from two tokens on the four-row and matrix-core
  // kernels are faster at every shape measured, and the router sends them there
  launch_m<1>(a, stream);
}

void spqr_unpack_launch(const uint32_t* codes, const uint32_t* stats1, int N, int K,
                        uint8_t* q, uint8_t* cs, uint8_t* cz, hipStream_t stream) {
  hipLaunchKernelGGL(spqr_unpack_kernel, dim3(1024), dim3(256), 0, stream, codes, stats1, N, K, q, cs, cz);
}

}  // namespace qlin
