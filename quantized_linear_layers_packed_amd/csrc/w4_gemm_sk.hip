// W4 dequant -> fp16 MFMA GEMM for batches past the GEMV range (group size 128
// or 256), gfx950.
//
// Y[m][n] = sum_g S[n][g] * sum_{k in g} x[m][k] * (q[n][k] - z[n][g])
//
// At larger batch the weight-only layer becomes compute bound and the dequant
// work is what erodes the gain (GPTQ bulletin, "İddia ve Gerçeklik").  Layout of
// the work:
//   * one workgroup = NW = 8 waves side by side along N (tiles of BM = 32 TM
//     rows x 256 columns); a wave owns all BM rows of the tile and 32 output
//     columns, so every packed word is turned into fp16 once and feeds TM matrix
//     instructions, and eight waves per CU hide each other's dequant work;
//   * B operand: a lane unpacks one word (8 codes of its column) per
//     v_mfma_f32_32x32x16_f16 into fp16 weights s * (q - z), in natural k
//     order: a byte permute + an and-or place each code in the mantissa of
//     1024.0, one packed fp16 subtraction removes 1024 + z (exact) and one packed
//     multiply by the group's fp16 scale rounds the weight once to fp16, as the
//     GPTQ kernels do, so the matrix cores accumulate across groups directly;
//   * A operand: the fp16 activation tile of one 128-wide K step (bf16 inputs
//     arrive as a row-scaled fp16 copy whose per-row power of two the epilogue
//     puts back), stored in LDS as 256-byte rows whose 16-byte chunks are
//     XOR-swizzled by the row, so the 32 rows an MFMA reads land in distinct
//     banks; double buffered;
//   * packed words, the group scale/zero and the activations are fetched R - 1
//     K steps ahead into R-deep register rings (every load unconditional, so the
//     compiler's in-order wait counts never drain the rings): with a few waves
//     per CU, the bytes in flight have to cover the memory latency;
//   * the (tile, K step) space is split evenly over one workgroup per CU
//     (stream-K); tiles shared by several workgroups are summed in K order by
//     the last workgroup to finish them.

#include <algorithm>
#include <type_traits>

#include "common.hpp"
#include "device.hpp"
#include "launch.hpp"
#include "splitk.hpp"
#include "workspace.hpp"

namespace qlin {

namespace {

constexpr int kKS = 128;        // K per step (16 packed words per column)

// Eight fp16 weights s * (q - z) in natural k order from one packed word: q - z
// is exact, the product by the fp16 scale is rounded once to fp16.
__device__ __forceinline__ h8_t dequant_nat(uint32_t w, h2_t zz, h2_t ss) {
  const uint32_t t = w >> 4;
  h8_t b;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    // byte j of w holds codes 2j (low nibble) and 2j + 1; t's byte j has code 2j + 1 low
    const uint32_t sel = static_cast<uint32_t>(j) | (0x0Cu << 8) | (static_cast<uint32_t>(4 + j) << 16) | (0x0Cu << 24);
    const uint32_t pr = __builtin_amdgcn_perm(t, w, sel);
    const h2_t d = (bitcast<h2_t>(and_or(pr, 0x000F000Fu, 0x64006400u)) - zz) * ss;
    b[2 * j] = d[0];
    b[2 * j + 1] = d[1];
  }
  return b;
}

// Eight exact fp16 values q - z in natural k order from one packed word (the
// and-or gives 1024 + q, the packed subtraction of 1024 + z is exact).
__device__ __forceinline__ h8_t codes_minus_zero(uint32_t w, h2_t zz) {
  const uint32_t t = w >> 4;
  h8_t b;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t sel = static_cast<uint32_t>(j) | (0x0Cu << 8) | (static_cast<uint32_t>(4 + j) << 16) | (0x0Cu << 24);
    const uint32_t pr = __builtin_amdgcn_perm(t, w, sel);
    const h2_t d = bitcast<h2_t>(and_or(pr, 0x000F000Fu, 0x64006400u)) - zz;
    b[2 * j] = d[0];
    b[2 * j + 1] = d[1];
  }
  return b;
}

template <int TM, int NW, int R, int RV, int OUTK>
__global__ __launch_bounds__(64 * NW) void w4_gemm_sk_kernel(
    const uint16_t* X, int M, int K, const uint32_t* qweight, const uint16_t* scales,
    const uint32_t* qzeros, int N, int gsh, int tiles_n, SkPlan plan, void* Y, const int* rowexp, float* ws,
    int* counters) {
  // (no __restrict__: with it the prefetch loads count as invariant and get sunk
  // across the step barriers to their first use, which defeats the prefetch)
  constexpr int kThreads = 64 * NW;           // NW waves side by side along N
  constexpr int kBN = 32 * NW;                // output columns per tile
  constexpr int BM = 32 * TM;
  constexpr int APT = BM * 16 / kThreads;   // 16-byte activation pieces per thread per step
  // 32- and 64-row tiles feed exact q - z to the matrix cores and apply the
  // scale per K step in fp32 (fewer VALU per matrix instruction there, and no
  // fp16 rounding of the weights); 128-row tiles dequantize to s (q - z) in
  // fp16, where the per-step rescale of 4 x 16 accumulators would cost more
  constexpr bool kExact = TM <= 2;
  static_assert(APT >= 1, "tile too small");
  extern __shared__ uint4 smem[];
  __shared__ int s_last;
  uint4* const As0 = smem;
  uint4* const As1 = smem + BM * 16;

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int col = lane & 31, h = lane >> 5;
  const int ng = K >> (7 + gsh);              // quantization groups per row
  const int nzw = (ng + 7) >> 3;               // zero-point words per row
  const int swz = col & 15;                    // chunk swizzle of the rows this lane reads

  const int p = xcd_tile(blockIdx.x, gridDim.x);
  long long u = sk_begin(plan, p);
  const long long u_end = sk_begin(plan, p + 1);

  while (u < u_end) {
    const int t = static_cast<int>(u / plan.ksteps);
    const int k0 = static_cast<int>(u - static_cast<long long>(t) * plan.ksteps);
    const int k1 = static_cast<int>(std::min<long long>(plan.ksteps, k0 + (u_end - u)));
    const int m0 = (t / tiles_n) * BM;
    const int n = (t % tiles_n) * kBN + 32 * wv + col;
    const bool nok = n < N;
    const size_t nn = static_cast<size_t>(min(n, N - 1));
    const uint32_t* qrow = qweight + nn * (K >> 3);
    const uint16_t* srow = scales + nn * ng;
    const uint32_t* zrow = qzeros + nn * nzw;

    // ---- loaders
    // Every load below is issued unconditionally (rows, columns and steps past
    // the end are clamped to valid addresses and masked at use): with loads
    // behind branches the count of younger loads would depend on the path and
    // the compiler would drain the whole prefetch queue before each use.
    uint4 av[R][APT];                          // activation ring: step k0 + j in set j % R
    auto load_a = [&](int s, uint4 (&v)[APT]) {
#pragma unroll
      for (int j = 0; j < APT; ++j) {
        const int piece = tid + j * kThreads;
        const int r = piece >> 4, c = piece & 15;
        const int m = min(m0 + r, M - 1);
        v[j] = *reinterpret_cast<const uint4*>(X + static_cast<size_t>(m) * K + s * kKS + 8 * c);
      }
    };
    // Rows past M are loaded from row M - 1 and left in place: a row of A only
    // feeds the same row of the product, and those rows are never stored.
    auto store_a = [&](uint4* dst, const uint4 (&src)[APT]) {
#pragma unroll
      for (int j = 0; j < APT; ++j) {
        const int piece = tid + j * kThreads;
        const int r = piece >> 4, c = piece & 15;
        // copied through a local first: storing src[j] straight to LDS made
        // the compiler keep the whole register ring in scratch memory
        const uint4 v = src[j];
        dst[r * 16 + (c ^ (r & 15))] = v;
      }
    };
    uint4 bq[R][2];                            // weight ring: step k0 + j in set j % R
    uint32_t bs[R], bz[R];
    auto load_b = [&](int s, uint4 (&w)[2], uint32_t& sc, uint32_t& zw) {
      const uint4* src = reinterpret_cast<const uint4*>(qrow) + 4 * s;
      w[0] = src[h];                           // words 4h .. 4h+3 of the step
      w[1] = src[2 + h];                       // words 8+4h .. 8+4h+3
      const int g = s >> gsh;
      sc = srow[g];
      zw = zrow[g >> 3];
    };

    f32x16_t acc[TM];
#pragma unroll
    for (int i = 0; i < TM; ++i) acc[i] = f32x16_t{};

    // ---- prologue
    const int klast = k1 - 1;
    // prologue in the steady-state issue order (weights of step j, then
    // activations of step j + 1), so the wait counts agree at the loop head
    load_a(k0, av[0]);
#pragma unroll
    for (int j = 0; j < R - 1; ++j) {
      load_b(min(k0 + j, klast), bq[j], bs[j], bz[j]);
      load_a(min(k0 + j + 1, klast), av[j + 1]);
    }
    store_a(As0, av[0]);
    __syncthreads();

    auto step = [&](auto set_c, int kk) {
      constexpr int S = decltype(set_c)::value;
      constexpr int SB = (S + R - 1) % R;      // set of step kk - 1, free since that step
      load_b(min(kk + R - 1, klast), bq[SB], bs[SB], bz[SB]);
      __builtin_amdgcn_sched_barrier(0);       // keep the prefetch issued here, ahead of the math
      const uint4* Ab = ((kk - k0) & 1) ? As1 : As0;
      const int g = kk >> gsh;
      const uint32_t z = (bz[S] >> (4 * (g & 7))) & 15u;
      const _Float16 zb = static_cast<_Float16>(1024.0f + static_cast<float>(z));
      const h2_t zz = {zb, zb};
      const _Float16 sh = bitcast<_Float16>(static_cast<uint16_t>(bs[S]));
      const h2_t ss = {sh, sh};
      // the A fragments of MFMA group st + 1 are read from LDS while group st
      // runs, so no matrix instruction waits on a read issued just before it
      auto read_a = [&](int st, h8_t (&a)[TM]) {
        const int c = 8 * (st >> 2) + 4 * h + (st & 3);
#pragma unroll
        for (int i = 0; i < TM; ++i) a[i] = bitcast<h8_t>(Ab[(32 * i + col) * 16 + (c ^ swz)]);
      };
      h8_t afr[2][TM];
      read_a(0, afr[0]);
      if constexpr (kExact) {
        // exact q - z into a step accumulator, scaled into the tile in fp32
        // after the step's matrix instructions (a K step lies in one group)
        const float sf = f16_bits_to_f32(static_cast<uint16_t>(bs[S]));
        f32x16_t accs[TM];
#pragma unroll
        for (int st = 0; st < 8; ++st) {
          if (st + 1 < 8) read_a(st + 1, afr[(st + 1) & 1]);
          __builtin_amdgcn_sched_barrier(0);   // the reads stay ahead of this group's math
          const uint4 q4 = bq[S][st >> 2];
          const uint32_t w = (st & 3) == 0 ? q4.x : (st & 3) == 1 ? q4.y : (st & 3) == 2 ? q4.z : q4.w;
          const h8_t b = codes_minus_zero(w, zz);
#pragma unroll
          for (int i = 0; i < TM; ++i)
            accs[i] = __builtin_amdgcn_mfma_f32_32x32x16_f16(afr[st & 1][i], b, st == 0 ? f32x16_t{} : accs[i], 0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
          for (int r = 0; r < RV; ++r) acc[i][r] = fmaf(sf, accs[i][r], acc[i][r]);
      } else {
#pragma unroll
        for (int st = 0; st < 8; ++st) {
          if (st + 1 < 8) read_a(st + 1, afr[(st + 1) & 1]);
          __builtin_amdgcn_sched_barrier(0);   // the reads stay ahead of this group's math
          const uint4 q4 = bq[S][st >> 2];
          const uint32_t w = (st & 3) == 0 ? q4.x : (st & 3) == 1 ? q4.y : (st & 3) == 2 ? q4.z : q4.w;
          const h8_t b = dequant_nat(w, zz, ss);
#pragma unroll
          for (int i = 0; i < TM; ++i)
            acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_f16(afr[st & 1][i], b, acc[i], 0, 0, 0);
        }
      }
      // the next step's activations (past the range end this rewrites the idle
      // buffer), then the fetch R steps ahead into the set of step kk
      // (emptied at the end of the previous step)
      constexpr int S1 = (S + 1) % R;
      store_a(((kk + 1 - k0) & 1) ? As1 : As0, av[S1]);
      load_a(min(kk + R, klast), av[S]);
      __builtin_amdgcn_sched_barrier(0);
      __syncthreads();
    };

    // Whole groups of R steps in an exit-free loop (no ring drain at the loop
    // head), except for two tiles that keep the step-by-step exits: the
    // 4 x 32-row, 8-wave tile, whose registers do not hold the duplicated tail
    // steps (it would spill), and the 32-row, 2-wave tile, which measured
    // 10% slower with the group loop on the long-K layers (more registers
    // freed for occupancy, but more K splits per tile).
    if constexpr ((TM == 4 && NW == 8) || (TM == 1 && NW == 2)) {
      int kk = k0;
      while (sk_run_steps<0, R>(step, kk, k1)) {
      }
    } else {
      sk_ring_steps<R>(step, k0, k1);
    }

    // ---- finish the tile: lane holds column n, rows 8*(r/4) + 4*h + r%4 of each
    // 32-row block; registers r >= RV hold rows past M only (RV < 16 when M is
    // small) and are neither stored nor summed
    bool write = true;
    if (k0 != 0 || k1 != plan.ksteps) {
      const int first = sk_owner(plan, static_cast<long long>(t) * plan.ksteps);
      const int last = sk_owner(plan, static_cast<long long>(t + 1) * plan.ksteps - 1);
      float* mine = ws + static_cast<size_t>(sk_slot(plan, p, t)) * (BM * kBN);
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int r = 0; r < RV; ++r) sk_store(mine + ((wv * TM + i) * 16 + r) * 64 + lane, acc[i][r]);
      write = sk_arrive_last(&counters[first], last - first, &s_last);
      if (write) {
        // K-order sum of every contributor's stored partial (this workgroup's
        // included), QC partials per batch with all their loads in flight at
        // once: the latency is paid once per batch, not once per partial
        constexpr int QC = 64 / RV;
#pragma unroll
        for (int i = 0; i < TM; ++i) {
          f32x16_t tot = f32x16_t{};
          for (int q0 = first; q0 <= last; q0 += QC) {
            float part[QC][RV];
#pragma unroll
            for (int j = 0; j < QC; ++j) {
              const int q = min(q0 + j, last);
              const float* src = ws + static_cast<size_t>(sk_slot(plan, q, t)) * (BM * kBN) +
                                 ((wv * TM + i) * 16) * 64 + lane;
#pragma unroll
              for (int r = 0; r < RV; ++r) part[j][r] = sk_load(src + r * 64);
            }
#pragma unroll
            for (int j = 0; j < QC; ++j)
              if (q0 + j <= last) {
#pragma unroll
                for (int r = 0; r < RV; ++r) tot[r] += part[j][r];
              }
          }
          acc[i] = tot;
        }
        if (tid == 0) sk_reset(&counters[first]);
      }
    }
    if (write && nok) {
      if (rowexp) {
        // row-scaled fp16 copy of bf16 activations: every row exponent loaded
        // first (clamped rows, no branches), then the exact rescale
        int ex[TM][16];
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
          for (int r = 0; r < 16; ++r) ex[i][r] = rowexp[min(m0 + 32 * i + 8 * (r >> 2) + 4 * h + (r & 3), M - 1)];
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[i][r] = ldexpf(acc[i][r], ex[i][r]);
      }
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int m = m0 + 32 * i + 8 * (r >> 2) + 4 * h + (r & 3);
          if (m < M) store_out<OUTK>(Y, static_cast<size_t>(m) * N + n, acc[i][r]);
        }
    }
    u += k1 - k0;
  }
}

template <int TM, int NW, int R, int RV, int OUTK>
qlin_status launch_sk(const W4Args& a, WsView ws, size_t* need, hipStream_t stream) {
  constexpr int BM = 32 * TM, BN = 32 * NW;
  constexpr size_t lds = static_cast<size_t>(2) * BM * 16 * sizeof(uint4);
  // resident workgroups per CU (register / LDS bound), queried once per
  // process (thread-safe initialisation of a function-local static)
  static const int occ = [] {
    int o = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&o, w4_gemm_sk_kernel<TM, NW, R, RV, OUTK>, 64 * NW, lds) !=
            hipSuccess || o <= 0)
      o = 1;
    return std::min(o, 2);
  }();
  const int tiles_m = (a.M + BM - 1) / BM;
  const int tiles_n = (a.N + BN - 1) / BN;
  const long long tiles = static_cast<long long>(tiles_m) * tiles_n;
  SkPlan plan;
  plan.ksteps = a.K / kKS;
  plan.units = tiles * plan.ksteps;
  plan.P = static_cast<int>(std::min<long long>(
      std::min<long long>(static_cast<long long>(occ) * device_cus(), kCounterSlots), plan.units));
  // At least kMinSteps K steps per workgroup: a split tile costs a round of
  // partial stores, an arrival and a read-back, which thin slices do not repay.
  // And one workgroup per tile, no split, when the tiles fill 2/3 of the slots.
  constexpr long long kMinSteps = 8;
  plan.P = static_cast<int>(std::max<long long>(1, std::min<long long>(plan.P, plan.units / kMinSteps)));
  if (tiles <= plan.P && 3 * tiles >= 2 * static_cast<long long>(plan.P)) plan.P = static_cast<int>(tiles);
  const size_t partial_bytes = static_cast<size_t>(2) * plan.P * BM * BN * sizeof(float);
  if (need) {
    *need = partial_bytes;
    return QLIN_OK;
  }
  if (ws.bytes < kCounterBytes + partial_bytes)
    return fail(QLIN_EINVAL, "qlin_w4_forward: workspace too small for the split-K GEMM");
  const int gsh = a.G == 256 ? 1 : 0;
  hipLaunchKernelGGL((w4_gemm_sk_kernel<TM, NW, R, RV, OUTK>), dim3(plan.P), dim3(64 * NW), lds, stream,
                     static_cast<const uint16_t*>(a.X), a.M, a.K, a.qweight, a.scales, a.qzeros, a.N, gsh, tiles_n,
                     plan, a.Y, a.rowexp, static_cast<float*>(ws.partials()), ws.counters());
  return QLIN_OK;
}

template <int TM, int NW, int R, int RV>
qlin_status launch_o(const W4Args& a, WsView ws, size_t* need, hipStream_t stream) {
  if (a.y_dtype == QLIN_F16) return launch_sk<TM, NW, R, RV, OUT_F16>(a, ws, need, stream);
  if (a.y_dtype == QLIN_BF16) return launch_sk<TM, NW, R, RV, OUT_BF16>(a, ws, need, stream);
  return launch_sk<TM, NW, R, RV, OUT_F32>(a, ws, need, stream);
}

}  // namespace

qlin_status w4_gemm_sk_launch(const W4Args& a, WsView ws, size_t* need, hipStream_t stream) {
  // RV: accumulator registers per 32-row block that can hold rows below M
  // (register r holds rows 8 (r / 4) + 4 h + r % 4, h the lane half)
  //
  // Tile width: 8 waves (256 columns) unless the layer is short along K
  // (K <= 16384) and gives at most 96 such tiles; then 4 waves (128 columns),
  // or 2 (64 columns) for batches of at most 64 rows and at most 48 tiles of
  // 256.  A split of a tile into S parts costs partial traffic of about
  // 8 BM S / K times its weight bytes, so short-K layers want more tiles and
  // fewer splits, while long-K layers split cheaply and keep the wider tiles
  // (fewer dequantized words per multiply-add).  Measured on the 7B-shaped
  // layers (three, fp16): 65.5 -> 50.6 us at 32 rows, 83.8 -> 64.0 at 64,
  // 130 -> 94 at 128, 128 -> 113 at 256; the 70B-shaped layers keep 8 waves
  // except the 8192 x 8192 one below 256 rows (29.7 -> 27.7 us at 32).
  // (batches up to 16 rows take the small-batch kernel at these group sizes)
  const int TM = a.M <= 32 ? 1 : a.M <= 64 ? 2 : 4;
  const long long tiles8 = static_cast<long long>((a.M + 32 * TM - 1) / (32 * TM)) * ((a.N + 255) / 256);
  const int nw = (a.K > 16384 || tiles8 > 96) ? 8 : (TM <= 2 && tiles8 <= 48) ? 2 : 4;
  // Register rings 3 deep at every tile height: measured against the former
  // 6 / 4 deep at 32 / 64 rows, 70B-shaped layers 151 -> 145 us at 32 rows and
  // 174 -> 166 at 64, 7B-shaped layers 52.4 -> 51.0 and 65.1 -> 63.2 (a 2-deep
  // ring: 166 / 170 on the 70B-shaped layers; a 4-deep one capped at 128 VGPRs
  // for two workgroups per CU: 172 at 32 rows).
  if (TM == 1) {
    if (nw == 2) return launch_o<1, 2, 3, 16>(a, ws, need, stream);
    if (nw == 4) return launch_o<1, 4, 3, 16>(a, ws, need, stream);
    return launch_o<1, 8, 3, 16>(a, ws, need, stream);
  }
  if (TM == 2) {
    if (nw == 2) return launch_o<2, 2, 3, 16>(a, ws, need, stream);
    if (nw == 4) return launch_o<2, 4, 3, 16>(a, ws, need, stream);
    return launch_o<2, 8, 3, 16>(a, ws, need, stream);
  }
  if (nw == 4) return launch_o<4, 4, 3, 16>(a, ws, need, stream);
  return launch_o<4, 8, 3, 16>(a, ws, need, stream);
}

}  // namespace qlin
