// W4 dequant -> fp16 MFMA GEMM on an LDS ring fed by direct loads (groups of
// 128 / 256, batches past the small-batch kernel), gfx950.
//
// Y[m][n] = sum_g S[n][g] * sum_{k in g} x[m][k] * (q[n][k] - z[n][g])
//
// The weight-only layer stays bound by the weight stream well past a handful of
// tokens, and at larger batches the dequant work is what erodes the gain (GPTQ
// bulletin, "İddia ve Gerçeklik").  Layout of the work:
//   * a WM x WN grid of waves, each owning 32 TM rows x 32 TN columns (TM x TN
//     blocks of v_mfma_f32_32x32x16_f16), tiles of BM = 32 TM WM rows x
//     BN = 32 TN WN columns, K steps of 128;
//   * both operands go from HBM straight into an NS-stage LDS ring (direct
//     loads, NS - 1 steps ahead, no registers): per step a 256-byte row of fp16
//     activations per tile row and the 64-byte row of packed codes (16 words)
//     per tile column, 16-byte chunks XOR-swizzled (activations by row & 15,
//     codes by (column >> 2) & 3) through the choice of which global chunk
//     each lane fetches, so the fragment reads fall in distinct banks;
//   * within a step, MFMA step st and lane half h use word 8h + st of the
//     column (codes k = 64h + 8st .. +7) and the activations of the same k:
//     a fixed permutation of k, the same for both operands.  Each lane reads
//     its column's eight words of the step with two 16-byte LDS reads, and
//     turns each into fp16 s (q - z) (an and-or places two codes in 1024.0's
//     mantissa, one packed subtraction of 1024 + z, exact, and one packed
//     multiply by the fp16 group scale, rounded once), which feeds TM matrix
//     instructions;
//   * the group scale and zero of a column come through the same ring, as the
//     16-byte chunks of the scale and zero rows that hold them: a load into
//     registers inside the loop, or a 4-byte direct load, made the compiler
//     wait for every outstanding load at each step;
//   * the (tile, K step) space is split over the workgroups as in the other
//     stream-K GEMMs: at least 8 K steps each, one workgroup per tile when the
//     tiles fill 2/3 of the slots; a shared tile is summed in K order by the
//     last contributor to arrive (splitk.hpp), so results do not depend on
//     timing.

#include <algorithm>

#include "common.hpp"
#include "device.hpp"
#include "launch.hpp"
#include "splitk.hpp"
#include "workspace.hpp"

namespace qlin {

namespace {

constexpr int kKS = 128;        // K per step: 16 packed words per column, 256 activation bytes per row

// Eight fp16 weights s * (q - z) in natural k order from one packed word (code
// j in bits 4j .. 4j + 3): q - z is exact, the product by the fp16 scale is
// rounded once to fp16.
__device__ __forceinline__ h8_t w4_dequant8(uint32_t w, h2_t zz, h2_t ss) {
  const uint32_t t = w >> 4;
  h8_t b;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    // byte j of w holds codes 2j (low nibble) and 2j + 1; t's byte j has code 2j + 1 low
    const uint32_t sel = static_cast<uint32_t>(j) | (0x0Cu << 8) | (static_cast<uint32_t>(4 + j) << 16) | (0x0Cu << 24);
    const uint32_t pr = __builtin_amdgcn_perm(t, w, sel);
    const h2_t d = (bitcast<h2_t>((pr & 0x000F000Fu) | 0x64006400u) - zz) * ss;
    b[2 * j] = d[0];
    b[2 * j + 1] = d[1];
  }
  return b;
}

template <int WM, int WN, int TM, int TN, int NS, int OUTK, int WPE>
__global__ __launch_bounds__(64 * WM * WN) __attribute__((amdgpu_waves_per_eu(WPE, WPE)))
void w4_tile_kernel(const uint16_t* __restrict__ X, int M, int K, const uint32_t* __restrict__ qweight,
                    const uint16_t* __restrict__ scales, const uint32_t* __restrict__ qzeros, int N, int gsh,
                    int tiles_m, SkPlan plan, void* __restrict__ Y, const int* __restrict__ rowexp,
                    float* __restrict__ ws, int* __restrict__ counters) {
  constexpr int NW = WM * WN;
  constexpr int BM = 32 * TM * WM, BN = 32 * TN * WN;
  constexpr int A_PIECES = BM * 16, B_PIECES = BN * 4;          // 16-byte pieces per stage
  constexpr int S_PIECES = 2 * BN;                              // per column a 16-byte chunk of scales and of zeros
  constexpr int STAGE = A_PIECES + B_PIECES + S_PIECES;
  constexpr int A_INS = BM / 4 / NW, B_INS = BN / 16 / NW;      // direct loads per wave per stage
  static_assert(BN % 64 == 0 && NW >= BN / 64, "whole 64-column statistic blocks, one wave or more each");
  constexpr int S_INS = 2;                                      // statistic loads per wave per stage
  static_assert(A_INS * 4 * NW == BM && B_INS * 16 * NW == BN, "row blocks split evenly over the waves");
  static_assert((NS - 2) * (A_INS + B_INS + S_INS) < 64, "vmcnt range");
  extern __shared__ uint4 smem[];
  __shared__ int s_last;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wv % WM, wn = wv / WM;
  const int col = lane & 31, h = lane >> 5;
  const int swz_a = col & 15;                                   // activation rows this lane reads: row & 15 = col & 15
  const int swz_b = (col >> 2) & 3;                             // code rows: (column >> 2) & 3
  const int ng = K >> (7 + gsh);                                // quantization groups per row
  const int nzw = (ng + 7) >> 3;                                // zero-point words per row
  const int kw = K >> 3;                                        // packed words per row
  const size_t nscales = static_cast<size_t>(N) * ng;           // >= 8 (checked by the launcher)
  const size_t nzeros = static_cast<size_t>(N) * nzw;           // >= 4 (checked by the launcher)
  // 16-byte chunk (start index, clamped inside its array) holding scale si / zero word zi
  auto scale_chunk = [&](size_t si) { return min(si & ~static_cast<size_t>(7), nscales - 8); };
  auto zero_chunk = [&](size_t zi) { return min(zi & ~static_cast<size_t>(3), nzeros - 4); };

  const int p = xcd_tile(blockIdx.x, gridDim.x);
  long long u = sk_begin(plan, p);
  const long long u_end = sk_begin(plan, p + 1);

  while (u < u_end) {
    const int t = static_cast<int>(u / plan.ksteps);
    const int k0 = static_cast<int>(u - static_cast<long long>(t) * plan.ksteps);
    const int k1 = static_cast<int>(std::min<long long>(plan.ksteps, k0 + (u_end - u)));
    const int klast = k1 - 1;
    const int m0 = (t % tiles_m) * BM;                          // M-blocks fastest: neighbours share weights
    const int n0 = (t / tiles_m) * BN;

    // Step j (clamped to the range) goes to LDS slot (j - k0) % NS: activation
    // rows, code rows, then the 16-byte chunks of the scale and zero rows that
    // hold each column's fp16 group scale and zero-point word.  Everything a step reads arrives by direct
    // loads, so the loop holds no loads into registers (whose waits the
    // compiler could not place precisely across the loop).  Rows past M /
    // columns past N read the last one (never stored); positions past the
    // range re-read its last step into slots no step of the range reads again.
    auto issue = [&](int j, uint4* slot) __attribute__((always_inline)) {
      const int s = min(j, klast);
      const int g = s >> gsh;
#pragma unroll
      for (int q = 0; q < A_INS; ++q) {
        const int rb = wv + NW * q;
        const int row = 4 * rb + (lane >> 4);
        const int c = (lane & 15) ^ (row & 15);                 // logical chunk stored at this piece
        const int m = min(m0 + row, M - 1);
        dma16(X + static_cast<size_t>(m) * K + s * kKS + 8 * c, slot + 64 * rb);
      }
#pragma unroll
      for (int q = 0; q < B_INS; ++q) {
        const int rb = wv + NW * q;
        const int cl = 16 * rb + (lane >> 2);
        const int c = (lane & 3) ^ ((cl >> 2) & 3);
        const int nn = min(n0 + cl, N - 1);
        dma16(qweight + static_cast<size_t>(nn) * kw + s * 16 + 4 * c, slot + A_PIECES + 64 * rb);
      }
      {
        // every wave: the scale chunks and the zero chunks of 64 columns
        // (waves past BN / 64 repeat a block, writing the same values); two
        // unconditional loads, no branch
        const int blk = wv % (BN / 64);
        const size_t nn = static_cast<size_t>(min(n0 + 64 * blk + lane, N - 1));
        uint4* dst = slot + A_PIECES + B_PIECES + 64 * blk;
        dma16(scales + scale_chunk(nn * ng + g), dst);
        dma16(qzeros + zero_chunk(nn * nzw + (g >> 3)), dst + BN);
      }
    };

    f32x16_t acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) acc[i][j] = f32x16_t{};

    wait_vmcnt<0>();                                            // nothing but the ring in flight below
#pragma unroll
    for (int j = 0; j < NS - 1; ++j) issue(k0 + j, smem + static_cast<size_t>(j) * STAGE);

    auto step = [&](auto slot_c, int kk) __attribute__((always_inline)) {
      constexpr int S = decltype(slot_c)::value;                // (kk - k0) % NS
      constexpr int SF = (S + NS - 1) % NS;                     // slot of step kk - 1, free after the barrier
      // this wave's loads of step kk: younger are the (NS - 2) later steps'
      wait_vmcnt<(NS - 2) * (A_INS + B_INS + S_INS)>();
      barrier_raw();                                            // everyone's; step kk - 1 finished
      // the step's statistics are read before the next step's direct loads go
      // out (read after them, the compiler waited for those loads first)
      // (every LDS read here is a whole-vector load: element reads of the
      // vector struct made the compiler wait for all direct loads first)
      const uint4* Ss = smem + static_cast<size_t>(S) * STAGE + A_PIECES + B_PIECES;
      u32x4_t scv[TN], zwv[TN];
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        scv[j] = bitcast<u32x4_t>(Ss[32 * TN * wn + 32 * j + col]);
        zwv[j] = bitcast<u32x4_t>(Ss[BN + 32 * TN * wn + 32 * j + col]);
      }
      __builtin_amdgcn_sched_barrier(0);
      issue(kk + NS - 1, smem + static_cast<size_t>(SF) * STAGE);
      const uint4* As = smem + static_cast<size_t>(S) * STAGE + (32 * TM * wm + col) * 16;
      const uint4* Bs = smem + static_cast<size_t>(S) * STAGE + A_PIECES + (32 * TN * wn + col) * 4;
      // the eight words of the step for each column block, and its statistics
      uint32_t bw[TN][8];
      h2_t zz[TN], ss[TN];
      const int g = kk >> gsh;
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int cl = 32 * TN * wn + 32 * j + col;
        const size_t nn = static_cast<size_t>(min(n0 + cl, N - 1));
        const u32x4_t w0 = bitcast<u32x4_t>(Bs[32 * 4 * j + ((2 * h) ^ swz_b)]);
        const u32x4_t w1 = bitcast<u32x4_t>(Bs[32 * 4 * j + ((2 * h + 1) ^ swz_b)]);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          bw[j][e] = w0[e];
          bw[j][4 + e] = w1[e];
        }
        // zero word and scale of the step, picked by bitwise selects (no
        // indexed access, no per-lane branch)
        const size_t zi = nn * nzw + (g >> 3);
        const int zp = static_cast<int>(zi - zero_chunk(zi));
        const uint32_t zm1 = 0u - static_cast<uint32_t>(zp & 1), zm2 = 0u - static_cast<uint32_t>((zp >> 1) & 1);
        const uint32_t zlo = (zwv[j][0] & ~zm1) | (zwv[j][1] & zm1), zhi = (zwv[j][2] & ~zm1) | (zwv[j][3] & zm1);
        const uint32_t zwd = (zlo & ~zm2) | (zhi & zm2);
        const uint32_t z = (zwd >> (4 * (g & 7))) & 15u;
        const _Float16 zb = static_cast<_Float16>(1024.0f + static_cast<float>(z));
        zz[j] = h2_t{zb, zb};
        const size_t si = nn * ng + g;
        const int sp = static_cast<int>(si - scale_chunk(si));
        const uint32_t sm1 = 0u - static_cast<uint32_t>((sp >> 1) & 1), sm2 = 0u - static_cast<uint32_t>((sp >> 2) & 1);
        const uint32_t slo = (scv[j][0] & ~sm1) | (scv[j][1] & sm1), shi = (scv[j][2] & ~sm1) | (scv[j][3] & sm1);
        const uint32_t sd = (slo & ~sm2) | (shi & sm2);
        const _Float16 sh = bitcast<_Float16>(static_cast<uint16_t>(sd >> (16 * (sp & 1))));
        ss[j] = h2_t{sh, sh};
      }
      // the activation fragments of MFMA step st + 1 are read while step st runs
      h8_t a[2][TM];
      auto read_a = [&](int st, h8_t (&av)[TM]) __attribute__((always_inline)) {
        const int c = (8 * h + st) ^ swz_a;
#pragma unroll
        for (int i = 0; i < TM; ++i) av[i] = bitcast<h8_t>(As[32 * 16 * i + c]);
      };
      read_a(0, a[0]);
#pragma unroll
      for (int st = 0; st < 8; ++st) {
        if (st + 1 < 8) read_a(st + 1, a[(st + 1) & 1]);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          const h8_t b = w4_dequant8(bw[j][st], zz[j], ss[j]);
#pragma unroll
          for (int i = 0; i < TM; ++i)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[st & 1][i], b, acc[i][j], 0, 0, 0);
        }
      }
    };
    int kk = k0;
    while (sk_run_steps<0, NS>(step, kk, k1)) {
    }
    wait_vmcnt<0>();                                            // loads past the range end
    __syncthreads();

    // ---- finish the tile: block (i, j) holds column n0 + 32 TN wn + 32 j + col,
    // rows m0 + 32 TM wm + 32 i + 8 (r / 4) + 4 h + r % 4
    bool write = true;
    if (k0 != 0 || k1 != plan.ksteps) {
      const int first = sk_owner(plan, static_cast<long long>(t) * plan.ksteps);
      const int last = sk_owner(plan, static_cast<long long>(t + 1) * plan.ksteps - 1);
      auto part_of = [&](int q) {
        return ws + static_cast<size_t>(sk_slot(plan, q, t)) * (BM * BN) + (wv * TM * TN * 16) * 64 + lane;
      };
      {
        float* mine = part_of(p);
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
          for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) sk_store(mine + ((i * TN + j) * 16 + r) * 64, acc[i][j][r]);
      }
      write = sk_arrive_last(&counters[first], last - first, &s_last);
      if (write) {
        // every contributor's partial (this one's included, read back) in K
        // order, each contributor's loads in flight at once
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
          for (int j = 0; j < TN; ++j) acc[i][j] = f32x16_t{};
        for (int q = first; q <= last; ++q) {
          const float* other = part_of(q);
          float part[TM][TN][16];
#pragma unroll
          for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j)
#pragma unroll
              for (int r = 0; r < 16; ++r) part[i][j][r] = sk_load(other + ((i * TN + j) * 16 + r) * 64);
#pragma unroll
          for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j)
#pragma unroll
              for (int r = 0; r < 16; ++r) acc[i][j][r] += part[i][j][r];
        }
        if (tid == 0) sk_reset(&counters[first]);
      }
    }
    if (write) {
      const int mb = m0 + 32 * TM * wm + 4 * h;
      if (rowexp) {
        // row-scaled fp16 copy of bf16 activations: every row exponent loaded
        // first (clamped rows, no branches), then the exact rescale
        int ex[TM][16];
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
          for (int r = 0; r < 16; ++r) ex[i][r] = rowexp[min(mb + 32 * i + 8 * (r >> 2) + (r & 3), M - 1)];
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
          for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = ldexpf(acc[i][j][r], ex[i][r]);
      }
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int n = n0 + 32 * TN * wn + 32 * j + col;
        if (n >= N) continue;
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int m = mb + 32 * i + 8 * (r >> 2) + (r & 3);
            if (m < M) store_out<OUTK>(Y, static_cast<size_t>(m) * N + n, acc[i][j][r]);
          }
      }
    }
    u += k1 - k0;
  }
}

template <int WM, int WN, int TM, int TN, int NS, int OUTK, int WPE>
qlin_status launch_t(const W4Args& a, WsView ws, size_t* need, hipStream_t stream) {
  constexpr int BM = 32 * TM * WM, BN = 32 * TN * WN, threads = 64 * WM * WN;
  constexpr size_t lds = static_cast<size_t>(NS) * (BM * 256 + BN * 64 + BN * 32);
  static_assert(lds + 16 <= 160 * 1024, "LDS ring within the 160 KB of a CU");
  static_assert(WPE * 4 % (WM * WN) == 0, "whole workgroups per CU");
  using K_t = decltype(&w4_tile_kernel<WM, WN, TM, TN, NS, OUTK, WPE>);
  const K_t kern = &w4_tile_kernel<WM, WN, TM, TN, NS, OUTK, WPE>;
  // resident workgroups per CU, queried once per instantiation and process
  // (thread-safe initialisation of a function-local static), after raising the
  // dynamic LDS limit
  static const int occ = [kern] {
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                              static_cast<int>(lds));
    int o = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&o, kern, threads, lds) != hipSuccess || o <= 0) o = 1;
    return std::min(o, WPE * 4 / (WM * WN));
  }();
  const int tiles_m = (a.M + BM - 1) / BM;
  const int tiles_n = (a.N + BN - 1) / BN;
  const long long tiles = static_cast<long long>(tiles_m) * tiles_n;
  SkPlan plan;
  plan.ksteps = a.K / kKS;
  plan.units = tiles * plan.ksteps;
  plan.P = static_cast<int>(std::min<long long>(
      std::min<long long>(static_cast<long long>(occ) * device_cus(), kCounterSlots), plan.units));
  // at least kMinSteps K steps per workgroup; one workgroup per tile when the
  // tiles fill 2/3 of the slots
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
  hipLaunchKernelGGL(kern, dim3(plan.P), dim3(threads), lds, stream, static_cast<const uint16_t*>(a.X), a.M, a.K,
                     a.qweight, a.scales, a.qzeros, a.N, gsh, tiles_m, plan, a.Y, a.rowexp,
                     static_cast<float*>(ws.partials()), ws.counters());
  return QLIN_OK;
}

template <int WM, int WN, int TM, int TN, int NS, int WPE = WM * WN / 4>
qlin_status launch_o(const W4Args& a, WsView ws, size_t* need, hipStream_t stream) {
  if (a.y_dtype == QLIN_F16) return launch_t<WM, WN, TM, TN, NS, OUT_F16, WPE>(a, ws, need, stream);
  if (a.y_dtype == QLIN_BF16) return launch_t<WM, WN, TM, TN, NS, OUT_BF16, WPE>(a, ws, need, stream);
  return launch_t<WM, WN, TM, TN, NS, OUT_F32, WPE>(a, ws, need, stream);
}

}  // namespace

bool w4_tile_supported(const W4Args& a) {
  // The case this kernel wins, measured against the register-ring GEMM: more
  // than 64 rows (TM = 4) on layers short along K (K <= 16384) with at most 96
  // tiles of 256 columns (there both kernels use 128-column tiles): 7B-shaped
  // layers at 128 rows 95 -> 85 us for the three, the 8192 x 8192 layer at 256
  // rows 61 -> 57 us.  Narrower batches (fewer than 8 waves per CU on these
  // layers) and the 256-column, long-K layers stay on the register rings.
  const long long ng = a.K / a.G;
  if (!((a.G == 128 || a.G == 256) && a.K % a.G == 0 && static_cast<long long>(a.N) * ng >= 8 &&
        static_cast<long long>(a.N) * ((ng + 7) / 8) >= 4))
    return false;
  const long long tiles8 = static_cast<long long>((a.M + 127) / 128) * ((a.N + 255) / 256);
  return a.M > 64 && a.K <= 16384 && tiles8 <= 96;
}

qlin_status w4_tile_launch(const W4Args& a, WsView ws, size_t* need, hipStream_t stream) {
  // one row of 4 waves side by side along N (WM = 1): each wave owns all 128
  // rows, so every packed word is dequantized once per tile and feeds 4 matrix
  // instructions (a grid with WM > 1 dequantizes every word WM times and
  // measured 2x slower); three stages of 44 KB
  return launch_o<1, 4, 4, 1, 3>(a, ws, need, stream);
}

}  // namespace qlin
