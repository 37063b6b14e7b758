// Large-tile MFMA GEMM over byte rows, shared by the int8 GEMM of the W8A8 path
// and the dense fp16 GEMM (gfx950).
//
// Y[m][n] = epilogue(sum_k A[m][k] B[n][k]), A [M][Kb] and B [N][Kb] as rows of
// Kb bytes.  v_mfma_i32_32x32x32_i8 and v_mfma_f32_32x32x16_f16 read their
// operands in the same byte layout (lane l: row l % 32, bytes 16 (l / 32) .. +15
// of the instruction's 32-byte K slice) and write the same 32 x 32 output
// layout, so one tiling serves both; the operation type supplies the
// instruction, the accumulator and the epilogue.
//
// A WM x WN grid of waves, each owning 32 TM rows x 32 TN columns (TM x TN
// blocks of 32 x 32), so a tile is BM = 32 TM WM rows x BN = 32 TN WN columns and
// every operand byte brought into LDS feeds BN (or BM) multiply-adds.  K steps
// of BK bytes (64 or 128), rows of BK bytes in LDS with their 16-byte chunks
// XOR-swizzled by row so that the 16 rows one quarter-wave of an MFMA operand
// read touches fall in distinct banks; within a step, MFMA step st and lane
// half h use chunk (BK / 32) h + st of both operands (a fixed permutation of k,
// the same for A and B).  Both operands stream from HBM straight into an
// NS-stage LDS ring (direct-to-LDS loads, NS - 1 steps ahead, no registers
// involved), the swizzle realised by choosing which global chunk each lane
// fetches.  One explicit vmcnt wait and one barrier per step.  The (tile, K
// step) space is split evenly over the workgroups (stream-K, or one workgroup
// per tile when the tiles nearly fill the device); a tile shared by
// several workgroups is finished by the last to arrive: exact integer partials
// are added to its own, float partials are all summed in K order, so the
// result never depends on arrival order.
#pragma once

#include <algorithm>

#include "common.hpp"
#include "device.hpp"
#include "splitk.hpp"
#include "workspace.hpp"

namespace qlin {

// WPE: waves per SIMD the register budget is fitted to (WM WN / 4 per resident
// workgroup).
template <class Op, int WM, int WN, int TM, int TN, int BK, int NS, int OUTK, int WPE>
__global__ __launch_bounds__(64 * WM * WN) __attribute__((amdgpu_waves_per_eu(WPE, WPE)))
void tile_gemm_kernel(const char* __restrict__ A, const char* __restrict__ B, int M, int N, int Kb, int tiles_m,
                      SkPlan plan, Op op, void* __restrict__ Y, typename Op::part_t* __restrict__ ws,
                      int* __restrict__ counters) {
  using acc_t = typename Op::acc_t;
  using part_t = typename Op::part_t;
  constexpr int NW = WM * WN;
  constexpr int BM = 32 * TM * WM, BN = 32 * TN * WN;
  constexpr int CH = BK / 16;                                   // 16-byte chunks per row
  constexpr int RPI = 64 / CH;                                  // rows per direct-load instruction
  constexpr int RSH = RPI == 16 ? 2 : 1;                        // swizzle: chunk ^ (row >> RSH) % CH
  constexpr int KST = BK / 32;                                  // MFMA steps per K step
  constexpr int A_PIECES = BM * CH, B_PIECES = BN * CH;         // 16-byte pieces per stage
  constexpr int STAGE = A_PIECES + B_PIECES;
  constexpr int A_INS = BM / RPI / NW, B_INS = BN / RPI / NW;   // direct loads per wave per stage
  static_assert(BK == 64 || BK == 128, "K step of 64 or 128 bytes");
  static_assert(A_INS * RPI * NW == BM && B_INS * RPI * NW == BN, "row blocks split evenly over the waves");
  static_assert((NS - 2) * (A_INS + B_INS) < 64, "vmcnt range");
  extern __shared__ uint4 smem[];
  __shared__ int s_last;

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int wm = wv % WM, wn = wv / WM;
  const int col = lane & 31, h = lane >> 5;
  const int swz = (col >> RSH) & (CH - 1);                      // swizzle of every row this lane reads
  const int lrow = lane / CH, lpos = lane % CH;                 // this lane's piece in a direct load

  const int p = xcd_tile(blockIdx.x, gridDim.x);
  long long u = sk_begin(plan, p);
  const long long u_end = sk_begin(plan, p + 1);

  while (u < u_end) {
    const int t = static_cast<int>(u / plan.ksteps);
    const int k0 = static_cast<int>(u - static_cast<long long>(t) * plan.ksteps);
    const int k1 = static_cast<int>(std::min<long long>(plan.ksteps, k0 + (u_end - u)));
    const int klast = k1 - 1;
    const int m0 = (t % tiles_m) * BM;                          // M-blocks fastest: neighbours share B rows
    const int n0 = (t / tiles_m) * BN;

    // Direct loads of step s = min(j, klast) into slot j % NS.  Wave wv loads the
    // RPI-row blocks wv, wv + NW, ... of A and of B.  Rows past M / N read the
    // last row (their results are never stored); positions past the range re-read
    // its last step into slots no step of the range reads again.
    auto issue = [&](int j) {
      const int s = min(j, klast);
      uint4* slot = smem + static_cast<size_t>(j % NS) * STAGE;
#pragma unroll
      for (int q = 0; q < A_INS; ++q) {
        const int rb = wv + NW * q;
        const int row = RPI * rb + lrow;
        const int c = lpos ^ ((row >> RSH) & (CH - 1));         // logical chunk stored at this piece
        const int m = min(m0 + row, M - 1);
        dma16(A + static_cast<size_t>(m) * Kb + s * BK + 16 * c, slot + 64 * rb);
      }
#pragma unroll
      for (int q = 0; q < B_INS; ++q) {
        const int rb = wv + NW * q;
        const int row = RPI * rb + lrow;
        const int c = lpos ^ ((row >> RSH) & (CH - 1));
        const int nn = min(n0 + row, N - 1);
        dma16(B + static_cast<size_t>(nn) * Kb + s * BK + 16 * c, slot + A_PIECES + 64 * rb);
      }
    };

    acc_t acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) acc[i][j] = acc_t{};

    wait_vmcnt<0>();                                            // nothing but the ring in flight below
#pragma unroll
    for (int j = 0; j < NS - 1; ++j) issue(k0 + j);

    for (int kk = k0; kk < k1; ++kk) {
      wait_vmcnt<(NS - 2) * (A_INS + B_INS)>();                 // this wave's loads of step kk
      barrier_raw();                                            // everyone's; step kk - 1 finished
      issue(kk + NS - 1);
      const uint4* As = smem + static_cast<size_t>(kk % NS) * STAGE + (32 * TM * wm + col) * CH;
      const uint4* Bs = smem + static_cast<size_t>(kk % NS) * STAGE + A_PIECES + (32 * TN * wn + col) * CH;
      // the operands of MFMA step st + 1 are read from LDS while step st runs,
      // so no matrix instruction waits on a read issued just before it
      i32x4_t a[2][TM], b[2][TN];
      auto read = [&](int st, i32x4_t (&av)[TM], i32x4_t (&bv)[TN]) {
        const int c = (KST * h + st) ^ swz;
#pragma unroll
        for (int i = 0; i < TM; ++i) av[i] = bitcast<i32x4_t>(As[32 * CH * i + c]);
#pragma unroll
        for (int j = 0; j < TN; ++j) bv[j] = bitcast<i32x4_t>(Bs[32 * CH * j + c]);
      };
      read(0, a[0], b[0]);
#pragma unroll
      for (int st = 0; st < KST; ++st) {
        if (st + 1 < KST) read(st + 1, a[(st + 1) & 1], b[(st + 1) & 1]);
        __builtin_amdgcn_sched_barrier(0);                      // the next step's reads stay ahead of this one's MFMAs
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
          for (int j = 0; j < TN; ++j) acc[i][j] = Op::mfma(a[st & 1][i], b[st & 1][j], acc[i][j]);
      }
    }
    wait_vmcnt<0>();                                            // loads past the range end
    __syncthreads();

    // ---- finish the tile: block (i, j) of this wave holds column n0 + 32 TN wn + 32 j + col,
    // rows m0 + 32 TM wm + 32 i + 8 (r / 4) + 4 h + r % 4
    bool write = true;
    if (k0 != 0 || k1 != plan.ksteps) {
      const int first = sk_owner(plan, static_cast<long long>(t) * plan.ksteps);
      const int last = sk_owner(plan, static_cast<long long>(t + 1) * plan.ksteps - 1);
      // this wave's part of workgroup q's partial: block (i, j), register r at
      // ((i TN + j) 16 + r) 64 + lane
      auto part_of = [&](int q) {
        return ws + static_cast<size_t>(sk_slot(plan, q, t)) * (BM * BN) + (wv * TM * TN * 16) * 64 + lane;
      };
      {
        part_t* mine = part_of(p);
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
          for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) sk_store(mine + ((i * TN + j) * 16 + r) * 64, static_cast<part_t>(acc[i][j][r]));
      }
      write = sk_arrive_last(&counters[first], last - first, &s_last);
      if (write) {
        if constexpr (!Op::kExact) {
          // float partials: every contributor's (this one's included, read
          // back) summed in K order
#pragma unroll
          for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j) acc[i][j] = acc_t{};
        }
        for (int q = first; q <= last; ++q) {
          if (Op::kExact && q == p) continue;                   // integer partials: the others added to its own
          const part_t* other = part_of(q);
          // every load of a contributor's part in flight at once, then the
          // adds: one memory round trip per contributor, not one per block
          part_t part[TM][TN][16];
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
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int n = n0 + 32 * TN * wn + 32 * j + col;
        if (n >= N) continue;
#pragma unroll
        for (int i = 0; i < TM; ++i)
          op.template store<OUTK>(Y, M, N, m0 + 32 * TM * wm + 32 * i + 4 * h, n, acc[i][j]);
      }
    }
    u += k1 - k0;
  }
}

// Launch over a caller workspace: the plan gives every resident workgroup slot
// of the device (at most kCounterSlots) an equal share of the (tile, K step)
// units; need != NULL only reports the partial-tile bytes.  Kb % BK == 0.
template <class Op, int WM, int WN, int TM, int TN, int BK, int NS, int OUTK, int WPE = WM * WN / 4>
qlin_status tile_gemm_launch(const char* fn, const void* A, const void* B, int M, int N, int Kb, const Op& op,
                             void* Y, WsView ws, size_t* need, hipStream_t stream) {
  constexpr int BM = 32 * TM * WM, BN = 32 * TN * WN, threads = 64 * WM * WN;
  constexpr size_t lds = static_cast<size_t>(NS) * (BM + BN) * BK;
  static_assert(lds + 16 <= 160 * 1024, "LDS ring within the 160 KB of a CU");
  static_assert(WPE * 4 % (WM * WN) == 0, "whole workgroups per CU");
  using K_t = decltype(&tile_gemm_kernel<Op, WM, WN, TM, TN, BK, NS, OUTK, WPE>);
  const K_t kern = &tile_gemm_kernel<Op, WM, WN, TM, TN, BK, NS, OUTK, WPE>;
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
  const int tiles_m = (M + BM - 1) / BM;
  const int tiles_n = (N + BN - 1) / BN;
  const long long tiles = static_cast<long long>(tiles_m) * tiles_n;
  SkPlan plan;
  plan.ksteps = Kb / BK;
  plan.units = tiles * plan.ksteps;
  plan.P = static_cast<int>(std::min<long long>(
      std::min<long long>(static_cast<long long>(occ) * device_cus(), kCounterSlots), plan.units));
  // One workgroup per tile, no K split, when the tiles fill at least 2/3 of
  // the resident slots: the split-K hand-off (partials written, counted, read
  // back) costs more than the idle third.  Measured on the int8 product
  // 256 x 11008 x 4096 (172 tiles of 128 x 128, 256 slots): 29.5 -> 25.6 us;
  // at half fill (128 tiles of 128 x 64 on 4096 x 4096) the split stays ahead.
  if (tiles <= plan.P && 3 * tiles >= 2 * static_cast<long long>(plan.P)) plan.P = static_cast<int>(tiles);
  const size_t partial_bytes = static_cast<size_t>(2) * plan.P * BM * BN * sizeof(typename Op::part_t);
  if (need) {
    *need = partial_bytes;
    return QLIN_OK;
  }
  if (ws.bytes < kCounterBytes + partial_bytes)
    return fail(QLIN_EINVAL, std::string(fn) + ": workspace too small for the split-K GEMM");
  hipLaunchKernelGGL(kern, dim3(plan.P), dim3(threads), lds, stream, static_cast<const char*>(A),
                     static_cast<const char*>(B), M, N, Kb, tiles_m, plan, op, Y,
                     static_cast<typename Op::part_t*>(ws.partials()), ws.counters());
  return QLIN_OK;
}

}  // namespace qlin
