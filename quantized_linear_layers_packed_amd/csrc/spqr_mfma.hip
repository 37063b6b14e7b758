// SpQR product for batches of 7..16 tokens (9..16 where N > K) on the matrix
// cores, gfx950.
//
// Y[m][n] = sum_g s_hat[n][g] * (sum_{k in g} x[m][k] q[n][k] - z_hat[n][g] * sum_{k in g} x[m][k])
//           + sum_{(n,k,v) in CSR} x[m][k] * v
//
// The SpQR bulletin ("İddia ve Gerçeklik") pairs a dense 3-bit matrix in groups
// of 16 with statistics that are themselves quantized, and a sparse fp16
// matrix of outliers applied to the same output.  With several tokens the
// GEMV's dot products (one v_dot2 per two weights per token) dominate; here
// each group's exact integer codes go through one v_mfma_f32_16x16x16_f16 for
// 16 tokens x 16 output columns, so the vector work per weight no longer grows
// with the batch (measured: flat from 2 to 16 tokens, ahead of the GEMV from 4
// tokens, or from 6 on layers with K >= 2N):
//   * P = sum_{k in g} x (1024 + q): the codes enter as fp16 1024 + q built by
//     a mask and an or (exact), and the 1024 is folded into the zero term
//     below; one MFMA per group and column tile, then acc += s_hat * P in fp32
//     (the statistics differ per group and column, so the rescale follows
//     every group);
//   * corr = sum_g s_hat (1024 + z_hat) * Xs[m][g], with Xs the group sums of x:
//     a v_mfma_f32_16x16x4_f32 per 4 groups, whose B operand is exactly the
//     statistic each lane decodes (lane quarter j: group 4h + j of its column),
//     so Y = acc - corr;
//   * within a chunk (32 codes in 3 words, two groups) lane quarter j holds
//     four codes of each group, two per mask-and-or, in the order the word
//     layout gives them; a prepass lays the activations out in that order
//     (Xp), with the group sums (Xs) and a transposed copy for the outliers
//     (XT), rows past M set to zero;
//   * one workgroup per 16 output columns; the K range is cut into super-steps
//     of 4 chunks and split over its KSW waves, each fetching its super-steps
//     D - 1 ahead into a register ring through buffer loads with scalar
//     offsets; the column's code bytes arrive once per wave (split over three
//     lane quarters) and reach the quarters that unpack them by ds_bpermute;
//   * the CSR entries of a column are dealt out over the workgroup's 4 KSW
//     lane quarters (x from XT for all 16 batch rows, the quarters' rows then
//     added so that each lane keeps its accumulator rows) into the same
//     accumulators, and the waves' parts are added in a fixed order through
//     LDS.  No atomics, results independent of timing.

#include <algorithm>
#include <type_traits>

#include "common.hpp"
#include "device.hpp"
#include "launch.hpp"
#include "splitk.hpp"

namespace qlin {

namespace {

typedef _Float16 h4_t __attribute__((ext_vector_type(4)));

constexpr int kPrepThreads = 64;          // small workgroups spread the short pass over more CUs

// Within-chunk offsets (k % 32) of the four codes lane quarter j unpacks for
// group a (codes 0..15 of the chunk) and group b (16..31), in unpack order: the
// low and high field of the first and-or, then of the second.
__host__ __device__ constexpr int order_a(int j, int e) {
  constexpr int t[4][4] = {{0, 5, 1, 6}, {2, 7, 3, 8}, {4, 9, 10, 13}, {11, 14, 12, 15}};
  return t[j][e];
}
__host__ __device__ constexpr int order_b(int j, int e) {
  constexpr int t[4][4] = {{16, 18, 17, 19}, {20, 25, 21, 26}, {22, 27, 23, 28}, {24, 29, 30, 31}};
  return t[j][e];
}

// One thread per (chunk c, batch row m < 16).  (Four threads per (chunk, row),
// one per lane quarter, measured slower: the pass is launch and latency bound.)
//   Xp [K/32][4][16] x 8 fp16: chunk c, quarter j, row m: order_a(j, 0..3), order_b(j, 0..3)
//   Xs [K/16][16] fp32: sum over the group's 16 x, in k order
//   XT [K][16] fp16
__global__ __launch_bounds__(kPrepThreads) void spqr_prep_kernel(const uint16_t* __restrict__ X, int M, int K,
                                                                 uint4* __restrict__ Xp, float* __restrict__ Xs,
                                                                 uint16_t* __restrict__ XT) {
  const int t = blockIdx.x * kPrepThreads + threadIdx.x;
  const int c = t >> 4, m = t & 15;
  if (c >= K / 32) return;
  uint16_t x[32];
  if (m < M) {
    const uint4* src = reinterpret_cast<const uint4*>(X + static_cast<size_t>(m) * K + 32 * c);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint4 v = src[i];
      const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        x[8 * i + 2 * h] = static_cast<uint16_t>(w[h] & 0xFFFFu);
        x[8 * i + 2 * h + 1] = static_cast<uint16_t>(w[h] >> 16);
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < 32; ++i) x[i] = 0;
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    uint32_t o[4];
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      o[e] = static_cast<uint32_t>(x[order_a(j, 2 * e)]) | (static_cast<uint32_t>(x[order_a(j, 2 * e + 1)]) << 16);
      o[2 + e] = static_cast<uint32_t>(x[order_b(j, 2 * e)]) | (static_cast<uint32_t>(x[order_b(j, 2 * e + 1)]) << 16);
    }
    Xp[(static_cast<size_t>(c) * 4 + j) * 16 + m] = make_uint4(o[0], o[1], o[2], o[3]);
  }
#pragma unroll
  for (int g = 0; g < 2; ++g) {
    float s = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) s += f16_bits_to_f32(x[16 * g + i]);
    Xs[(static_cast<size_t>(2 * c + g)) * 16 + m] = s;
  }
#pragma unroll
  for (int i = 0; i < 32; ++i) XT[(static_cast<size_t>(32 * c + i)) * 16 + m] = x[i];
}

// Raw buffer resource over `bytes` bytes at p (gfx9 descriptor word 3 for
// untyped 32-bit accesses).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, static_cast<int>(bytes), 0x00020000);
}

// fp16 pair (1024 + c_lo, 1024 + c_hi) of field f (bits 3f..3f+2) of both
// halves of w, for a field index held in a register (shift amount 3f).  Plain
// operations, not the inline-asm v_and_or_b32 of the GEMV kernels: with the
// asm form in this kernel's register ring the outputs were wrong whenever a
// ring slot was refilled (results became right once the asm was replaced,
// with no other change).
__device__ __forceinline__ uint32_t pair_at(uint32_t w, uint32_t shift) {
  return ((w >> shift) & 0x00070007u) | 0x64006400u;
}

// Everything a super-step (4 chunks = 8 groups of the wave's 16 columns) reads
// from memory.  The column's 48 code bytes are loaded once, split over lane
// quarters 0..2 (16 bytes each; quarter 3 repeats quarter 2's), and handed to
// the quarters that need them with ds_bpermute, so every load instruction
// brings 768 distinct bytes instead of four copies of 192.
template <int CT>
struct SuperStep {
  uint4 cw[CT];          // code bytes 16 min(j, 2) .. +15 of the super-step, this lane's column of tile c
  uint32_t st[CT][3];    // first-level statistic codes of the block (16 groups)
  uint2 ss[CT];          // second-level statistics of the block (4 fp16)
  uint4 xa[4];           // operand fragments of the 4 chunks (row r16, quarter j), shared by the tiles
  float xs[2];           // group sums of groups 8u + j and 8u + 4 + j, row r16
};

template <int KSW, int D, int CT, int OUTK>
__global__ __launch_bounds__(64 * KSW) void spqr_mfma_kernel(
    const uint32_t* codes, const uint32_t* stats1, const uint16_t* stats2, const int32_t* row_ptr,
    const int32_t* col_idx, const uint16_t* vals, const uint4* Xp, const float* Xs, const uint16_t* XT, int M, int K,
    int N, void* Y) {
  __shared__ f32x4_t red[KSW][CT][64];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r16 = lane & 15, j = lane >> 4;      // MFMA: A row / B,D column = r16; k quarter / D row quarter = j
  const int n0 = blockIdx.x * 16 * CT;
  const int nchunk = K >> 5, nblk = K >> 8;
  const int nsup = K >> 7;                       // super-steps of 4 chunks
  const int u0 = (wv * nsup) / KSW, u1 = ((wv + 1) * nsup) / KSW;

  // Per-lane unpack plan of quarter j: the field (shift 3f) of each of its two
  // and-ors per group, in the order of order_a / order_b.
  const uint32_t sa0 = j == 0 ? 0u : j == 1 ? 6u : j == 2 ? 12u : 3u;      // group a, first and-or
  const uint32_t sa1 = j == 0 ? 3u : j == 1 ? 9u : j == 2 ? 0u : 6u;       // group a, second
  const uint32_t sb0 = j == 0 ? 9u : j == 1 ? 0u : j == 2 ? 6u : 12u;      // group b, first
  const uint32_t sb1 = j == 0 ? 12u : j == 1 ? 3u : 9u;                    // group b, second (j = 3: spare bits)
  const uint32_t m3 = j == 3 ? ~0u : 0u;                                   // lane quarter 3

  int ncol[CT];
#pragma unroll
  for (int c = 0; c < CT; ++c) ncol[c] = min(n0 + 16 * c + r16, N - 1);
  // Buffer loads: each array is one resource (base and byte size in scalar
  // registers); a lane's loop-invariant byte offset is its VGPR operand and the
  // super-step's part is the wave-uniform scalar offset, so the loop keeps no
  // per-lane address arithmetic (whose temporaries the register allocator would
  // place in registers of loads still in flight, draining the ring).  Offsets
  // past an array's size read zeros instead of faulting.
  const __amdgpu_buffer_rsrc_t rc = make_rsrc(codes, static_cast<uint32_t>(N) * static_cast<uint32_t>(nchunk * 12));
  const __amdgpu_buffer_rsrc_t rs1 = make_rsrc(stats1, static_cast<uint32_t>(N) * static_cast<uint32_t>(nblk * 12));
  const __amdgpu_buffer_rsrc_t rs2 = make_rsrc(stats2, static_cast<uint32_t>(N) * static_cast<uint32_t>(nblk * 8));
  const __amdgpu_buffer_rsrc_t rxp = make_rsrc(Xp, static_cast<uint32_t>(K) * 32u);
  const __amdgpu_buffer_rsrc_t rxs = make_rsrc(Xs, static_cast<uint32_t>(K) * 4u);
  int voff_c[CT], voff_s1[CT], voff_s2[CT];
#pragma unroll
  for (int c = 0; c < CT; ++c) {
    voff_c[c] = ncol[c] * (nchunk * 12) + 16 * min(j, 2);      // code bytes of this lane's column and quarter
    voff_s1[c] = ncol[c] * (nblk * 12);
    voff_s2[c] = ncol[c] * (nblk * 8);
  }
  const int voff_xp = (j * 16 + r16) * 16;
  const int voff_xs = (j * 16 + r16) * 4;

  f32x4_t acc[CT], corr[CT];
#pragma unroll
  for (int c = 0; c < CT; ++c) acc[c] = corr[c] = f32x4_t{};

  // every load of a super-step, unconditional (super-steps past the range re-read its last)
  auto load = [&](int u, SuperStep<CT>& d) __attribute__((always_inline)) {
    const int blk = u >> 1;
#pragma unroll
    for (int c = 0; c < CT; ++c) {
      d.cw[c] = bitcast<uint4>(__builtin_amdgcn_raw_buffer_load_b128(rc, voff_c[c], 48 * u, 0));
      const u32x4_t st = __builtin_amdgcn_raw_buffer_load_b128(rs1, voff_s1[c], 12 * blk, 0);
      d.st[c][0] = st[0];
      d.st[c][1] = st[1];
      d.st[c][2] = st[2];
      d.ss[c] = bitcast<uint2>(__builtin_amdgcn_raw_buffer_load_b64(rs2, voff_s2[c], 8 * blk, 0));
    }
#pragma unroll
    for (int t = 0; t < 4; ++t)
      d.xa[t] = bitcast<uint4>(__builtin_amdgcn_raw_buffer_load_b128(rxp, voff_xp, (4 * u + t) * 1024, 0));
#pragma unroll
    for (int h = 0; h < 2; ++h)
      d.xs[h] = bitcast<float>(__builtin_amdgcn_raw_buffer_load_b32(rxs, voff_xs, (8 * u + 4 * h) * 64, 0));
  };

  auto compute = [&](int u, const SuperStep<CT>& d) __attribute__((always_inline)) {
    const int q = u & 1;                         // which half of the block
    float SSs[CT], ZSs[CT], SSz[CT], ZSz[CT];
    uint32_t cwv[CT][4];
#pragma unroll
    for (int c = 0; c < CT; ++c) {
      SSs[c] = f16_bits_to_f32(static_cast<uint16_t>(d.ss[c].x & 0xFFFFu));
      ZSs[c] = f16_bits_to_f32(static_cast<uint16_t>(d.ss[c].x >> 16));
      SSz[c] = f16_bits_to_f32(static_cast<uint16_t>(d.ss[c].y & 0xFFFFu));
      ZSz[c] = f16_bits_to_f32(static_cast<uint16_t>(d.ss[c].y >> 16));
      cwv[c][0] = d.cw[c].x;
      cwv[c][1] = d.cw[c].y;
      cwv[c][2] = d.cw[c].z;
      cwv[c][3] = d.cw[c].w;
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      // statistics of group 8q + 4h + j of the block (this lane's column):
      // 6-bit field at bit 6 (8q + 4h + j) of the block's 96-bit stream
      const int bit = 6 * (8 * q + 4 * h + j);
      const uint32_t sh = static_cast<uint32_t>(bit & 31);
      float s_hat[CT];
#pragma unroll
      for (int c = 0; c < CT; ++c) {
        // the word holding the field's low bit and the next one (a field at
        // bit >= 64 ends within the last word: 6 * 15 + 6 = 96); words selected
        // first, then one funnel shift, so no lane takes a branch
        // (copied to locals first: a select between elements of the ring
        // became a dynamic index into it, which put the whole ring in scratch)
        const uint32_t t0 = d.st[c][0], t1 = d.st[c][1], t2 = d.st[c][2];
        const uint32_t lo = bit < 32 ? t0 : bit < 64 ? t1 : t2;
        const uint32_t hi = bit < 32 ? t1 : t2;
        const uint32_t f = __builtin_amdgcn_alignbit(hi, lo, sh) & 63u;
        s_hat[c] = SSs[c] * (static_cast<float>(f & 7u) - ZSs[c]);
        const float z_hat = SSz[c] * (static_cast<float>(f >> 3) - ZSz[c]);
        corr[c] = __builtin_amdgcn_mfma_f32_16x16x4f32(d.xs[h], s_hat[c] * (1024.0f + z_hat), corr[c], 0, 0, 0);
      }
#pragma unroll
      for (int cc = 0; cc < 2; ++cc) {
        const int t = 2 * h + cc;                // chunk of the super-step
        // its words 3t .. 3t+2 from the lane quarters that loaded them
        uint32_t w[CT][3];
#pragma unroll
        for (int c = 0; c < CT; ++c)
#pragma unroll
          for (int e = 0; e < 3; ++e) {
            const int wi = 3 * t + e;
            w[c][e] = static_cast<uint32_t>(
                __builtin_amdgcn_ds_bpermute(4 * (r16 + 16 * (wi >> 2)), static_cast<int>(cwv[c][wi & 3])));
          }
#pragma unroll
        for (int ab = 0; ab < 2; ++ab) {
          const uint2 av = ab ? make_uint2(d.xa[t].z, d.xa[t].w) : make_uint2(d.xa[t].x, d.xa[t].y);
#pragma unroll
          for (int c = 0; c < CT; ++c) {
            uint32_t p0, p1;
            if (ab == 0) {                       // group a: words 0 / 1
              p0 = pair_at(j < 3 ? w[c][0] : w[c][1], sa0);
              p1 = pair_at(j < 2 ? w[c][0] : w[c][1], sa1);
            } else {                             // group b: words 1 / 2, spare bits
              p0 = pair_at(j == 0 ? w[c][1] : w[c][2], sb0);
              const uint32_t sp0 = ((w[c][0] >> 15) & 0x00010001u) | 0x64006400u;
              const uint32_t sp1 = ((w[c][1] >> 14) & 0x00020002u) | sp0;
              const uint32_t spare = ((w[c][2] >> 13) & 0x00040004u) | sp1;
              // quarter 3 takes the spare bits: a bitwise select (one v_bfi),
              // not a per-lane branch
              const uint32_t reg = pair_at(j == 0 ? w[c][1] : w[c][2], sb1);
              p1 = (spare & m3) | (reg & ~m3);
            }
            const f32x4_t P = __builtin_amdgcn_mfma_f32_16x16x16f16(bitcast<h4_t>(av),
                                                                    bitcast<h4_t>(make_uint2(p0, p1)), f32x4_t{}, 0, 0, 0);
            // s_hat of group 4h + 2cc + ab of the super-step: decoded by quarter 2cc + ab
            const float sg = bitcast<float>(
                __builtin_amdgcn_ds_bpermute(4 * (r16 + 16 * (2 * cc + ab)), bitcast<int>(s_hat[c])));
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[c][i] = fmaf(sg, P[i], acc[c][i]);
          }
        }
      }
    }
  };

  // Outlier pass (after the dense loop): CSR bounds, then rounds of kU entries
  // per lane quarter, each round's x loads issued before the next round's
  // entries are fetched and before its own math.  (Fetching the bounds and the
  // first round ahead of the dense loop kept 10 more registers live through it,
  // 3 waves per SIMD instead of 4, and measured 10% slower.)
  constexpr int kU = 4;
  constexpr int kStreams = 4 * KSW;              // lane quarters of the workgroup, one entry stream each
  int e1[CT], ef[CT], kk0[CT][kU];
  float v0[CT][kU];

  auto csr_round = [&](int c, int e, int (&kk)[kU], float (&v)[kU]) __attribute__((always_inline)) {
#pragma unroll
    for (int uu = 0; uu < kU; ++uu) {
      const int eu = e + kStreams * uu;
      const int ec = min(eu, e1[c] - 1);
      kk[uu] = col_idx[ec];
      v[uu] = eu < e1[c] ? f16_bits_to_f32(vals[ec]) : 0.0f;
    }
  };
  auto csr_first = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int c = 0; c < CT; ++c) {
      if (ef[c] < e1[c]) {
        csr_round(c, ef[c], kk0[c], v0[c]);
      } else {
#pragma unroll
        for (int uu = 0; uu < kU; ++uu) {
          kk0[c][uu] = 0;
          v0[c][uu] = 0.0f;
        }
      }
    }
  };

  if (u0 < u1) {
    const int ulast = u1 - 1;
    SuperStep<CT> ring[D];
    // the prologue's slots are issued in slot order (no interleaving by the
    // scheduler): the wait counts at the loop head hold for this entry and for
    // the back edge alike only if both leave the slots' loads in that order
#pragma unroll
    for (int i = 0; i < D - 1; ++i) {
      load(min(u0 + i, ulast), ring[i]);
      __builtin_amdgcn_sched_barrier(0);
    }
    // super-step u in slot S: fetch u + D - 1 into the slot u - 1 freed, then compute u
    auto step = [&](auto slot_c, int u) __attribute__((always_inline)) {
      constexpr int S = decltype(slot_c)::value;
      constexpr int SF = (S + D - 1) % D;
      load(min(u + D - 1, ulast), ring[SF]);
      __builtin_amdgcn_sched_barrier(0);
      compute(u, ring[S]);
    };
    sk_ring_steps<D>(step, u0, u1);
  }

  // outliers, tile by tile: lane quarter j of wave wv takes CSR entries
  // (4 wv + j) + 4 KSW i of its column, for all 16 batch rows (x from XT), four
  // entries per round with every load issued first; the quarters' partial rows
  // are then added so that quarter j keeps rows 4j .. 4j+3 (the accumulator
  // layout)
#pragma unroll
  for (int c = 0; c < CT; ++c) {
    const int eb = row_ptr[ncol[c]];
    e1[c] = n0 + 16 * c + r16 < N ? row_ptr[ncol[c] + 1] : eb;
    ef[c] = eb + 4 * wv + j;                     // this quarter's first entry
  }
  csr_first();
#pragma unroll
  for (int c = 0; c < CT; ++c) {
    float o[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) o[r] = 0.0f;
    int kk[kU];
    float v[kU];
#pragma unroll
    for (int uu = 0; uu < kU; ++uu) {
      kk[uu] = kk0[c][uu];
      v[uu] = v0[c][uu];
    }
    for (int e = ef[c]; e < e1[c];) {
      uint4 xt[kU][2];
#pragma unroll
      for (int uu = 0; uu < kU; ++uu) {
        const uint4* src = reinterpret_cast<const uint4*>(XT + static_cast<size_t>(kk[uu]) * 16);
        xt[uu][0] = src[0];
        xt[uu][1] = src[1];
      }
      float vc[kU];
#pragma unroll
      for (int uu = 0; uu < kU; ++uu) vc[uu] = v[uu];
      // the next round's entries, loaded before this round's math (unconditional:
      // inside the loop e1 - 1 is a valid entry, and entries past e1 weigh 0)
      e += kStreams * kU;
      csr_round(c, e, kk, v);
#pragma unroll
      for (int uu = 0; uu < kU; ++uu)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const uint32_t ww[4] = {xt[uu][hh].x, xt[uu][hh].y, xt[uu][hh].z, xt[uu][hh].w};
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            o[8 * hh + 2 * i] = fmaf(vc[uu], f16_bits_to_f32(static_cast<uint16_t>(ww[i] & 0xFFFFu)), o[8 * hh + 2 * i]);
            o[8 * hh + 2 * i + 1] = fmaf(vc[uu], f16_bits_to_f32(static_cast<uint16_t>(ww[i] >> 16)), o[8 * hh + 2 * i + 1]);
          }
        }
    }
    // quarters 0,1 keep rows 0..7 and quarters 2,3 rows 8..15, then even quarters
    // the first four of those, odd quarters the last four
    const bool upper = j >= 2;
    float k8[8];
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const float send = upper ? o[r] : o[r + 8];
      const float keep = upper ? o[r + 8] : o[r];
      k8[r] = keep + __shfl_xor(send, 32, 64);
    }
    const bool odd = (j & 1) != 0;
    f32x4_t out4;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float send = odd ? k8[r] : k8[r + 4];
      const float keep = odd ? k8[r + 4] : k8[r];
      out4[r] = keep + __shfl_xor(send, 16, 64);
    }
    red[wv][c][lane] = (acc[c] - corr[c]) + out4;
  }
  __syncthreads();
  if (wv == 0) {
#pragma unroll
    for (int c = 0; c < CT; ++c) {
      f32x4_t tot = red[0][c][lane];
#pragma unroll
      for (int w2 = 1; w2 < KSW; ++w2) tot += red[w2][c][lane];
      const int n = n0 + 16 * c + r16;
      if (n < N) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int m = 4 * j + i;
          if (m < M) store_out<OUTK>(Y, static_cast<size_t>(m) * N + n, tot[i]);
        }
      }
    }
  }
}

template <int KSW, int D, int CT>
void launch_t(const SpqrArgs& a, const SpqrPrep& p, hipStream_t stream) {
  const dim3 grid((a.N + 16 * CT - 1) / (16 * CT));
  if (a.y_dtype == QLIN_F16)
    hipLaunchKernelGGL((spqr_mfma_kernel<KSW, D, CT, OUT_F16>), grid, dim3(64 * KSW), 0, stream, a.codes, a.stats1,
                       a.stats2, a.row_ptr, a.col_idx, a.vals, p.Xp, p.Xs, p.XT, a.M, a.K, a.N, a.Y);
  else
    hipLaunchKernelGGL((spqr_mfma_kernel<KSW, D, CT, OUT_F32>), grid, dim3(64 * KSW), 0, stream, a.codes, a.stats1,
                       a.stats2, a.row_ptr, a.col_idx, a.vals, p.Xp, p.Xs, p.XT, a.M, a.K, a.N, a.Y);
}

}  // namespace

size_t spqr_prep_bytes(int K) {
  return ws_round(static_cast<size_t>(K) * 32) + ws_round(static_cast<size_t>(K) * 4) +
         ws_round(static_cast<size_t>(K) * 32);
}

SpqrPrep spqr_prep_view(char* base, int K) {
  SpqrPrep p;
  p.Xp = reinterpret_cast<uint4*>(base);
  p.Xs = reinterpret_cast<float*>(base + ws_round(static_cast<size_t>(K) * 32));
  p.XT = reinterpret_cast<uint16_t*>(base + ws_round(static_cast<size_t>(K) * 32) + ws_round(static_cast<size_t>(K) * 4));
  return p;
}

void spqr_mfma_launch(const SpqrArgs& a, const SpqrPrep& p, hipStream_t stream) {
  const int threads = (a.K / 32) * 16;
  hipLaunchKernelGGL(spqr_prep_kernel, dim3((threads + kPrepThreads - 1) / kPrepThreads), dim3(kPrepThreads), 0,
                     stream, a.X, a.M, a.K, const_cast<uint4*>(p.Xp), const_cast<float*>(p.Xs),
                     const_cast<uint16_t*>(p.XT));
  // Two column tiles per wave where rows are long against the column count
  // (one activation fragment then feeds two tiles, halving the activation
  // reads, at 165 VGPRs: one workgroup per CU): the 6656 x 17920 layer
  // measured 63.7 -> 55.5 us at M = 8 / 16, while the 17920 x 6656 layer
  // (57 -> 64) and the square one keep one tile and two workgroups per CU.
  if (a.K >= 2 * a.N) launch_t<8, 2, 2>(a, p, stream);
  else launch_t<8, 2, 1>(a, p, stream);
}

}  // namespace qlin
