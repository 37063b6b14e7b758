// Decoding of the SpQR 32-code chunk layout shared by the GEMV kernels.
//
// A chunk holds the 3-bit codes of 32 consecutive weights of one row (two
// groups of 16) in three 32-bit words.  Field i (bits 3i .. 3i+2) of the low
// and of the high 16-bit half of a word hold two codes of the same group, so
// one shift and one v_and_or_b32 give an fp16 pair (1024 + 8 c_lo,
// 1024 + 8 c_hi), exact, ready for packed fp16 arithmetic against activation
// pairs staged in the same order (pair_lo / pair_hi give the order).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "device.hpp"

namespace qlin {

// fp16 pair (1024 + 8 c_lo, 1024 + 8 c_hi) from field i of both halves of w:
// a shift and one v_and_or_b32.
__device__ __forceinline__ uint32_t field_pair(uint32_t w, int i) {
  constexpr uint32_t MAGIC = 0x64006400u;
  const uint32_t mask = 0x00380038u;
  switch (i) {
    case 0: return and_or(w << 3, mask, MAGIC);
    case 1: return and_or(w, mask, MAGIC);
    case 2: return and_or(w >> 3, mask, MAGIC);
    case 3: return and_or(w >> 6, mask, MAGIC);
    default: return and_or(w >> 9, mask, MAGIC);
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
  // (b14, b15) from the spare bits 15 / 31 of the three words
  const uint32_t t0 = and_or(w0 >> 12, 0x00080008u, 0x64006400u);
  const uint32_t t1 = and_or_v(w1 >> 11, 0x00100010u, t0);
  p[15] = and_or_v(w2 >> 10, 0x00200020u, t1);
}

// Within-chunk offsets (k % 32) of the two codes of pair p.
__host__ __device__ constexpr int pair_lo(int p) {
  return p < 5 ? p : p < 8 ? p + 5 : p == 8 ? 16 : p == 9 ? 17 : p < 15 ? p + 10 : 30;
}
__host__ __device__ constexpr int pair_hi(int p) {
  return p < 5 ? p + 5 : p < 8 ? p + 8 : p == 8 ? 18 : p == 9 ? 19 : p < 15 ? p + 15 : 31;
}

// Inverse: (pair << 1 | half) of within-chunk offset o, without branches (it
// runs once per outlier, in divergent lanes): the pair is o - d(o), d a step
// function rising by 5, 3, 2, 5 and 1 at offsets 5, 13, 18, 25 and 31, and the
// offsets held in high halves are the set bits of 0xBE0CE3E0 (5-9, 13-15,
// 18-19, 25-29 and 31), as pair_lo / pair_hi above lay them out.
__device__ __forceinline__ int pair_slot(int o) {
  const int d = (o >= 5 ? 5 : 0) + (o >= 13 ? 3 : 0) + (o >= 18 ? 2 : 0) + (o >= 25 ? 5 : 0) + (o >= 31 ? 1 : 0);
  const int half = static_cast<int>((0xBE0CE3E0u >> o) & 1u);
  return ((o - d) << 1) | half;
}

__device__ __forceinline__ uint32_t half_of(const uint32_t u[16], int o) {
  return (u[o >> 1] >> (16 * (o & 1))) & 0xFFFFu;
}

}  // namespace qlin
