// Device-side types and helpers for the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace qlin {

typedef _Float16 h2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf2_t __attribute__((ext_vector_type(2)));
typedef _Float16 h8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef int i32x4_t __attribute__((ext_vector_type(4)));
typedef int i32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// 128-bit streaming load (marked non-temporal: weights are read exactly once).
__device__ __forceinline__ uint4 load_stream16(const void* p) {
  const u32x4_t v = __builtin_nontemporal_load(static_cast<const u32x4_t*>(p));
  return make_uint4(v[0], v[1], v[2], v[3]);
}

template <typename To, typename From>
__device__ __forceinline__ To bitcast(const From& f) {
  static_assert(sizeof(To) == sizeof(From), "size mismatch");
  return __builtin_bit_cast(To, f);
}

// fp32 += a.lo*b.lo + a.hi*b.hi for two packed fp16 / bf16 pairs (v_dot2).
__device__ __forceinline__ float dot2_f16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2(bitcast<h2_t>(a), bitcast<h2_t>(b), c, false);
}
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(bitcast<bf2_t>(a), bitcast<bf2_t>(b), c, false);
}

__device__ __forceinline__ float f16_bits_to_f32(uint16_t h) { return static_cast<float>(bitcast<_Float16>(h)); }
__device__ __forceinline__ float bf16_bits_to_f32(uint16_t h) { return bitcast<float>(static_cast<uint32_t>(h) << 16); }

// Output element stores for the three output dtypes (round to nearest even).
enum OutKind { OUT_F16 = 0, OUT_BF16 = 1, OUT_F32 = 2 };

template <int OK>
__device__ __forceinline__ void store_out(void* Y, size_t idx, float v) {
  if constexpr (OK == OUT_F16) {
    static_cast<_Float16*>(Y)[idx] = static_cast<_Float16>(v);
  } else if constexpr (OK == OUT_BF16) {
    static_cast<__bf16*>(Y)[idx] = static_cast<__bf16>(v);
  } else {
    static_cast<float*>(Y)[idx] = v;
  }
}

// XCD-aware tile order.  Workgroups are dispatched round-robin over the 8 XCDs
// (each with its own L2), so linear workgroup b lands on XCD b % 8.  This maps
// b to a tile index such that every XCD owns one contiguous range of tiles;
// with tiles numbered M-block fastest, the workgroups of one XCD share weight
// columns and neighbouring activation rows in their L2.  Bijective on [0, T).
__device__ __forceinline__ int xcd_tile(int b, int T) {
  constexpr int X = 8;
  const int per = T / X, rem = T % X;
  const int xcd = b % X, slot = b / X;
  const int base = xcd < rem ? xcd * (per + 1) : rem * (per + 1) + (xcd - rem) * per;
  return base + slot;
}

// ---------------------------------------------------------------------------
// Direct global -> LDS loads (gfx950 global_load_lds_dwordx4).  Each lane reads
// 16 bytes at its own global address; the wave's 64 pieces land contiguously at
// lds_wave_base + 16 * lane (the LDS address must be the same for the whole
// wave).  These count in vmcnt like ordinary loads but write no VGPR, so a ring
// of stages in LDS carries no loop state in registers.
typedef __attribute__((address_space(3))) void* lds_void_ptr;
typedef __attribute__((address_space(1))) void* global_void_ptr;

__device__ __forceinline__ void dma16(const void* global_src, void* lds_wave_base) {
  __builtin_amdgcn_global_load_lds((global_void_ptr)(const_cast<void*>(global_src)), (lds_void_ptr)(lds_wave_base),
                                   16, 0, 0);
}

// s_waitcnt vmcnt(N) (expcnt and lgkmcnt untouched).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Workgroup barrier without the memory fence of __syncthreads (which would
// also wait for every outstanding direct-to-LDS load); the empty asm keeps the
// compiler from moving memory accesses across it.
__device__ __forceinline__ void barrier_raw() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Sum over the 64 lanes of a wavefront.
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  return v;
}

// ---------------------------------------------------------------------------
// 4-bit codes -> packed 16-bit pairs without per-code conversion.
//
// A 32-bit word holds codes n0..n7 (n_j in bits 4j..4j+3).  Four and-or steps
// give four registers with the pairs (n_j, n_{j+4}), j = 0..3, placed inside
// the mantissa of a 16-bit float whose exponent makes the code an exact
// integer offset: fp16 0x6400 | (q << 4) = 1024 + 16 q, bf16 0x4300 | (q << 3)
// = 128 + 8 q.  A dot product against activation pairs (x_j, x_{j+4}) then
// yields B * sum(x) + D * sum(x q), from which sum(x q) is recovered with the
// separately accumulated sum(x).

// (a & m) | c in one v_and_or_b32.  gfx9 reads at most one scalar operand per
// VALU instruction, so the mask is kept in a VGPR and the magic constant is the
// scalar operand; left to itself the compiler splits this into and + or.
__device__ __forceinline__ uint32_t and_or(uint32_t a, uint32_t m, uint32_t c) {
  uint32_t r;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(m), "s"(c));
  return r;
}

// Same with the or-operand in a VGPR.
__device__ __forceinline__ uint32_t and_or_v(uint32_t a, uint32_t m, uint32_t c) {
  uint32_t r;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(m), "v"(c));
  return r;
}

// Unpacked codes for the GEMV's fp16 dot products.  Register j of a word holds
// the codes of k = j and k = j + 4 (the pairs the activation staging builds).
//
// fp16 activations: one shift and four and-ors.  Registers 0 and 2 take the
// low nibble of each byte into mantissa bits 0..3 of 1024.0 (value 1024 + q),
// registers 1 and 3 the high nibble into bits 4..7 (value 1024 + 16 q).  The
// staging divides the activations paired with registers 1 and 3 by 16 (exact
// in fp16 above 2^-10) so one dot-product chain gives
//   acc = sum x q + 1024 sum_{0,2} x + 64 sum_{1,3} x,
// and a chunk's sum x (q - z) = acc - (E + z S), E = 1024 (se + so),
// S = se + 16 so with se / so the chunk's sums over registers 0, 2 / the scaled
// 1, 3 (staging computes both).
struct W4F16 {
  static constexpr uint32_t MAGIC = 0x64006400u;
  __device__ __forceinline__ static void unpack(uint32_t w, uint32_t p[4]) {
    const uint32_t lo = 0x000F000Fu, hi = 0x00F000F0u;
    const uint32_t w8 = w >> 8;
    p[0] = and_or(w, lo, MAGIC);
    p[1] = and_or(w, hi, MAGIC);
    p[2] = and_or(w8, lo, MAGIC);
    p[3] = and_or(w8, hi, MAGIC);
  }
  __device__ __forceinline__ static uint32_t code_of(int j, uint16_t half) {
    return (j & 1) ? (half >> 4) & 15u : half & 15u;
  }
  __device__ __forceinline__ static float dot(uint32_t a, uint32_t b, float c) { return dot2_f16(a, b, c); }
  // scale the odd pairs by 1/16 and accumulate (se, so) with dot products by (1, 1)
  __device__ __forceinline__ static void stage(uint32_t P[4], float2& es) {
    const h2_t sixteenth = {static_cast<_Float16>(0.0625f), static_cast<_Float16>(0.0625f)};
    P[1] = bitcast<uint32_t>(bitcast<h2_t>(P[1]) * sixteenth);
    P[3] = bitcast<uint32_t>(bitcast<h2_t>(P[3]) * sixteenth);
    es.x = dot2_f16(P[0], 0x3C003C00u, es.x);
    es.x = dot2_f16(P[2], 0x3C003C00u, es.x);
    es.y = dot2_f16(P[1], 0x3C003C00u, es.y);
    es.y = dot2_f16(P[3], 0x3C003C00u, es.y);
  }
  __device__ __forceinline__ static float2 sums(float2 es) {
    return make_float2(1024.0f * (es.x + es.y), fmaf(16.0f, es.y, es.x));
  }
  __device__ __forceinline__ static float finish(float acc, float2 es, float z) { return acc - fmaf(z, es.y, es.x); }
};

// bf16 activations: every code goes to mantissa bits 3..6 of 128.0 (value
// 128 + 8 q; a bf16 mantissa has no room for the high-nibble trick):
//   sum x (q - z) = acc / 8 - (16 + z) sum x.
struct W4BF16 {
  static constexpr uint32_t MAGIC = 0x43004300u, MASK = 0x00780078u;
  __device__ __forceinline__ static void unpack(uint32_t w, uint32_t p[4]) {
    const uint32_t mask = MASK;
    p[0] = and_or(w << 3, mask, MAGIC);
    p[1] = and_or(w >> 1, mask, MAGIC);
    p[2] = and_or(w >> 5, mask, MAGIC);
    p[3] = and_or(w >> 9, mask, MAGIC);
  }
  __device__ __forceinline__ static uint32_t code_of(int, uint16_t half) { return (half >> 3) & 15u; }
  __device__ __forceinline__ static float dot(uint32_t a, uint32_t b, float c) { return dot2_bf16(a, b, c); }
  __device__ __forceinline__ static void stage(uint32_t P[4], float2& es) {
#pragma unroll
    for (int j = 0; j < 4; ++j) es.x = dot2_bf16(P[j], 0x3F803F80u, es.x);
  }
  __device__ __forceinline__ static float2 sums(float2 es) { return make_float2(0.0f, es.x); }
  __device__ __forceinline__ static float finish(float acc, float2 es, float z) {
    return fmaf(acc, 0.125f, -(16.0f + z) * es.y);
  }
};

// Activation pairs matching the unpack order above: from 8 consecutive 16-bit
// values h0..h7 (as four 32-bit words u0..u3 = (h0,h1),(h2,h3),(h4,h5),(h6,h7))
// build (h0,h4), (h1,h5), (h2,h6), (h3,h7).
__device__ __forceinline__ void pair_up(const uint32_t u[4], uint32_t P[4]) {
  P[0] = __builtin_amdgcn_perm(u[2], u[0], 0x05040100u);
  P[1] = __builtin_amdgcn_perm(u[2], u[0], 0x07060302u);
  P[2] = __builtin_amdgcn_perm(u[3], u[1], 0x05040100u);
  P[3] = __builtin_amdgcn_perm(u[3], u[1], 0x07060302u);
}

}  // namespace qlin
