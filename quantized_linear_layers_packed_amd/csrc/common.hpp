// Internal helpers shared by the library's translation units (host and device).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstring>
#include <string>

#include "../../include/qlin.h"

namespace qlin {

// ---------------------------------------------------------------------------
// Error reporting (thread-local message + status)

void set_error(const std::string& msg);
void clear_error();
qlin_status fail(qlin_status s, const std::string& msg);

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Launch-error check after hipLaunchKernelGGL.
qlin_status check_launch(const char* what);

// ---------------------------------------------------------------------------
// Host-side IEEE half / bfloat16 conversions (round to nearest, ties to even).

inline uint32_t f32_bits(float f) { uint32_t u; std::memcpy(&u, &f, 4); return u; }
inline float bits_f32(uint32_t u) { float f; std::memcpy(&f, &u, 4); return f; }

inline uint16_t host_f32_to_f16(float f) {
  const uint32_t x = f32_bits(f);
  const uint32_t sign = (x >> 16) & 0x8000u;
  const uint32_t ax = x & 0x7FFFFFFFu;
  if (ax >= 0x7F800000u) {                        // inf / nan
    return static_cast<uint16_t>(sign | 0x7C00u | (ax > 0x7F800000u ? (0x200u | ((ax >> 13) & 0x3FFu)) : 0u));
  }
  if (ax >= 0x477FF000u) return static_cast<uint16_t>(sign | 0x7C00u);   // >= 65520 -> inf
  if (ax < 0x38800000u) {                         // below 2^-14: subnormal half or zero
    if (ax <= 0x33000000u) return static_cast<uint16_t>(sign);            // <= 2^-25 -> 0
    const uint32_t e = ax >> 23;
    const uint32_t m = (ax & 0x7FFFFFu) | 0x800000u;
    const uint32_t shift = 126u - e;              // value / 2^-24 = m >> shift
    uint32_t r = m >> shift;
    const uint32_t rem = m & ((1u << shift) - 1u);
    const uint32_t halfway = 1u << (shift - 1u);
    if (rem > halfway || (rem == halfway && (r & 1u))) ++r;
    return static_cast<uint16_t>(sign | r);
  }
  uint32_t r = (ax >> 13) - (112u << 10);
  const uint32_t rem = ax & 0x1FFFu;
  if (rem > 0x1000u || (rem == 0x1000u && (r & 1u))) ++r;
  return static_cast<uint16_t>(sign | r);
}

inline float host_f16_to_f32(uint16_t h) {
  const uint32_t sign = static_cast<uint32_t>(h & 0x8000u) << 16;
  const uint32_t e = (h >> 10) & 0x1Fu;
  const uint32_t m = h & 0x3FFu;
  if (e == 0x1Fu) return bits_f32(sign | 0x7F800000u | (m << 13));
  if (e == 0) {
    if (m == 0) return bits_f32(sign);
    // subnormal: m * 2^-24
    const float v = static_cast<float>(m) * 5.9604644775390625e-08f;
    return sign ? -v : v;
  }
  return bits_f32(sign | ((e + 112u) << 23) | (m << 13));
}

inline bool host_f16_is_finite(uint16_t h) { return ((h >> 10) & 0x1Fu) != 0x1Fu; }

}  // namespace qlin
