// Host-side thresholds of the fused AdamW step's gradient range on 16-bit
// patterns (host code only, no HIP): the step checks its 16-bit gradients
// by their magnitude patterns, which order like the values (infinity above
// every finite pattern, NaN patterns above infinity).
#pragma once

#include <cmath>
#include <cstdint>
#include <cstring>

namespace fo {

// value of a nonnegative 16-bit pattern p <= infinity of bfloat16 (bf16) or
// IEEE binary16
inline float grad16_value(bool bf16, uint32_t p) {
  if (bf16) {
    const uint32_t u = p << 16;
    float f;
    std::memcpy(&f, &u, 4);
    return f;
  }
  const uint32_t e = (p >> 10) & 0x1Fu, m = p & 0x3FFu;
  if (e == 0x1Fu) return INFINITY;
  return e ? std::ldexp((float)(m | 0x400u), (int)e - 25) : std::ldexp((float)m, -24);
}

// the largest pattern p in [0, infinity] with value(p) < x (strict) or
// value(p) <= x, for x > 0 (p = 0 always qualifies)
inline uint32_t grad16_last(bool bf16, float x, bool strict) {
  uint32_t lo = 0, hi = bf16 ? 0x7F80u : 0x7C00u;
  while (lo < hi) {
    const uint32_t mid = (lo + hi + 1) / 2;
    const float v = grad16_value(bf16, mid);
    if (strict ? (v < x) : (v <= x)) lo = mid; else hi = mid - 1;
  }
  return lo;
}

}  // namespace fo
