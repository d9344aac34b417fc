// CPU check of the 16-bit gradient-range thresholds (fo_grad16.hpp) against
// brute force over every pattern, for bfloat16 and binary16, on thresholds
// at, between and around pattern values.  Prints "ok <cases>" or the first
// failure and exits 1.
#include <cmath>
#include <cstdio>
#include <cstdint>
#include <cstring>
#include <vector>

#include "../../precision_optimizer_state_amd/csrc/fo_grad16.hpp"

static float from_bits(uint32_t u) { float f; std::memcpy(&f, &u, 4); return f; }

int main() {
  long cases = 0;
  for (int fmt = 0; fmt < 2; ++fmt) {
    const bool bf16 = fmt == 0;
    const uint32_t top = bf16 ? 0x7F80u : 0x7C00u;
    // values must increase with the pattern (the ordering the kernel relies on)
    for (uint32_t p = 1; p <= top; ++p)
      if (!(fo::grad16_value(bf16, p) > fo::grad16_value(bf16, p - 1))) {
        std::printf("failed: %s value not increasing at %#x\n", bf16 ? "bf16" : "fp16", p);
        return 1;
      }
    // binary16 decode spot checks: smallest subnormal, smallest normal, max
    if (!bf16 && (fo::grad16_value(false, 1) != std::ldexp(1.0f, -24) ||
                  fo::grad16_value(false, 0x400) != std::ldexp(1.0f, -14) ||
                  fo::grad16_value(false, 0x7BFF) != 65504.0f)) {
      std::printf("failed: binary16 decode\n");
      return 1;
    }
    std::vector<float> val(top + 1);
    for (uint32_t p = 0; p <= top; ++p) val[p] = fo::grad16_value(bf16, p);
    for (uint32_t xb = 0x00000001u; xb < 0x7F800000u; xb += 0x0003F3A1u) {
      for (int d = -2; d <= 2; ++d) {
        const float x = from_bits(xb + (uint32_t)d);
        if (!(x > 0.0f)) continue;
        for (int strict = 0; strict < 2; ++strict) {
          uint32_t want = 0;
          for (uint32_t p = 0; p <= top; ++p)
            if (strict ? (val[p] < x) : (val[p] <= x)) want = p;
          const uint32_t got = fo::grad16_last(bf16, x, strict != 0);
          ++cases;
          if (got != want) {
            std::printf("failed: %s x=%a strict=%d got %#x want %#x\n", bf16 ? "bf16" : "fp16", x, strict, got, want);
            return 1;
          }
        }
      }
    }
    // thresholds exactly at pattern values
    for (uint32_t p = 1; p < top; p += 7) {
      const float x = fo::grad16_value(bf16, p);
      cases += 2;
      if (fo::grad16_last(bf16, x, true) != p - 1 || fo::grad16_last(bf16, x, false) != p) {
        std::printf("failed: %s at pattern %#x\n", bf16 ? "bf16" : "fp16", p);
        return 1;
      }
    }
  }
  std::printf("ok %ld\n", cases);
  return 0;
}
