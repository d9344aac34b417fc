/*
 * CPU check of the residual-corrected division the fused kernels use
 * (q0 = RN(a*r), e = RN(b*q0 - a) by one FMA, q = RN(q0 - e*r) by one FMA,
 * with r = RN(1/b)) against IEEE division.  The C library's fmaf and the
 * hardware divide are the IEEE operations, as on the device.
 *
 *   mode "hard": every pair (a, b), b with significand in [1, 2), whose
 *     quotient lies within K units of a round-to-nearest midpoint (units of
 *     2^-47 for quotients in [1, 2), 2^-48 in [1/2, 1)), found by solving
 *     B*N == -k (mod 2^m) for each divisor significand B.  Away from
 *     midpoints the corrected quotient is within a few 2^-24 ulps of a/b, so
 *     these are the only pairs that can round differently; the sequence is
 *     invariant under scaling a and b by powers of two while every value
 *     stays normal.
 *   mode "fp16": every divisor with an 11-bit significand (binary16 block
 *     scales) and its square (22 bits), against every dividend significand
 *     in two binades, exhaustively.
 * Prints "<mode> candidates <n> mismatches <m>".
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

static inline float u2f(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static inline uint32_t f2u(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }
static inline float corrected(float a, float b, float r) {
  const float q0 = a * r;
  const float e = fmaf(b, q0, -a);
  return fmaf(-e, r, q0);
}
static uint64_t inv_odd(uint64_t x) {   /* inverse of an odd x modulo 2^64 (Newton) */
  uint64_t y = x;
  for (int i = 0; i < 6; ++i) y *= 2 - x * y;
  return y;
}

static void hard(void) {
  const int K = 16;
  long long cand = 0, bad = 0;
#pragma omp parallel for reduction(+ : cand, bad) schedule(dynamic, 1024)
  for (uint64_t B = 1ull << 23; B < (1ull << 24); ++B) {
    const float b = u2f((127u << 23) | (uint32_t)(B - (1ull << 23)));
    const float r = 1.0f / b;
    for (int q = 0; q < 2; ++q)               /* quotient in [1/2, 1) or [1, 2) */
      for (int m = 24; m <= 25; ++m)          /* the dividend's binade */
        for (int k = -K; k <= K; ++k) {
          if (k == 0) continue;
          const int64_t c = -k;
          const int t = __builtin_ctzll(B);
          if (((uint64_t)c & ((1ull << t) - 1)) != 0) continue;
          const uint64_t mod = 1ull << (m - t);
          const uint64_t N0 = ((uint64_t)(c >> t) * inv_odd(B >> t)) & (mod - 1);
          for (uint64_t N = N0; N < (1ull << 25); N += mod) {
            if (N <= (1ull << 24) || !(N & 1)) continue;          /* odd: a midpoint */
            const __int128 prod = (__int128)B * N + k;
            if (prod % ((__int128)1 << m)) continue;
            const uint64_t A = (uint64_t)(prod >> m);
            if (A < (1ull << 23) || A >= (1ull << 24)) continue;
            const int ea = q ? (m == 24 ? -23 : -22) : (m == 24 ? -24 : -23);
            const float a = ldexpf((float)A, ea);
            const double quo = (double)a / (double)b;
            if (q ? !(quo >= 1.0 && quo < 2.0) : !(quo >= 0.5 && quo < 1.0)) continue;
            cand++;
            if (f2u(corrected(a, b, r)) != f2u(a / b)) bad++;
          }
        }
  }
  printf("hard candidates %lld mismatches %lld\n", cand, bad);
}

static void fp16(void) {
  long long cand = 0, bad = 0;
  for (int sq = 0; sq < 2; ++sq) {
#pragma omp parallel for reduction(+ : cand, bad) schedule(dynamic)
    for (int k = 0; k < 1024; ++k) {
      float s = 1.0f + (float)k / 1024.0f;
      if (sq) s = s * s;                       /* exact: 22-bit significand */
      const float r = 1.0f / s;
      for (uint32_t M = 0; M < (1u << 23); ++M)
        for (int h = 0; h < 2; ++h) {
          const float a = u2f(((h ? 126u : 127u) << 23) | M);
          cand++;
          if (f2u(corrected(a, s, r)) != f2u(a / s)) bad++;
        }
    }
  }
  printf("fp16 candidates %lld mismatches %lld\n", cand, bad);
}

int main(int argc, char** argv) {
  if (argc > 1 && !strcmp(argv[1], "hard")) hard();
  else if (argc > 1 && !strcmp(argv[1], "fp16")) fp16();
  else { fprintf(stderr, "usage: %s hard|fp16\n", argv[0]); return 2; }
  return 0;
}
