// fo_device.hpp -- device-side numerics of the fused low-precision optimizer
// step for gfx950 (CDNA4, wave64).
//
// Everything here works on IEEE-754 bit patterns with integer arithmetic where
// that is exact and cheap; the floating-point operations that remain are
// single IEEE operations (compiled without contraction, with correctly
// rounded division and square root, f32 and f16 denormals preserved).
//
// Weight split (16-bit theta' + N-bit ECC): Davis Blalock's FlashOptim
// thread, posts on weight splitting and the ECC bits; blog "FlashOptim:
// Breaking the Memory Wall with 24-bit Weights and Companded States",
// Methodology section 1.  The ECC is the signed offset of the f32 value from
// theta' in units of 2^-N of the 16-bit spacing on the value's side, rounded
// half to even; theta' is the f32 value rounded to nearest with ties away
// from zero.
//
// Key identity used for bf16: the f32 encoding of a bf16 value is its bit
// pattern shifted left by 16, and inside any binade (and across the binade
// boundary below a power of two, where both the bf16 spacing and the f32
// spacing halve) one bf16 spacing is exactly 2^16 f32 spacings.  Hence the
// side-aware offset is the signed difference of the magnitude bit patterns:
//     bits(|x|) - bits(|theta'|) = sext16(low 16 bits of bits(|x|))
// and reconstruction is a single integer add on the f32 pattern (valid for
// either sign, because the sign bit is untouched).  fp16 has the same
// property with 2^13 f32 spacings per fp16 spacing, except below the smallest
// fp16 normal, where a float path is used.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fo {

enum { BF16 = 0, FP16 = 1 };
// state codecs: 8-bit companded, 8-bit linear, 4-bit companded (two codes a
// byte), and 8-bit companded with bfloat16 block scales (binary16 otherwise)
enum { COMPANDED = 0, LINEAR = 1, COMPANDED4 = 2, COMPANDED_BF16S = 3 };
// the codec of a state's codes, and whether its block scales are bfloat16
template <int CODEC> constexpr int code_codec = (CODEC == COMPANDED_BF16S) ? COMPANDED : CODEC;
template <int CODEC> constexpr bool scale_bf16 = (CODEC == COMPANDED_BF16S);
template <int CODEC> constexpr int code_bits = (CODEC == COMPANDED4) ? 4 : 8;

// Pointers into device memory are declared in the global address space so the
// compiler emits global_* (not flat_*) memory instructions: flat accesses share
// the LDS wait counter and would make every LDS table lookup wait for all
// in-flight HBM loads.
#define FO_GLOBAL __attribute__((address_space(1)))
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint32_t f2u(float x) { return __float_as_uint(x); }
__device__ __forceinline__ float u2f(uint32_t x) { return __uint_as_float(x); }

__device__ __forceinline__ float h2f(uint32_t h) {  // binary16 pattern -> f32 (exact)
  return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}

// ---------------------------------------------------------------------------
// 16-bit element access inside packed dwords
// ---------------------------------------------------------------------------
template <int WFMT> struct W16;
template <> struct W16<BF16> {
  static __device__ __forceinline__ float lo(uint32_t w) { return u2f(w << 16); }
  static __device__ __forceinline__ float hi(uint32_t w) { return u2f(w & 0xFFFF0000u); }
};
template <> struct W16<FP16> {
  static __device__ __forceinline__ float lo(uint32_t w) { return h2f(w & 0xFFFFu); }
  static __device__ __forceinline__ float hi(uint32_t w) { return h2f(w >> 16); }
};

template <int WFMT>
__device__ __forceinline__ float widen(uint32_t w, int half) {
  return half ? W16<WFMT>::hi(w) : W16<WFMT>::lo(w);
}

// ---------------------------------------------------------------------------
// ECC decode: theta' (already widened to f32, exact) + rho -> f32 master
// ---------------------------------------------------------------------------
// The same decode straight from the packed words for bf16: one byte permute
// (v_perm_b32: bytes 4-7 from `w`, 0-3 from `e`, selector 0x0C gives 0)
// forms u = (theta' << 16) | (rho's bits << SH) -- rho's byte in bits 8-15
// for ECC8, its half in bits 0-15 for ECC16 -- and (u ^ B) - B with
// B = 0x8000, rho's sign bit in both layouts, turns the field from two's
// complement into the signed addend, giving bits(theta') + (rho << SH) in
// one XOR-add.  h: the weight's half in `w`; b: rho's byte (ECC8) or half
// (ECC16) in `e`.
template <int ECC>
__device__ __forceinline__ float ecc_decode_bf16_packed(uint32_t w, uint32_t e, int h, int b) {
  uint32_t sel, bias;
  if constexpr (ECC == 8) {
    sel = ((uint32_t)(5 + 2 * h) << 24) | ((uint32_t)(4 + 2 * h) << 16) | ((uint32_t)b << 8) | 0x0Cu;
    bias = 0x8000u;
  } else {
    sel = ((uint32_t)(5 + 2 * h) << 24) | ((uint32_t)(4 + 2 * h) << 16) | ((uint32_t)(2 * b + 1) << 8) |
          (uint32_t)(2 * b);
    bias = 0x8000u;
  }
  const uint32_t u = __builtin_amdgcn_perm(w, e, sel);
  return u2f((u ^ bias) - bias);
}

template <int WFMT, int ECC>
__device__ __forceinline__ float ecc_decode(float t, int32_t rho) {
  if constexpr (WFMT == BF16) {
    // one bf16 spacing = 2^16 f32 spacings; rho counts 2^-N of it
    constexpr int SH = 16 - ECC;
    return u2f(f2u(t) + ((uint32_t)rho << SH));
  } else {
    static_assert(ECC == 8, "fp16 supports an 8-bit ECC");
    if (fabsf(t) > 0x1p-14f)                     // |theta'| above the smallest fp16 normal (or inf)
      return u2f(f2u(t) + ((uint32_t)rho << 5)); // one fp16 spacing = 2^13 f32 spacings
    // zero, subnormal and the smallest normal (and NaN, which stays NaN): spacing
    // 2^-24 on both sides; the offset rho * 2^-32 (exact) is applied to the magnitude.
    // Product and sum are both exact here, so one fused multiply-add gives the
    // same value as the separate operations.
    return __builtin_fmaf((float)rho, __builtin_copysignf(0x1p-32f, t), t);
  }
}

// ---------------------------------------------------------------------------
// ECC encode (split): f32 -> (theta' pattern in the low 16 bits, rho)
// ---------------------------------------------------------------------------
struct SplitOut { uint32_t h; int32_t rho; };

// round-half-to-even of a signed integer divided by 2^r, 1 <= r <= 30
__device__ __forceinline__ int32_t rne_shift(int32_t d, int r) {
  return (d + ((1 << (r - 1)) - 1) + ((d >> r) & 1)) >> r;
}

template <int WFMT, int ECC>
__device__ __forceinline__ SplitOut ecc_encode(float x) {
  const uint32_t xb = f2u(x);
  const uint32_t ab = xb & 0x7FFFFFFFu;
  SplitOut o;
  if constexpr (WFMT == BF16) {
    o.h = (ab + 0x8000u) >> 16;                        // RNA on the magnitude
    const int32_t L = ((int32_t)(ab << 16)) >> 16;     // bits(|x|) - bits(|theta'|)
    if constexpr (ECC == 8) {
      o.rho = min(rne_shift(L, 8), 127);
    } else {
      o.rho = L;                                       // exact: in [-2^15, 2^15)
    }
    if (ab >= 0x7F7F8000u) {                           // RNA overflow, inf, nan (rare)
      if (ab > 0x7F800000u)       { o.h = 0x7FC0u; o.rho = 0; }
      else if (ab == 0x7F800000u) { o.h = 0x7F80u; o.rho = 0; }
      else                        { o.h = 0x7F7Fu; o.rho = (ECC == 8) ? 127 : 32767; }
    }
  } else {
    static_assert(ECC == 8, "fp16 supports an 8-bit ECC");
    if (ab >= 0x38800000u) {                           // |x| >= 2^-14
      o.h = ((ab + 0x1000u) >> 13) - (112u << 10);     // RNA, rebias 127 -> 15
      const int32_t L = ((int32_t)(ab << 19)) >> 19;   // sext13
      o.rho = min(rne_shift(L, 5), 127);
      if (o.h >= 0x7C00u) {                            // overflow (|x| >= 65520), inf, nan
        if (ab > 0x7F800000u)       { o.h = 0x7E00u; o.rho = 0; }
        else if (ab == 0x7F800000u) { o.h = 0x7C00u; o.rho = 0; }
        else                        { o.h = 0x7BFFu; o.rho = 127; }
      }
    } else {
      // |x| < 2^-14: fp16 values are multiples of 2^-24.  |x| = M * 2^(E-23);
      // in units of 2^-24, |x| = M / 2^s with s = -(E+1) >= 14.
      const uint32_t e = ab >> 23;
      const uint32_t M = e ? ((ab & 0x7FFFFFu) | 0x800000u) : ab;
      const int s = e ? (126 - (int)e) : 125;
      uint32_t k = 0;
      int32_t diff = (int32_t)M;
      if (s <= 24) {
        k = (M + (1u << (s - 1))) >> s;               // RNA
        diff = (int32_t)M - (int32_t)(k << s);
      }
      // delta = diff * 2^(E-23) * 2^8 / 2^-24 = diff / 2^(s-8)
      const int r = s - 8;
      int32_t rho = (r >= 25) ? 0 : rne_shift(diff, r);
      o.rho = max(min(rho, 127), -128);
      o.h = k;                                         // k = 1024 is the smallest normal
    }
  }
  o.h |= (xb >> 16) & 0x8000u;
  return o;
}

// byte/half selection helpers (v_perm_b32: bytes 0-3 = src1, 4-7 = src0)
__device__ __forceinline__ uint32_t perm(uint32_t hi_src, uint32_t lo_src, uint32_t sel) {
  return __builtin_amdgcn_perm(hi_src, lo_src, sel);
}
// low bytes of four words -> one packed word
__device__ __forceinline__ uint32_t pack4_byte0(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  return perm(perm(d, c, 0x0C0C0400u), perm(b, a, 0x0C0C0400u), 0x05040100u);
}

// Split of 8 consecutive values into packed theta' (4 dwords) and ECC (ECC/4
// dwords).  bf16 fast path, valid while every value of the wave is below the
// bf16 overflow tie and not NaN: theta' = high half of (bits + 0x8000) (RNA on
// the magnitude; the sign bit is untouched), ECC8 = round-half-even of
// sext16(low half) / 256 clamped at 127, ECC16 = the low half of the pattern
// (the offset itself).
// fp16 fast path below.  Otherwise every element goes through ecc_encode.
template <int WFMT, int ECC>
__device__ __forceinline__ void split8(const float (&x)[8], uint32_t (&wo)[4], uint32_t (&eo)[ECC / 4]) {
  if constexpr (WFMT == BF16) {
    uint64_t special = 0;
#pragma unroll
    for (int k = 0; k < 8; ++k) special |= __builtin_amdgcn_ballot_w64(!(fabsf(x[k]) < 0x1.ffp+127f));
    if (special == 0) {
      uint32_t t[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) t[k] = f2u(x[k]) + 0x8000u;
#pragma unroll
      for (int i = 0; i < 4; ++i) wo[i] = perm(t[2 * i + 1], t[2 * i], 0x07060302u);
      if constexpr (ECC == 8) {
        // rho = round_half_even(L / 256) clamped to 127, L = sext16(low half).
        // The low half of t = bits + 0x8000 is T = L + 2^15, so the float with
        // pattern 0x4B000000 | T is 2^23 + T and one FMA forms T/256 = 128 +
        // L/256 exactly; v_cvt_pk_u8_f32 rounds it half to even, saturates
        // at 255 (rho = 127) and writes it into its byte, and the XOR with 0x80
        // turns offset binary into two's complement (checked against the
        // integer form on all 2^16 low halves)
        uint32_t e0 = 0u, e1 = 0u;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const float y = __builtin_fmaf(u2f((t[k] & 0xFFFFu) | 0x4B000000u), 0x1p-8f, -32768.0f);
          if (k < 4) e0 = __builtin_amdgcn_cvt_pk_u8_f32(y, k, e0);
          else e1 = __builtin_amdgcn_cvt_pk_u8_f32(y, k - 4, e1);
        }
        eo[0] = e0 ^ 0x80808080u;
        eo[1] = e1 ^ 0x80808080u;
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) eo[i] = perm(f2u(x[2 * i + 1]), f2u(x[2 * i]), 0x05040100u);
      }
      return;
    }
  } else {
    // fp16 + ECC8, valid while every value of the wave is finite and below
    // the RNA overflow threshold 65520.  theta' starts as the hardware
    // round-to-nearest-even conversion t; d = |x| - |t| is exact (Sterbenz,
    // or t = 0), and rho = rint(d * 2^8 / ulp_side(t)) = rint(ldexp(d, k))
    // with k = 145 - max(biased exponent of x, 113) (113: the fp16 subnormal
    // spacing 2^-24).  The exponent of x itself gives the spacing on x's side
    // of t: above t, and below a t that is not a power of two, x shares t's
    // binade; below a power of two t (the inner side, half spacing) x lies in
    // the binade under it.  RNE and RNA differ only on an exact tie that RNE
    // rounded towards zero, which shows as d * 2^k == +128 exactly: then
    // theta' moves one pattern away from zero and rho = -128.  Any other value
    // rounding to 128 clamps to 127.  rho is rounded half to even by adding
    // 1.5 * 2^23 (|d * 2^k| <= 128): the sum's pattern is 0x4B400000 + rho,
    // whose low byte is rho's two's-complement byte.
    uint64_t special = 0;
#pragma unroll
    for (int k = 0; k < 8; ++k) special |= __builtin_amdgcn_ballot_w64(!(fabsf(x[k]) < 65520.0f));
    if (special == 0) {
      uint32_t H[8], R[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const _Float16 hh = (_Float16)x[k];
        const float t = (float)hh;
        const float d = fabsf(x[k]) - fabsf(t);
        const int eb = (int)((f2u(x[k]) >> 23) & 0xFFu);
        const int sh = 145 - max(eb, 113);
        const float rf = __builtin_ldexpf(d, sh);
        const bool tie = (rf == 128.0f);
        const uint32_t rb = min(f2u(rf + 0x1.8p23f), 0x4B40007Fu);   // rho <= 127
        H[k] = (uint32_t)__builtin_bit_cast(uint16_t, hh) + (tie ? 1u : 0u);
        R[k] = tie ? 0x4B3FFF80u : rb;                               // low byte: rho (tie: -128)
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) wo[i] = perm(H[2 * i + 1], H[2 * i], 0x05040100u);
      eo[0] = pack4_byte0(R[0], R[1], R[2], R[3]);
      eo[1] = pack4_byte0(R[4], R[5], R[6], R[7]);
      return;
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) wo[i] = 0;
#pragma unroll
  for (int i = 0; i < ECC / 4; ++i) eo[i] = 0;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const SplitOut so = ecc_encode<WFMT, ECC>(x[k]);
    wo[k >> 1] |= so.h << (16 * (k & 1));
    if constexpr (ECC == 8) eo[k >> 2] |= ((uint32_t)so.rho & 0xFFu) << (8 * (k & 3));
    else eo[k >> 1] |= ((uint32_t)so.rho & 0xFFFFu) << (16 * (k & 1));
  }
}

// ---------------------------------------------------------------------------
// Block scales: smallest binary16 >= x (x >= 0), saturating at 65504
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t ru_fp16(float x) {
  const uint32_t ux = f2u(x) & 0x7FFFFFFFu;            // callers pass |.| or sqrt: sign ignored
  if (ux > 0x7F800000u) return 0x7E00u;                // NaN
  if (ux >= 0x477FE000u) return 0x7BFFu;               // >= 65504 (and +inf)
  const uint32_t e = ux >> 23;
  if (e >= 113u)                                       // >= 2^-14: truncate, then bump if inexact
    return ((ux >> 13) - (112u << 10)) + ((ux & 0x1FFFu) != 0u);
  const uint32_t M = e ? ((ux & 0x7FFFFFu) | 0x800000u) : ux;
  const int s = e ? (126 - (int)e) : 125;              // value = M / 2^s units of 2^-24
  if (s >= 25) return M ? 1u : 0u;
  return (M + (1u << s) - 1u) >> s;                    // ceil
}

// Block scales of the bfloat16-scale codec: smallest bfloat16 >= x (x >= 0,
// subnormal values included), saturating at the largest finite bfloat16
// 0x7F7F; NaN -> 0x7FC0.  On non-negative patterns the bfloat16 pattern of a
// value is the high half of its f32 pattern, so rounding up is adding
// 0xFFFF before taking the high half.
__device__ __forceinline__ uint32_t ru_bf16(float x) {
  const uint32_t ux = f2u(x) & 0x7FFFFFFFu;            // callers pass |.| or sqrt: sign ignored
  if (ux > 0x7F800000u) return 0x7FC0u;                // NaN
  return min((ux + 0xFFFFu) >> 16, 0x7F7Fu);           // +inf and values past 0x7F7F saturate
}
// stored scale pattern -> f32 (exact) in the codec's scale format
template <int CODEC>
__device__ __forceinline__ float scale_f32(uint32_t bits) {
  if constexpr (scale_bf16<CODEC>) return u2f(bits << 16);
  else return h2f(bits);
}
// The fast forms of the steps take block scales in binary16's range only:
// zero, or [2^-24, 65504].  There the fast division and reciprocal are exact
// for every divisor with at most 22 significand bits (bfloat16 has 8), and
// the decoded states keep the magnitudes the fast update is valid for.  A
// bfloat16 scale outside it (NaN and +-Inf included) sends its wave to the
// IEEE forms.  Tested on the pattern, without short-circuit branches (which
// split the scale loads of a tile): +0, or 0x33800000 (2^-24) through
// 0x477FE000 (65504); -0, negative values and NaN fall outside.
__device__ __forceinline__ bool scale_in_fast_range(float s) {
  const uint32_t u = f2u(s);
  return (u == 0u) | (u - 0x33800000u <= 0x477FE000u - 0x33800000u);
}

// ---------------------------------------------------------------------------
// Cross-lane helpers (DPP inside a quad of 4 lanes = one 32-element block)
// ---------------------------------------------------------------------------
template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
  // quad_perm reads a lane of the same quad, so every lane has a source and
  // the old value is never used (bound_ctrl set: no copy of it is made)
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, true));
}
// quad_perm selectors
constexpr int QP_SWAP1 = 0xB1;   // [1,0,3,2]
constexpr int QP_SWAP2 = 0x4E;   // [2,3,0,1]
template <int J> constexpr int qp_bcast() { return J * 0x55; }   // [J,J,J,J]

// IEEE maxNum (a quiet NaN operand loses to a number) of operands that are
// never signaling NaNs.  fmaxf has to quiet a signaling NaN first, so the
// compiler puts a canonicalising v_max_f32 x, x, x in front of every operand
// it cannot prove quiet (here: all of them, after selects and lane moves);
// writing v_max_f32 / v_max3_f32 directly drops those.  Callers pass only
// arithmetic results, lane copies of them and the quiet NaN constant.
__device__ __forceinline__ float max_quiet(float a, float b) {
  float r;
  asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}
__device__ __forceinline__ float max3_quiet(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}
// maxNum(|a|, |b|) and maxNum(m, |a|, |b|)
__device__ __forceinline__ float max_abs_quiet(float a, float b) {
  float r;
  asm("v_max_f32_e64 %0, |%1|, |%2|" : "=v"(r) : "v"(a), "v"(b));
  return r;
}
__device__ __forceinline__ float max3_abs_quiet(float m, float a, float b) {
  float r;
  asm("v_max3_f32 %0, %1, |%2|, |%3|" : "=v"(r) : "v"(m), "v"(a), "v"(b));
  return r;
}

__device__ __forceinline__ float quad_max(float x) {   // IEEE maxNum over the 4 lanes
  x = max_quiet(x, dpp_f<QP_SWAP1>(x));
  x = max_quiet(x, dpp_f<QP_SWAP2>(x));
  return x;
}
template <int J>
__device__ __forceinline__ float quad_bcast(float x) { return dpp_f<qp_bcast<J>()>(x); }

// ---------------------------------------------------------------------------
// Exact fast arithmetic (gfx950)
// ---------------------------------------------------------------------------
// Correctly rounded square root from the hardware estimate: v_sqrt_f32 is
// within one ulp, and the residuals v - s'*s of the two neighbours decide the
// rounding exactly (no float lies strictly between s_lo*s and the squared
// midpoint).  The residuals are exact for v >= 2^-96; v = 0, inf and NaN pass
// through unchanged.  Callers keep v out of (0, 2^-96) or fall back to the
// IEEE expansion.
__device__ __forceinline__ float sqrt_corrected(float v) {
  float s = __builtin_amdgcn_sqrtf(v);
  const float s_dn = u2f(f2u(s) - 1u), s_up = u2f(f2u(s) + 1u);
  const float r_dn = __builtin_fmaf(-s_dn, s, v);
  const float r_up = __builtin_fmaf(-s_up, s, v);
  s = (r_dn <= 0.0f) ? s_dn : s;
  s = (r_up > 0.0f) ? s_up : s;
  return s;
}
// Cheaper correctly rounded square root for v = 0 and 2^-96 <= v < 2^128 - 2^104
// (every finite v from 2^-96 up but the largest): on gfx950 the hardware
// estimate a of the square root of v's successor is never below RN(sqrt(v))
// and at most one ulp above it (fo_selftest mode 6 checks every v of that
// range), so only the lower neighbour dn of a is a candidate, and the
// residual v - dn*a decides between them as in sqrt_corrected.  For v = 0 the
// successor is not taken: a = 0, dn is a NaN pattern and the test fails.
__device__ __forceinline__ float sqrt_fast(float v) {
  const uint32_t u = f2u(v);
  const float a = __builtin_amdgcn_sqrtf(u2f(u + (u != 0u ? 1u : 0u)));
  const float dn = u2f(f2u(a) - 1u);
  return (__builtin_fmaf(-dn, a, v) <= 0.0f) ? dn : a;
}
__device__ __forceinline__ bool sqrt_needs_scaling(float v) {   // 0 < v < 2^-96
  return (f2u(v) - 1u) < 0x0F7FFFFFu;
}
// Correctly rounded reciprocal for positive normal b < 2^126: one Newton step
// on the hardware estimate.  Verified exhaustively on gfx950 (fo_selftest);
// callers fall back to IEEE division outside that range.
__device__ __forceinline__ float rcp_refined(float b) {
  const float y0 = __builtin_amdgcn_rcpf(b);
  const float e = __builtin_fmaf(-b, y0, 1.0f);
  return __builtin_fmaf(e, y0, y0);
}
// Correctly rounded quotient a/b from r = RN(1/b): q0 = RN(a*r) is within two
// ulps of a/b; the residual e = b*q0 - a is formed by one FMA, and one more
// FMA q0 - e*r lands within a few 2^-24 ulps of a/b, closer than any binary32
// quotient comes to a rounding midpoint (Markstein's residual correction; the
// negated residual keeps the sign of a zero quotient).  Valid while no
// intermediate leaves the normal range: |a| >= 2^-100 or a = 0, |a/b| < 2^120.
// Checked on the CPU against IEEE division on every pair whose quotient lies
// within 16*2^-47 (relative) of a midpoint, exhaustively for divisors with
// 22-bit significands, and on random pairs; on the device by fo_selftest.
__device__ __forceinline__ float div_refined(float a, float b, float r) {
  const float q0 = a * r;
  const float e = __builtin_fmaf(b, q0, -a);
  return __builtin_fmaf(-e, r, q0);
}

// ---------------------------------------------------------------------------
// State codecs
// ---------------------------------------------------------------------------
// A state block has a binary16 scale s.  Encoding normalises with one
// correctly rounded division z = x/s (div_refined with R = RN(1/s), computed
// once per block); decoding multiplies the code by the block's level spacing:
//   momentum, companded:  m = RN(s * LUT[q])                 (multiplier s)
//   momentum, linear:     m = RN(D * q),  D = RN(s/127)
//   variance, companded:  t = RN(D * q),  D = RN(s/255), v = RN(t*t)
//   variance, linear:     v = RN(D * q),  D = RN(RN(s*s)/255)
// (RN(s*s) is exact: binary16 significands have 11 bits.)  A NaN element gets
// code 0; values past the end codes saturate.

// Momentum encode by interval table: a = |z| in [0,1] is keyed by bits 17..30
// of its f32 pattern (exponent and 6 mantissa bits), clamped to
// [MENC_BASE, MENC_BASE + MENC_NAN]: every a below 2^-9 shares the first key,
// and keys above a = 1 (which the fast encode only sees for NaN) share the
// last, whose code is 0 and whose threshold (NaN) no value reaches.  Every
// other key interval holds at most one of the code thresholds (2k+1)/(507-2k)
// (checked exactly for all 577 keys; one mantissa bit fewer would put two
// thresholds into some intervals just below 1), so
// code(a) = menc[key].code + (a >= menc[key].thr).
struct MEnc { float thr; int32_t code; };
constexpr int MENC_SHIFT = 17;
constexpr uint32_t MENC_BASE = 0x3B000000u >> MENC_SHIFT;                 // 2^-9
constexpr int MENC_N = (int)((0x3F800000u >> MENC_SHIFT) - MENC_BASE) + 1;  // keys up to a = 1
constexpr int MENC_NAN = MENC_N;                                           // NaN (and a > 1)
// The 4-bit momentum code round(7*phi(a)) (codec COMPANDED4) is taken the
// same way from a table keyed by bits 21..30 of a (exponent and 2 mantissa
// bits), clamped to [M4_BASE, M4_BASE + M4_NAN]: every a below 2^-5 shares the
// first key, and every other key interval holds at most one of the seven
// thresholds (2k+1)/(27-2k) (they are 1/27, 3/25, 5/23, 1/3, 9/19, 11/17 and
// 13/15, each in its own quarter-binade at or above 2^-5).
constexpr int M4_SHIFT = 21;
constexpr uint32_t M4_BASE = 0x3D000000u >> M4_SHIFT;                     // 2^-5
constexpr int M4_N = (int)((0x3F800000u >> M4_SHIFT) - M4_BASE) + 1;      // keys up to a = 1
constexpr int M4_NAN = M4_N;
constexpr int M4_CAP = 24;
static_assert(M4_CAP > M4_NAN, "4-bit interval table capacity");
constexpr int MENC_CAP = 608;                            // pads the tables to 6 KiB
static_assert(MENC_CAP > MENC_NAN, "interval table capacity");
// Codec tables (built once per device by k_init_tables, copied into LDS):
//   lut[q + 128]  = RN32(q / (254 - |q|)) for q in [-127, 127]: momentum levels;
//                   lut[0] (code -128, never written by the encoder) = lut[1]
//   menc[k]       = interval table of the momentum code as above
//   lut4[c]       = RN32(q / (14 - |q|)) for the 4-bit pattern c = 0..15 of
//                   the code q (two's complement; pattern 8, the code -8, is
//                   never written and decodes as -7): 4-bit momentum levels
//   menc4[k]      = interval table of the 4-bit momentum code
struct CodecTables { float lut[256]; MEnc menc[MENC_CAP]; float lut4[16]; MEnc menc4[M4_CAP]; };
constexpr int LUT_BIAS = 128;
static_assert(sizeof(CodecTables) == 6 * 1024, "six 1-KiB chunks: one 64-lane x 16-B load each");

// thr[k] = smallest f32 >= (2k+1)/(4L-1-2k), the a at which round(L*phi(a))
// steps from k to k+1 (k < L): L*2a/(1+a) = k + 1/2 solved for a
__device__ __forceinline__ float code_threshold(int k, int L) {
  const float a = (float)(2 * k + 1), b = (float)(4 * L - 1 - 2 * k);
  float t = a / b;                                      // nearest
  if (__builtin_fmaf(t, b, -a) < 0.0f) t = u2f(f2u(t) + 1u);     // exact residual: step up
  return t;
}
// interval table entry of key interval [lo, hi) for thresholds thr[0..L)
__device__ __forceinline__ MEnc interval_entry(float lo, float hi, const float* thr, int L) {
  int code = 0;
  for (int k = 0; k < L; ++k) code += (thr[k] <= lo) ? 1 : 0;
  MEnc e;
  e.code = code;
  e.thr = (code < L && thr[code] < hi) ? thr[code] : 2.0f;
  return e;
}

// Builds the tables (one workgroup; thr holds 127 + 7 floats).
__device__ __forceinline__ void build_tables(FO_GLOBAL CodecTables* out, float* thr, int tid, int nthreads) {
  float* thr4 = thr + 127;
  for (int i = tid; i < 256; i += nthreads) {
    const int q = max(i - LUT_BIAS, -127);
    const int aq = q < 0 ? -q : q;
    out->lut[i] = (float)q / (float)(254 - aq);         // IEEE division
  }
  for (int i = tid; i < 16; i += nthreads) {
    const int q = (i < 8) ? i : max(i - 16, -7);
    const int aq = q < 0 ? -q : q;
    out->lut4[i] = (float)q / (float)(14 - aq);
  }
  for (int k = tid; k < 127; k += nthreads) thr[k] = code_threshold(k, 127);
  for (int k = tid; k < 7; k += nthreads) thr4[k] = code_threshold(k, 7);
  __syncthreads();
  for (int key = tid; key < MENC_CAP; key += nthreads) {
    MEnc e;
    if (key < MENC_N) {
      e = interval_entry((key == 0) ? 0.0f : u2f((MENC_BASE + key) << MENC_SHIFT),
                         u2f((MENC_BASE + key + 1) << MENC_SHIFT), thr, 127);
    } else {
      e.code = 0;
      e.thr = __builtin_nanf("");
    }
    out->menc[key].thr = e.thr;
    out->menc[key].code = e.code;
  }
  for (int key = tid; key < M4_CAP; key += nthreads) {
    MEnc e;
    if (key < M4_N) {
      e = interval_entry((key == 0) ? 0.0f : u2f((M4_BASE + key) << M4_SHIFT),
                         u2f((M4_BASE + key + 1) << M4_SHIFT), thr4, 7);
    } else {
      e.code = 0;
      e.thr = __builtin_nanf("");
    }
    out->menc4[key].thr = e.thr;
    out->menc4[key].code = e.code;
  }
}

// Code of a = |z| for 0 <= a <= 1 or NaN (NaN -> 0), sign of z applied; BITS
// = 8 (codes in [-127, 127]) or 4 (codes in [-7, 7]).
template <int BITS>
__device__ __forceinline__ int32_t momentum_code(float z, const CodecTables& T) {
  MEnc e;
  if constexpr (BITS == 8) {
    const uint32_t kb = __builtin_amdgcn_ubfe(f2u(z), MENC_SHIFT, 14);
    const uint32_t key = min(max(kb, MENC_BASE), MENC_BASE + (uint32_t)MENC_NAN) - MENC_BASE;   // v_med3_u32
    e = T.menc[key];
  } else {
    const uint32_t kb = __builtin_amdgcn_ubfe(f2u(z), M4_SHIFT, 10);
    const uint32_t key = min(max(kb, M4_BASE), M4_BASE + (uint32_t)M4_NAN) - M4_BASE;
    e = T.menc4[key];
  }
  const int32_t q = e.code + (fabsf(z) >= e.thr ? 1 : 0);
  return (z < 0.0f) ? -q : q;
}

// momentum, companded, fast form: s > 0 finite with |m| <= s, or s = 0 / NaN
// (then z is NaN and the code 0).  R = RN(1/s).
template <int BITS = 8>
__device__ __forceinline__ int32_t encode_m_companded(float m, float s, float R, const CodecTables& T) {
  return momentum_code<BITS>(div_refined(m, s, R), T);
}
// momentum, companded, any m and s (IEEE division, clamp at |z| = 1)
template <int BITS = 8>
__device__ __forceinline__ int32_t encode_m_companded_ieee(float m, float s, const CodecTables& T) {
  const float z = m / s;
  if (z != z) return 0;
  return momentum_code<BITS>(__builtin_copysignf(fminf(fabsf(z), 1.0f), z), T);
}
// momentum, linear: y = RN(127 * RN(m/s)); fast form for |m| <= s, the IEEE
// form clamps |y| to 127; NaN -> 0
__device__ __forceinline__ int32_t encode_m_linear(float m, float s, float R) {
  const float y = 127.0f * div_refined(m, s, R);
  return (y == y) ? (int32_t)__builtin_rintf(y) : 0;
}
__device__ __forceinline__ int32_t encode_m_linear_ieee(float m, float s) {
  const float y = 127.0f * (m / s);
  return (y == y) ? (int32_t)__builtin_rintf(fmaxf(fminf(y, 127.0f), -127.0f)) : 0;
}

// variance: y = RN(255 * RN(x/s)), x = sqrt_rn(v) with the companded codec's
// scale s, or x = v with the linear codec's s*s; the code clamp(rne(y), 0, 255)
// goes into byte `k` of `acc`.  v_cvt_pk_u8_f32 rounds half to even,
// saturates, and turns NaN into 0 (checked over every f32 by fo_selftest).
// The fast form needs x finite; the IEEE form takes any x.
__device__ __forceinline__ uint32_t encode_v_into(float x, float s, float R, uint32_t k, uint32_t acc) {
  return __builtin_amdgcn_cvt_pk_u8_f32(255.0f * div_refined(x, s, R), k, acc);
}
__device__ __forceinline__ uint32_t encode_v_into_ieee(float x, float s, uint32_t k, uint32_t acc) {
  return __builtin_amdgcn_cvt_pk_u8_f32(255.0f * (x / s), k, acc);
}

// 4-bit variance: y = RN(15 * RN(x/s)), code clamp(rne(y), 0, 15) into byte k
// of acc.  The fast form needs x <= s (then y <= 15; NaN still gives 0); the
// IEEE form takes any x and clamps the byte to 15.
__device__ __forceinline__ uint32_t encode_v4_into(float x, float s, float R, uint32_t k, uint32_t acc) {
  return __builtin_amdgcn_cvt_pk_u8_f32(15.0f * div_refined(x, s, R), k, acc);
}
__device__ __forceinline__ uint32_t encode_v4_ieee(float x, float s) {
  return min(__builtin_amdgcn_cvt_pk_u8_f32(15.0f * (x / s), 0, 0u), 15u);
}

// Nibble packing of 8 codes of a lane (element i in bits [4i, 4i+4) of one
// word: element 2b in the low nibble of byte b, 2b+1 in its high nibble).
// even / odd hold the codes of elements 0,2,4,6 / 1,3,5,7 in their bytes
// (any sign extension above the nibble is dropped).
__device__ __forceinline__ uint32_t pack_nibbles(uint32_t even, uint32_t odd) {
  return (even & 0x0F0F0F0Fu) | ((odd << 4) & 0xF0F0F0F0u);
}

}  // namespace fo
