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
enum { COMPANDED = 0, LINEAR = 1 };

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
        // rho = round_half_even(L / 256) clamped to 127, L = sext16(low half):
        // 128 + L/256 is exact in one FMA, v_cvt_pk_u8_f32 rounds it half to
        // even, saturates at 255 (rho = 127) and writes it into its byte, and
        // the XOR with 0x80 turns offset binary into two's complement (checked
        // against the integer form on all 2^16 low halves)
        uint32_t e0 = 0u, e1 = 0u;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const float y = __builtin_fmaf((float)(int16_t)f2u(x[k]), 0x1p-8f, 128.0f);
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

// ---------------------------------------------------------------------------
// Cross-lane helpers (DPP inside a quad of 4 lanes = one 32-element block)
// ---------------------------------------------------------------------------
template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}
// quad_perm selectors
constexpr int QP_SWAP1 = 0xB1;   // [1,0,3,2]
constexpr int QP_SWAP2 = 0x4E;   // [2,3,0,1]
template <int J> constexpr int qp_bcast() { return J * 0x55; }   // [J,J,J,J]

__device__ __forceinline__ float quad_max(float x) {   // IEEE maxNum over the 4 lanes
  x = fmaxf(x, dpp_f<QP_SWAP1>(x));
  x = fmaxf(x, dpp_f<QP_SWAP2>(x));
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
// through unchanged.  Callers fall back to the IEEE expansion when any lane
// has 0 < v < 2^-96 (sqrt_needs_scaling).
__device__ __forceinline__ float sqrt_corrected(float v) {
  float s = __builtin_amdgcn_sqrtf(v);
  const float s_dn = u2f(f2u(s) - 1u), s_up = u2f(f2u(s) + 1u);
  const float r_dn = __builtin_fmaf(-s_dn, s, v);
  const float r_up = __builtin_fmaf(-s_up, s, v);
  s = (r_dn <= 0.0f) ? s_dn : s;
  s = (r_up > 0.0f) ? s_up : s;
  return s;
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

// ---------------------------------------------------------------------------
// State codecs
// ---------------------------------------------------------------------------
// Momentum encode by interval table: a in [0,1] is keyed by the top 15 bits of
// its f32 pattern (sign, exponent and 6 mantissa bits), counted from 2^-9 (every
// a below 2^-9 shares key 0).  Every key interval holds at most one of the code
// thresholds (2k+1)/(507-2k) (checked exactly for all 577 keys; one mantissa bit
// fewer would put two thresholds into some intervals just below 1), so
// code(a) = menc[key].code + (a >= menc[key].thr).
struct MEnc { float thr; int32_t code; };
constexpr int MENC_SHIFT = 17;
constexpr uint32_t MENC_BASE = 0x3B000000u >> MENC_SHIFT;                 // 2^-9
constexpr int MENC_N = (int)((0x3F800000u >> MENC_SHIFT) - MENC_BASE) + 1;  // keys up to a = 1
constexpr int MENC_CAP = 640;                            // pads the tables to 6 KiB
static_assert(MENC_CAP >= MENC_N, "interval table capacity");
// Codec tables (built once per device by k_init_tables, copied into LDS):
//   lut[q + 128] = RN32(q / (254 - |q|)) for q in [-127, 127]: momentum levels;
//                  lut[0] (code -128, never written by the encoder) = lut[1]
//   menc[k]      = interval table of the momentum code as above
struct CodecTables { float lut[256]; MEnc menc[MENC_CAP]; };
constexpr int LUT_BIAS = 128;
static_assert(sizeof(CodecTables) == 6 * 1024, "six 1-KiB chunks: one 64-lane x 16-B load each");

// Builds the tables (one workgroup).  thr[k] = smallest f32 >= (2k+1)/(507-2k),
// the |z| at which round(127*phi(|z|)) steps from k to k+1.
__device__ __forceinline__ void build_tables(FO_GLOBAL CodecTables* out, float* thr, int tid, int nthreads) {
  for (int i = tid; i < 256; i += nthreads) {
    const int q = max(i - LUT_BIAS, -127);
    const int aq = q < 0 ? -q : q;
    out->lut[i] = (float)q / (float)(254 - aq);         // IEEE division
  }
  for (int k = tid; k < 127; k += nthreads) {
    const float a = (float)(2 * k + 1), b = (float)(507 - 2 * k);
    float t = a / b;                                    // nearest
    if (__builtin_fmaf(t, b, -a) < 0.0f) t = u2f(f2u(t) + 1u);   // exact residual: step up
    thr[k] = t;
  }
  __syncthreads();
  for (int key = tid; key < MENC_CAP; key += nthreads) {
    MEnc e;
    if (key < MENC_N) {
      const float lo = (key == 0) ? 0.0f : u2f((MENC_BASE + key) << MENC_SHIFT);
      const float hi = u2f((MENC_BASE + key + 1) << MENC_SHIFT);
      int code = 0;
      for (int k = 0; k < 127; ++k) code += (thr[k] <= lo) ? 1 : 0;
      e.code = code;
      e.thr = (code < 127 && thr[code] < hi) ? thr[code] : 2.0f;
    } else {
      e.code = 127;
      e.thr = 2.0f;
    }
    out->menc[key].thr = e.thr;
    out->menc[key].code = e.code;
  }
}

// momentum, companded: z = m*R (R = RN32(1/s)); q = sign(z)*round(127*phi(min(|z|,1)))
__device__ __forceinline__ int32_t encode_m_companded(float m, float R, const CodecTables& T) {
  const float z = m * R;
  const float a = fminf(fabsf(z), 1.0f);                  // NaN -> 1
  const uint32_t key = __builtin_elementwise_sub_sat(f2u(a) >> MENC_SHIFT, MENC_BASE);
  const MEnc e = T.menc[key];
  const int32_t q = e.code + (a >= e.thr ? 1 : 0);
  return (z < 0.0f) ? -q : q;
}

// Clamping happens in float with IEEE minNum/maxNum, which also sends NaN to
// the upper bound, so the float->int conversions below always see in-range values.
__device__ __forceinline__ int32_t encode_m_linear(float m, float C) {
  const float y = fmaxf(fminf(m * C, 127.0f), -127.0f);   // C = RN32(127/s); NaN -> 127
  return (int32_t)__builtin_rintf(y);
}

// variance: y = x*C, C = RN32(255/s) (companded, x = sqrt(v)) or RN32(255/s^2)
// (linear, x = v); code = clamp(round_half_even(y), 0, 255) written into byte
// `k` of `acc` (v_cvt_pk_u8_f32 rounds half to even and saturates; verified
// against rint+clamp over every non-NaN f32 by fo_selftest; it turns NaN into
// 0, hence the fminf first).
__device__ __forceinline__ uint32_t encode_v_into(float x, float C, uint32_t k, uint32_t acc) {
  const float y = fminf(x * C, 255.0f);                    // x*C >= 0; NaN -> 255
  return __builtin_amdgcn_cvt_pk_u8_f32(y, k, acc);
}

constexpr float K127 = 1.0f / 127.0f;   // RN32(1/127), constant-folded
constexpr float K255 = 1.0f / 255.0f;   // RN32(1/255)

}  // namespace fo
