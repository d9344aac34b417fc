// fo_kernels.hpp -- HIP kernels (gfx950) of the fused low-precision optimizer step.
//
// Fused step layout (one pass per element, HBM-bound, no MFMA):
//   * A wave owns a "wave tile" of 2048 consecutive elements of one tensor,
//     processed as 4 sub-tiles of 512.  In sub-tile j, lane l holds elements
//     [512 j + 8 l, 512 j + 8 l + 8): every load/store instruction of the wave
//     covers one contiguous span (1 KiB for 16-bit streams, 512 B for byte
//     streams) with 16-byte (resp. 8-byte) accesses per lane.
//   * A 32-element block is one quad of 4 lanes.  Block maxima are reduced
//     with two DPP quad permutes, never through LDS.
//   * Per-block arithmetic (scale rounding, reciprocals) is done once per
//     block: lane 4Q+j owns block (sub-tile j, quad Q), and the results are
//     broadcast back to the quad with one DPP quad permute per sub-tile.
//   * Every quotient and square root of the update and the codecs is
//     correctly rounded, from corrected hardware estimates (fo_device.hpp)
//     whose exactness fo_selftest checks on the device.
//   * A launch covers a range of the step's wave tiles with one wave per tile
//     (the host issues one launch per 2^18 tiles; the tile loop below also
//     serves smaller grids).  A tile never crosses a tensor, and the last tile
//     of a tensor takes a masked path; the tensor of a tile is found through a
//     tile-bucket index built by the host.
//   * Each wave of a fused step copies the 6-KiB codec tables into its own
//     LDS with asynchronous buffer-to-LDS loads issued ahead of its tile's
//     loads; no wave waits for another, so these kernels run one wave per
//     workgroup (four for AdamW with a 16-bit ECC, see adamw_tile_waves).
//   * Rare inputs (NaN/Inf/overflowing weights, tiny variances, out-of-range
//     denominators) leave the fast arithmetic through wave-uniform branches
//     onto IEEE sequences; the results are identical either way.
// Pages: FlashOptim thread (Davis Blalock) and the blog "FlashOptim: Breaking
// the Memory Wall with 24-bit Weights and Companded States" (Methodology
// sections 1 and 2) define what is computed; the launch structure is ours.
#pragma once

#include "fo_device.hpp"

namespace fo {

constexpr int WAVE = 64;
constexpr int EPL = 8;                     // elements per lane per sub-tile
constexpr int SUB = WAVE * EPL;            // 512
constexpr int NSUB = 4;
constexpr int TILE = SUB * NSUB;           // 2048 elements per wave tile
constexpr int WAVES_PER_WG = 4;           // element-wise kernels
constexpr int WG = WAVE * WAVES_PER_WG;    // 256 threads
// Waves per workgroup of the tile kernels (fused steps, stream probe).  A wave
// needs nothing from its neighbours (private LDS tables, no barrier), and a
// one-wave group releases its slot and LDS as soon as its tile is done: on the
// Llama-8B list that measured 16.74-16.76 -> 16.58 ms against 4-wave groups.
// The AdamW kernels with a 16-bit ECC (176 VGPRs, two waves per SIMD) ran
// 1.6% slower that way and keep 4-wave groups.
template <int ECC> constexpr int adamw_tile_waves = (ECC == 16) ? 4 : 1;
constexpr int SGDM_TILE_WAVES = 1;
// Block ownership (lane 4Q+j owns block 16j+Q of the tile) needs exactly one
// sub-tile per lane of a quad: 4 sub-tiles, 64 blocks, 64 lanes.
static_assert(NSUB == 4 && TILE / 32 == WAVE, "one owned block per lane");

// Device copy of one tensor of a step (built by the host launcher).  The
// launch table is the non-empty tensors' descriptors, a sentinel (tile_begin =
// total tiles, n = the bucket shift) and an int32 tile-bucket index: entry b
// is the tensor holding tile b << shift.
constexpr int TILE_BUCKET_SHIFT_MIN = 8;
struct alignas(16) TensorDesc {
  uint64_t w16, ecc, grad, q1, s1, q2, s2;  // q2/s2 unused by SGD-M
  int64_t n;
  int64_t tile_begin;                       // first global wave-tile index
};
static_assert(sizeof(TensorDesc) == 80, "descriptor layout");

struct AdamWConsts {
  float b1, b2, omb1, omb2, decay, step_size, ibc2, eps;
  float wd;         // coupled (L2) weight decay of Adam; unused by AdamW
  // Range of (effective) gradients for which the exact fast arithmetic holds:
  // g = 0 or g_lo <= |g| <= g_hi.  The host derives it from the
  // hyperparameters and the ranges of the decoded states, so that every
  // variance lies outside (0, 2^-96), every denominator in [eps, 2^126), every
  // nonzero momentum at or above 2^-100 and every quotient below 2^120
  // (the preconditions of sqrt_fast, rcp_refined and div_refined).
  uint32_t g_lo2;   // 2 * bits(g_lo) - 2: compared with 2 * bits(g) - 2
  float g_hi;
  // the same range on the 16-bit gradient patterns' magnitudes a (AdamW):
  // a = 0 or g16_lo < a <= g16_hi, g16_lo the largest pattern below g_lo
  uint32_t g16_lo, g16_hi;
  int fast;         // 0: no such range (e.g. eps = 0); every wave takes the IEEE form
};
struct SGDMConsts {
  float lr, mu, wd;
  float damp1;    // 1 - dampening
  int nesterov;
  int first;      // step 1 (and every step at momentum 0): the buffer is set to d
};

template <typename T> using gp = FO_GLOBAL T*;

// ---------------------------------------------------------------------------
// vector access (masked for the last, partial tile of a tensor)
// ---------------------------------------------------------------------------
// Every stream is touched once per step, so full-group loads and stores (and
// the block-scale accesses of the fused steps) carry the nontemporal hint.
// Measured on MI355X (Llama-8B list): 19.1 -> 17.8 ms; the hint on loads only
// or on stores only changes nothing.
template <int NDW>
struct DW { uint32_t w[NDW]; };

// load 8 elements of ESZ bytes (2*ESZ dwords)
template <int ESZ, bool FULL>
__device__ __forceinline__ DW<2 * ESZ> load8(gp<const uint8_t> base, int cnt) {
  DW<2 * ESZ> r;
  if (FULL || cnt >= 8) {
    if constexpr (ESZ == 2) {
      const u32x4 v = __builtin_nontemporal_load((gp<const u32x4>)base);
      r.w[0] = v.x; r.w[1] = v.y; r.w[2] = v.z; r.w[3] = v.w;
    } else {
      const u32x2 v = __builtin_nontemporal_load((gp<const u32x2>)base);
      r.w[0] = v.x; r.w[1] = v.y;
    }
    return r;
  }
#pragma unroll
  for (int i = 0; i < 2 * ESZ; ++i) r.w[i] = 0;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    if (k < cnt) {
      uint32_t x;
      if constexpr (ESZ == 2) x = ((gp<const uint16_t>)base)[k];
      else x = base[k];
      r.w[(k * ESZ) >> 2] |= x << (8 * ((k * ESZ) & 3));
    }
  }
  return r;
}

template <int ESZ, bool FULL>
__device__ __forceinline__ void store8(gp<uint8_t> base, const uint32_t* w, int cnt) {
  if (FULL || cnt >= 8) {
    if constexpr (ESZ == 2) __builtin_nontemporal_store(u32x4{w[0], w[1], w[2], w[3]}, (gp<u32x4>)base);
    else __builtin_nontemporal_store(u32x2{w[0], w[1]}, (gp<u32x2>)base);
    return;
  }
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    if (k < cnt) {
      const uint32_t x = w[(k * ESZ) >> 2] >> (8 * ((k * ESZ) & 3));
      if constexpr (ESZ == 2) ((gp<uint16_t>)base)[k] = (uint16_t)x;
      else base[k] = (uint8_t)x;
    }
  }
}

// 8 4-bit codes of a lane (one word; element i in bits [4i, 4i+4)).  A
// partial group of cnt < 8 elements reads and writes the (cnt+1)/2 bytes
// that hold them; the unused high nibble of an odd count is written as 0.
template <bool FULL>
__device__ __forceinline__ DW<1> load_nib8(gp<const uint8_t> base, int cnt) {
  DW<1> r;
  if (FULL || cnt >= 8) {
    r.w[0] = __builtin_nontemporal_load((gp<const uint32_t>)base);
    return r;
  }
  r.w[0] = 0;
#pragma unroll
  for (int b = 0; b < 4; ++b)
    if (2 * b < cnt) r.w[0] |= (uint32_t)base[b] << (8 * b);
  return r;
}
template <bool FULL>
__device__ __forceinline__ void store_nib8(gp<uint8_t> base, uint32_t w, int cnt) {
  if (FULL || cnt >= 8) {
    __builtin_nontemporal_store(w, (gp<uint32_t>)base);
    return;
  }
  w &= (1u << (4 * cnt)) - 1u;                 // cnt < 8: the nibbles past the end are 0
#pragma unroll
  for (int b = 0; b < 4; ++b)
    if (2 * b < cnt) base[b] = (uint8_t)(w >> (8 * b));
}
// the code words of 8 elements under a codec: 2 words of bytes or 1 of nibbles
template <int CODEC> constexpr int code_words = code_bits<CODEC> / 4;
template <int CODEC, bool FULL>
__device__ __forceinline__ DW<code_words<CODEC>> load_codes(gp<const uint8_t> base, int cnt) {
  if constexpr (CODEC == COMPANDED4) return load_nib8<FULL>(base, cnt);
  else return load8<1, FULL>(base, cnt);
}
template <int CODEC, bool FULL>
__device__ __forceinline__ void store_codes(gp<uint8_t> base, const uint32_t* w, int cnt) {
  if constexpr (CODEC == COMPANDED4) store_nib8<FULL>(base, w[0], cnt);
  else store8<1, FULL>(base, w, cnt);
}

// element k of a packed group.  A nibble word splits once into the nibbles
// of its even and of its odd elements, one per byte (NibHalves), so each
// element is then a byte select, which the byte-operand forms of the
// conversions and shifts take at no cost.  The empty asm statements emit
// nothing; they keep the compiler from folding the split back into one bit
// extract per element.
struct NibHalves { uint32_t ev, od; };
__device__ __forceinline__ NibHalves nib_halves(uint32_t w) {
  NibHalves h{w & 0x0F0F0F0Fu, (w >> 4) & 0x0F0F0F0Fu};
  asm("" : "+v"(h.ev));
  asm("" : "+v"(h.od));
  return h;
}
__device__ __forceinline__ uint32_t nib4(const NibHalves& h, int k) {
  return (((k & 1) ? h.od : h.ev) >> (8 * (k >> 1))) & 0xFFu;
}
// the decode operand of a lane's loaded code words
template <int CODEC>
__device__ __forceinline__ auto code_operand(const DW<code_words<CODEC>>& q) {
  if constexpr (CODEC == COMPANDED4) return nib_halves(q.w[0]);
  else return q;
}
__device__ __forceinline__ int32_t s8(const DW<2>& v, int k) {
  return ((int32_t)(v.w[k >> 2] << (24 - 8 * (k & 3)))) >> 24;
}
__device__ __forceinline__ uint32_t u8(const DW<2>& v, int k) { return (v.w[k >> 2] >> (8 * (k & 3))) & 0xFFu; }
__device__ __forceinline__ int32_t s16(const DW<4>& v, int k) {
  return ((int32_t)(v.w[k >> 1] << (16 - 16 * (k & 1)))) >> 16;
}
template <int WFMT>
__device__ __forceinline__ float wid(const DW<4>& v, int k) {
  return widen<WFMT>(v.w[k >> 1], k & 1);
}
template <int ECC>
__device__ __forceinline__ int32_t rho_at(const DW<ECC / 4>& e, int k) {
  if constexpr (ECC == 8) return s8(e, k);
  else return s16(e, k);
}

__device__ __forceinline__ float bcast_j(float x, int j) {   // j is a compile-time constant after unrolling
  return j == 0 ? quad_bcast<0>(x) : j == 1 ? quad_bcast<1>(x) : j == 2 ? quad_bcast<2>(x) : quad_bcast<3>(x);
}

// ---------------------------------------------------------------------------
// state codecs inside a tile
// ---------------------------------------------------------------------------
enum { MOMENTUM_STATE = 0, VARIANCE_STATE = 1 };

// decode multiplier of a block with scale s (see the codec summary in
// fo_device.hpp).  The level spacings RN(s/127), RN(s/255), RN(s*s/255) are
// correctly rounded divisions by a constant: div_refined with the constant's
// rounded reciprocal (exact for every dividend: the CPU check covers all
// divisors with 11-bit significands).  A non-finite s divides to itself.  A
// bfloat16 scale may lie below the fast division's dividend range (2^-100):
// such a block's spacing is one IEEE division.
template <int KIND, int CODEC>
__device__ __forceinline__ float decode_mult(float s) {
  constexpr int CC = code_codec<CODEC>;
  // RN(1/127), RN(1/255), RN(1/15)
  constexpr float R127 = 1.0f / 127.0f, R255 = 1.0f / 255.0f, R15 = 1.0f / 15.0f;
  if constexpr (KIND == MOMENTUM_STATE && CC != LINEAR) return s;
  const float x = (KIND == VARIANCE_STATE && CC == LINEAR) ? s * s : s;
  const float q = (CC == COMPANDED4)          ? div_refined(x, 15.0f, R15)
                  : (KIND == MOMENTUM_STATE) ? div_refined(x, 127.0f, R127)
                                             : div_refined(x, 255.0f, R255);
  if constexpr (scale_bf16<CODEC>) return (fabsf(x) >= 0x1p-100f && fabsf(x) <= 0x1p126f) ? q : x / 255.0f;
  return (fabsf(x) <= 0x1p126f) ? q : x;
}
// q: the lane's code words of 8 elements (DW<2> of bytes, or the NibHalves
// of one nibble word under COMPANDED4)
template <int KIND, int CODEC, class QW>
__device__ __forceinline__ float decode_state(const QW& q, int i, float dm, const CodecTables& T) {
  if constexpr (CODEC == COMPANDED4) {
    if constexpr (KIND == MOMENTUM_STATE) {
      return dm * T.lut4[nib4(q, i)];
    } else {
      const float t = dm * (float)nib4(q, i);
      return t * t;
    }
  } else if constexpr (KIND == MOMENTUM_STATE) {
    const int32_t c = s8(q, i);
    return (CODEC == COMPANDED) ? dm * T.lut[c + LUT_BIAS] : dm * (float)c;
  } else {
    const float t = dm * (float)u8(q, i);
    return (CODEC == COMPANDED) ? t * t : t;
  }
}
// The value a state's block maximum and its codes are taken from: the state
// itself, or for a variance-kind state under a companded codec its square
// root (which the rule supplies).
template <int KIND, int CODEC> constexpr bool encodes_root = (KIND == VARIANCE_STATE && CODEC != LINEAR);

// ---------------------------------------------------------------------------
// update rules
// ---------------------------------------------------------------------------
// A fused step is one pass per element: widen the gradient, reconstruct the
// f32 master, decode the rule's states, apply the rule, split the new master,
// recompute the block scales of the new states and re-encode them.  All of it
// but the rule is shared (fused_tile below).  A rule is a type with
//   static constexpr int NSTATE;               1 or 2 stored 8-bit states
//   template <int K> static constexpr int KIND; MOMENTUM_STATE (int8 codes,
//                                              softsign-like compander) or
//                                              VARIANCE_STATE (uint8 codes,
//                                              square-root compander)
//   using Consts = ...;                        per-step scalars from the host
//   template <int NSUB> static bool tile_slow(const Consts&,
//                      const DW<4> (&G)[NSUB]);  the tile's 16-bit gradient
//                                              words as loaded: true (wave-
//                                              uniform) asks for the IEEE form
//   static void update(const Consts&, bool ieee, float (&th)[EPL],
//                      const float (&g)[EPL], float (&st)[NSTATE][EPL],
//                      float (&root)[NSTATE][EPL]);
// update() gets the decoded master th, the widened gradient g and the decoded
// states st of EPL elements of one lane, and leaves the new master in th and
// the new states in st.  For each VARIANCE_STATE it also leaves the correctly
// rounded square root of the new state in root (only read under the companded
// codec).  The whole wave calls update() together, so a rule may branch
// wave-uniformly (ballot) between a fast exact form and the IEEE form; ieee
// (wave-uniform) asks for the IEEE form, because a stored scale of the tile is
// not finite or tile_slow said so.  A new rule needs a kernel that runs
// fused_tile with it and a host entry point that fills its Consts.

// AdamW (decoupled decay) or, with L2, Adam (decay added to the gradient):
// m = b1*m + (1-b1)*g; v = b2*v + (1-b2)*g*g; th = th*decay;
// th = th - step_size * (m / (sqrt(v)*ibc2 + eps)), each operation one IEEE
// rounding (division and square root correctly rounded).
// the two ways out of the fast range, each one compare: 0 < |g| < g_lo
// (2*bits(g) - 2 wraps to the top for g = +-0), and |g| > g_hi or NaN
__device__ __forceinline__ bool grad_below_fast_range(float g, uint32_t lo2) { return ((f2u(g) << 1) - 2u) < lo2; }
__device__ __forceinline__ bool grad_above_fast_range(float g, float hi) { return !(fabsf(g) <= hi); }
// The same test for a whole tile of 16-bit gradients, on the words as
// loaded: with a the magnitude pattern of a gradient (monotone in |g|, NaN
// above infinity), a gradient is out of range when a > g16_hi, or when
// a - 1 < g16_lo (a - 1 wraps to 0xFFFF for a = 0).  Two packed 16-bit
// maxima / minima per word keep the largest a and the smallest a - 1 of the
// lane; wave-uniform result.
typedef uint16_t u16x2 __attribute__((ext_vector_type(2)));
template <int NSUBT>
__device__ __forceinline__ bool tile_grads_out_of_range(const DW<4> (&G)[NSUBT], uint32_t g16_lo, uint32_t g16_hi) {
  u16x2 mx = {0, 0}, mn = {0xFFFF, 0xFFFF};
  const u16x2 one = {1, 1};
#pragma unroll
  for (int j = 0; j < NSUBT; ++j)
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const u16x2 a = __builtin_bit_cast(u16x2, G[j].w[w] & 0x7FFF7FFFu);
      mx = __builtin_elementwise_max(mx, a);
      mn = __builtin_elementwise_min(mn, a - one);
    }
  const uint32_t hi = max((uint32_t)mx.x, (uint32_t)mx.y), lo = min((uint32_t)mn.x, (uint32_t)mn.y);
  return __builtin_amdgcn_ballot_w64(hi > g16_hi || lo < g16_lo) != 0;
}
template <bool L2>
struct AdamWRule {
  static constexpr int NSTATE = 2;
  template <int K> static constexpr int KIND = (K == 0) ? MOMENTUM_STATE : VARIANCE_STATE;
  using Consts = AdamWConsts;
  // AdamW's gradient is the 16-bit input: its range is checked once per tile
  // on the loaded words; Adam's effective gradient g + wd*th is checked
  // element by element in update()
  template <int NSUBT>
  static __device__ __forceinline__ bool tile_slow(const Consts& c, const DW<4> (&G)[NSUBT]) {
    if constexpr (L2) return false;
    else return tile_grads_out_of_range(G, c.g16_lo, c.g16_hi);
  }
  static __device__ __forceinline__ void update(const Consts& c, bool ieee, float (&th)[EPL], const float (&g)[EPL],
                                                float (&st)[2][EPL], float (&root)[2][EPL]) {
    uint64_t slow = (c.fast && !ieee) ? 0ull : ~0ull;
#pragma unroll
    for (int k = 0; k < EPL; ++k) {
      float gk = g[k];
      if constexpr (L2) gk = gk + c.wd * th[k];
      st[0][k] = c.b1 * st[0][k] + c.omb1 * gk;
      st[1][k] = c.b2 * st[1][k] + c.omb2 * (gk * gk);
      th[k] = th[k] * c.decay;
      if constexpr (L2)
        slow |= __builtin_amdgcn_ballot_w64(grad_below_fast_range(gk, c.g_lo2)) |
                __builtin_amdgcn_ballot_w64(grad_above_fast_range(gk, c.g_hi));
    }
    float q[EPL];
    if (!slow) {
#pragma unroll
      for (int k = 0; k < EPL; ++k) {
        root[1][k] = sqrt_fast(st[1][k]);
        const float den = root[1][k] * c.ibc2 + c.eps;
        q[k] = div_refined(st[0][k], den, rcp_refined(den));
      }
    } else {
#pragma unroll
      for (int k = 0; k < EPL; ++k) {
        root[1][k] = __builtin_sqrtf(st[1][k]);
        const float den = root[1][k] * c.ibc2 + c.eps;
        q[k] = st[0][k] / den;
      }
    }
#pragma unroll
    for (int k = 0; k < EPL; ++k) th[k] = th[k] - c.step_size * q[k];
  }
};

// SGD with momentum (torch.optim.SGD): d = g + wd*th; b = d at the first step
// (and every step at momentum 0), else b = mu*b + (1-dampening)*d;
// th = th - lr * (Nesterov ? d + mu*b : b).
struct SGDMRule {
  static constexpr int NSTATE = 1;
  template <int K> static constexpr int KIND = MOMENTUM_STATE;
  using Consts = SGDMConsts;
  template <int NSUBT>
  static __device__ __forceinline__ bool tile_slow(const Consts&, const DW<4> (&)[NSUBT]) { return false; }
  static __device__ __forceinline__ void update(const Consts& c, bool, float (&th)[EPL], const float (&g)[EPL],
                                                float (&st)[1][EPL], float (&)[1][EPL]) {
#pragma unroll
    for (int k = 0; k < EPL; ++k) {
      const float dd = g[k] + c.wd * th[k];
      const float b = c.first ? dd : c.mu * st[0][k] + c.damp1 * dd;
      const float u = c.nesterov ? dd + c.mu * b : b;
      th[k] = th[k] - c.lr * u;
      st[0][k] = b;
    }
  }
};

// ---------------------------------------------------------------------------
// codes of 8 elements of a lane
// ---------------------------------------------------------------------------
// x holds what the codes are taken from (the state, or the variance's square
// root under a companded codec), s the block's divisor and R = RN(1/s);
// ieee (wave-uniform) selects the forms that take any x and s.  o receives
// the packed codes: 2 words of bytes, or 1 word of nibbles.
template <int CODEC>
__device__ __forceinline__ void encode_group(int kind, const float (&x)[EPL], float s, float R, bool ieee,
                                             const CodecTables& tabs, uint32_t* o) {
  static_assert(EPL == 8, "8 codes per lane");
  if (kind == MOMENTUM_STATE) {
    uint32_t q[EPL];
    if (!ieee) {
#pragma unroll
      for (int i = 0; i < EPL; ++i)
        q[i] = (uint32_t)((CODEC == LINEAR)      ? encode_m_linear(x[i], s, R)
                          : (CODEC == COMPANDED) ? encode_m_companded<8>(x[i], s, R, tabs)
                                                 : encode_m_companded<4>(x[i], s, R, tabs));
    } else {
#pragma unroll
      for (int i = 0; i < EPL; ++i)
        q[i] = (uint32_t)((CODEC == LINEAR)      ? encode_m_linear_ieee(x[i], s)
                          : (CODEC == COMPANDED) ? encode_m_companded_ieee<8>(x[i], s, tabs)
                                                 : encode_m_companded_ieee<4>(x[i], s, tabs));
    }
    if constexpr (CODEC == COMPANDED4) {
      o[0] = pack_nibbles(pack4_byte0(q[0], q[2], q[4], q[6]), pack4_byte0(q[1], q[3], q[5], q[7]));
    } else {
      o[0] = pack4_byte0(q[0], q[1], q[2], q[3]);
      o[1] = pack4_byte0(q[4], q[5], q[6], q[7]);
    }
  } else if constexpr (CODEC == COMPANDED4) {
    uint32_t ev = 0u, od = 0u;                 // codes of the even / odd elements, one per byte
    if (!ieee) {
#pragma unroll
      for (int i = 0; i < EPL; i += 2) {
        ev = encode_v4_into(x[i], s, R, i >> 1, ev);
        od = encode_v4_into(x[i + 1], s, R, i >> 1, od);
      }
    } else {
#pragma unroll
      for (int i = 0; i < EPL; i += 2) {
        ev |= encode_v4_ieee(x[i], s) << (4 * i);
        od |= encode_v4_ieee(x[i + 1], s) << (4 * i);
      }
    }
    o[0] = pack_nibbles(ev, od);
  } else {
    o[0] = o[1] = 0u;
    if (!ieee) {
#pragma unroll
      for (int i = 0; i < EPL; ++i) o[i >> 2] = encode_v_into(x[i], s, R, i & 3, o[i >> 2]);
    } else {
#pragma unroll
      for (int i = 0; i < EPL; ++i) o[i >> 2] = encode_v_into_ieee(x[i], s, i & 3, o[i >> 2]);
    }
  }
}

// ---------------------------------------------------------------------------
// fused step: one wave tile for any update rule
// ---------------------------------------------------------------------------
template <class R, int WFMT, int ECC, int CODEC, bool FULL>
__device__ __forceinline__ void fused_tile(const TensorDesc& d, int64_t e0, int lane, const CodecTables& tabs,
                                           const typename R::Consts& c) {
  constexpr int NS = R::NSTATE;
  constexpr int EB = ECC / 8;                                  // ECC bytes per element
  constexpr int K0 = R::template KIND<0>;
  constexpr int K1 = R::template KIND<NS - 1>;
  constexpr int CC = code_codec<CODEC>;                        // the codes' codec
  constexpr bool SBF = scale_bf16<CODEC>;                      // bfloat16 block scales
  constexpr int QW = code_words<CC>;                           // code words per lane and sub-tile
  const int Q = lane >> 2, p = lane & 3;
  const gp<const uint8_t> grad = (gp<const uint8_t>)d.grad + e0 * 2;
  const gp<uint8_t> w16 = (gp<uint8_t>)d.w16 + e0 * 2;
  const gp<uint8_t> ecc = (gp<uint8_t>)d.ecc + e0 * EB;
  gp<uint8_t> qp[NS];
  gp<uint16_t> sp[NS];
  qp[0] = (gp<uint8_t>)d.q1 + e0 * QW / 2;                    // code bytes: e0 or e0 / 2
  sp[0] = (gp<uint16_t>)d.s1 + (e0 >> 5);
  if constexpr (NS == 2) {
    qp[NS - 1] = (gp<uint8_t>)d.q2 + e0 * QW / 2;
    sp[NS - 1] = (gp<uint16_t>)d.s2 + (e0 >> 5);
  }
  const int64_t rem = d.n - e0;                                // valid elements from e0 on
  const int own = p * 16 + Q;                                  // owned block within the tile
  const bool own_ok = FULL || (int64_t)own * 32 < rem;

  // ---- issue the tile's loads ---------------------------------------------
  DW<4> G[NSUB], W[NSUB];
  DW<2 * EB> E[NSUB];
  DW<QW> SQ[NS][NSUB];
  int cnt[NSUB];
  // the gradients first: the rule's tile-wide range check waits for them
  // only (the vector memory counter retires loads in issue order)
#pragma unroll
  for (int j = 0; j < NSUB; ++j) {
    const int off = j * SUB + lane * EPL;
    cnt[j] = FULL ? 8 : (int)max((int64_t)0, min((int64_t)8, rem - off));
    G[j] = load8<2, FULL>(grad + off * 2, cnt[j]);
  }
  // master, ECC and state codes of sub-tile j
  auto issue_loads = [&](int j) {
    const int off = j * SUB + lane * EPL;
    W[j] = load8<2, FULL>(w16 + off * 2, cnt[j]);
    E[j] = load8<EB, FULL>(ecc + off * EB, cnt[j]);
#pragma unroll
    for (int k = 0; k < NS; ++k) SQ[k][j] = load_codes<CC, FULL>(qp[k] + off * QW / 2, cnt[j]);
  };
  // the first half now, the second half once sub-tile 0 is updated: fewer
  // bytes in flight per wave at once measure about 0.7% faster on every
  // format than issuing the whole tile up front (one sub-tile ahead is slower)
  static_assert(NSUB == 4, "loads issued in two halves of two sub-tiles");
  issue_loads(0);
  issue_loads(1);
  float dm_own[NS];
  bool nonfinite = false;
#pragma unroll
  for (int k = 0; k < NS; ++k) {
    const float sold = scale_f32<CODEC>(own_ok ? (uint32_t)__builtin_nontemporal_load(sp[k] + own) : 0u);
    dm_own[k] = (k == 0) ? decode_mult<K0, CODEC>(sold) : decode_mult<K1, CODEC>(sold);
    nonfinite |= SBF ? !scale_in_fast_range(sold) : !(fabsf(sold) <= 65504.0f);
  }
  // a NaN or infinite stored scale (the encoder writes NaN only for an all-NaN
  // block) makes NaN or infinite states, and a bfloat16 scale outside the
  // fast range states the fast update does not take: the rule then takes its
  // IEEE form (or the rule finds the tile's gradients outside its fast range)
  const bool ieee = (__builtin_amdgcn_ballot_w64(nonfinite) != 0) || R::tile_slow(c, G);

  float X[NS][NSUB][EPL];                  // what each state's codes are taken from
  float own_max[NS];
#pragma unroll
  for (int k = 0; k < NS; ++k) own_max[k] = 0.0f;

#pragma unroll
  for (int j = 0; j < NSUB; ++j) {
    float th[EPL], g[EPL], st[NS][EPL], root[NS][EPL];
    float dm[NS];
#pragma unroll
    for (int k = 0; k < NS; ++k) dm[k] = bcast_j(dm_own[k], j);
    const auto q0 = code_operand<CC>(SQ[0][j]);
    const auto q1 = code_operand<CC>(SQ[NS - 1][j]);
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      g[i] = wid<WFMT>(G[j], i);
      if constexpr (WFMT == BF16)
        th[i] = ecc_decode_bf16_packed<ECC>(W[j].w[i >> 1], E[j].w[(i * ECC) >> 5], i & 1, (ECC == 8) ? (i & 3) : (i & 1));
      else
        th[i] = ecc_decode<WFMT, ECC>(wid<WFMT>(W[j], i), rho_at<ECC>(E[j], i));
      st[0][i] = decode_state<K0, CC>(q0, i, dm[0], tabs);
      if constexpr (NS == 2) st[NS - 1][i] = decode_state<K1, CC>(q1, i, dm[NS - 1], tabs);
    }
    R::update(c, ieee, th, g, st, root);
    if (j == 0) {                       // the barriers keep the second half here
      __builtin_amdgcn_sched_barrier(0);
      issue_loads(2);
      issue_loads(3);
      __builtin_amdgcn_sched_barrier(0);
    }

    // split the new master and store it
    uint32_t wo[4], eo[ECC / 4];
    split8<WFMT, ECC>(th, wo, eo);
    const int off = j * SUB + lane * EPL;
    store8<2, FULL>(w16 + off * 2, wo, cnt[j]);
    store8<EB, FULL>(ecc + off * EB, eo, cnt[j]);

    // block maxima: maxNum skips NaN, and lanes past the end of a short last
    // block feed NaN, so only the block's valid elements count and a block
    // whose valid elements are all NaN keeps a NaN maximum (and scale)
#pragma unroll
    for (int k = 0; k < NS; ++k) {
      const bool root_k = (k == 0) ? encodes_root<K0, CC> : encodes_root<K1, CC>;
      const bool mom_k = ((k == 0) ? K0 : K1) == MOMENTUM_STATE;
      float a[EPL];
#pragma unroll
      for (int i = 0; i < EPL; ++i) {
        const float x = root_k ? root[k][i] : st[k][i];
        X[k][j][i] = x;
        a[i] = (FULL || i < cnt[j]) ? x : __builtin_nanf("");
      }
      static_assert(EPL == 8, "maxima of 8 elements per lane");
      float mx = mom_k ? max_abs_quiet(a[0], a[1]) : max_quiet(a[0], a[1]);
#pragma unroll
      for (int i = 2; i < EPL; i += 2) mx = mom_k ? max3_abs_quiet(mx, a[i], a[i + 1]) : max3_quiet(mx, a[i], a[i + 1]);
      mx = quad_max(mx);
      own_max[k] = (p == j) ? mx : own_max[k];
    }
  }

  // ---- new block scales and encode constants (owned block) ---------------
  float s_own[NS], r_own[NS];
  bool sat = false;
#pragma unroll
  for (int k = 0; k < NS; ++k) {
    const int kind = (k == 0) ? K0 : K1;
    const bool lin_var = (kind == VARIANCE_STATE && CC == LINEAR);
    const uint32_t sb = SBF ? ru_bf16(own_max[k]) : ru_fp16(lin_var ? __builtin_sqrtf(own_max[k]) : own_max[k]);
    if (own_ok) __builtin_nontemporal_store((uint16_t)sb, sp[k] + own);
    const float sf = scale_f32<CODEC>(sb);
    s_own[k] = lin_var ? sf * sf : sf;                       // the divisor of the normalisation (exact)
    // RN(1/divisor) for the fast encodes; a zero divisor gives NaN, which
    // codes the block's zeros (and NaNs) 0 as the division 0/0 would
    r_own[k] = rcp_refined(s_own[k]);
    // the fast encodes need |x| <= s (momentum, and 4-bit variance, whose
    // conversion saturates at 255 instead of 15) or a finite x (variance)
    sat |= (kind == MOMENTUM_STATE || CC == COMPANDED4) ? (own_max[k] > 65504.0f)
                                                        : (own_max[k] == __builtin_inff());
    if constexpr (SBF) sat |= !scale_in_fast_range(sf);
  }
  const bool sat_wave = __builtin_amdgcn_ballot_w64(sat) != 0;

#pragma unroll
  for (int j = 0; j < NSUB; ++j) {
    const int off = j * SUB + lane * EPL;
#pragma unroll
    for (int k = 0; k < NS; ++k) {
      const int kind = (k == 0) ? K0 : K1;
      const float sdiv = bcast_j(s_own[k], j), rdiv = bcast_j(r_own[k], j);
      uint32_t o[QW];
      encode_group<CC>(kind, X[k][j], sdiv, rdiv, sat_wave, tabs, o);
      store_codes<CC, FULL>(qp[k] + off * QW / 2, o, cnt[j]);
    }
  }
}

// ---------------------------------------------------------------------------
// stream probe: the byte streams of one fused AdamW tile, no arithmetic
// ---------------------------------------------------------------------------
template <int ECC, bool FULL>
__device__ __forceinline__ void probe_tile(const TensorDesc& d, int64_t e0, int lane, uint32_t key) {
  constexpr int EB = ECC / 8;
  const int Q = lane >> 2, p = lane & 3;
  const gp<const uint8_t> grad = (gp<const uint8_t>)d.grad + e0 * 2;
  const gp<uint8_t> w16 = (gp<uint8_t>)d.w16 + e0 * 2;
  const gp<uint8_t> ecc = (gp<uint8_t>)d.ecc + e0 * EB;
  const gp<uint8_t> mq = (gp<uint8_t>)d.q1 + e0;
  const gp<uint8_t> vq = (gp<uint8_t>)d.q2 + e0;
  const gp<uint16_t> ms = (gp<uint16_t>)d.s1 + (e0 >> 5);
  const gp<uint16_t> vs = (gp<uint16_t>)d.s2 + (e0 >> 5);
  const int64_t rem = d.n - e0;
  const int own = p * 16 + Q;
  const bool own_ok = FULL || (int64_t)own * 32 < rem;
  DW<4> G[NSUB], W[NSUB];
  DW<2 * EB> E[NSUB];
  DW<2> MQ[NSUB], VQ[NSUB];
  int cnt[NSUB];
  // the gradients first: the rule's tile-wide range check waits for them
  // only (the vector memory counter retires loads in issue order)
#pragma unroll
  for (int j = 0; j < NSUB; ++j) {
    const int off = j * SUB + lane * EPL;
    cnt[j] = FULL ? 8 : (int)max((int64_t)0, min((int64_t)8, rem - off));
    G[j] = load8<2, FULL>(grad + off * 2, cnt[j]);
  }
  // the same two halves as the fused tile
  auto issue_loads = [&](int j) {
    const int off = j * SUB + lane * EPL;
    W[j] = load8<2, FULL>(w16 + off * 2, cnt[j]);
    E[j] = load8<EB, FULL>(ecc + off * EB, cnt[j]);
    MQ[j] = load8<1, FULL>(mq + off, cnt[j]);
    VQ[j] = load8<1, FULL>(vq + off, cnt[j]);
  };
  issue_loads(0);
  issue_loads(1);
  const uint32_t sm = own_ok ? (uint32_t)ms[own] : 0u;
  const uint32_t sv = own_ok ? (uint32_t)vs[own] : 0u;
#pragma unroll
  for (int j = 0; j < NSUB; ++j) {
    // fold the gradient into the key so it is really read
    const uint32_t k2 = key & (G[j].w[0] ^ G[j].w[1] ^ G[j].w[2] ^ G[j].w[3]);
#pragma unroll
    for (int i = 0; i < 4; ++i) W[j].w[i] ^= k2;
#pragma unroll
    for (int i = 0; i < 2 * EB; ++i) E[j].w[i] ^= key;
    MQ[j].w[0] ^= key; MQ[j].w[1] ^= key; VQ[j].w[0] ^= key; VQ[j].w[1] ^= key;
    if (j == 0) {
      __builtin_amdgcn_sched_barrier(0);
      issue_loads(2);
      issue_loads(3);
      __builtin_amdgcn_sched_barrier(0);
    }
    const int off = j * SUB + lane * EPL;
    store8<2, FULL>(w16 + off * 2, W[j].w, cnt[j]);
    store8<EB, FULL>(ecc + off * EB, E[j].w, cnt[j]);
    store8<1, FULL>(mq + off, MQ[j].w, cnt[j]);
    store8<1, FULL>(vq + off, VQ[j].w, cnt[j]);
  }
  if (own_ok) { ms[own] = (uint16_t)(sm ^ key); vs[own] = (uint16_t)(sv ^ key); }
}

// ---------------------------------------------------------------------------
// HBM probe: plain read, write, copy or in-place update streams in the fused
// kernels' access style (16-byte nontemporal accesses, each instruction
// covering 1 KiB), one wave per chunk of U KiB
// ---------------------------------------------------------------------------
template <int U>
__global__ void __launch_bounds__(WAVE) k_hbm_probe(uint8_t* dst, const uint8_t* src, int64_t chunk0, int mode,
                                                    uint32_t key) {
  const int lane = threadIdx.x;
  const int64_t base = (chunk0 + blockIdx.x) * (int64_t)(1024 * U) + lane * 16;
  if (mode == 1) {
#pragma unroll
    for (int i = 0; i < U; ++i)
      __builtin_nontemporal_store(u32x4{key, key, key, key}, (gp<u32x4>)(dst + base + i * 1024));
    return;
  }
  u32x4 v[U];
#pragma unroll
  for (int i = 0; i < U; ++i) v[i] = __builtin_nontemporal_load((gp<const u32x4>)(src + base + i * 1024));
  if (mode >= 2) {                         // 2: copy to dst; 3: dst updated in place (src == dst)
#pragma unroll
    for (int i = 0; i < U; ++i) __builtin_nontemporal_store(v[i] ^ key, (gp<u32x4>)(dst + base + i * 1024));
    return;
  }
  uint32_t acc = 0;
#pragma unroll
  for (int i = 0; i < U; ++i) acc ^= v[i].x ^ v[i].y ^ v[i].z ^ v[i].w;
  if (acc == key) ((gp<uint32_t>)dst)[0] = acc;   // keeps the loads; key is chosen not to match
}

// ---------------------------------------------------------------------------
// multi-tensor kernels
// ---------------------------------------------------------------------------
__device__ __forceinline__ int find_tensor(const TensorDesc* __restrict__ tab, int count, int64_t T) {
  // the tensor of tile T lies between the entries of T's bucket and the next
  const int shift = (int)tab[count].n;
  const int32_t* bk = reinterpret_cast<const int32_t*>(tab + count + 1);
  const int64_t b = T >> shift;
  int lo = bk[b], hi = bk[b + 1];          // largest t in [lo, hi] with tile_begin <= T
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (tab[mid].tile_begin <= T) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// Waves stride over the tiles [tile0, tile_end) of the step's global wave-tile
// list (one tile per wave with the default flat grid).  When a wave leaves its tensor, the tensor of
// its tile is found through the tile-bucket index (a short binary search over
// the first-tile indices of one bucket's tensors).
template <int WPG, typename F>
__device__ __forceinline__ void tile_loop(const TensorDesc* __restrict__ tab, int count, int64_t tile0,
                                          int64_t tile_end, F&& body) {
  const int lane = threadIdx.x & (WAVE - 1);
  const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t nwaves = (int64_t)gridDim.x * WPG;
  int t = 0;
  int64_t t_begin = 0, t_end = -1;
  for (int64_t T = tile0 + (int64_t)blockIdx.x * WPG + wid; T < tile_end; T += nwaves) {
    if (T >= t_end) {
      t = find_tensor(tab, count, T);
      t_begin = tab[t].tile_begin;
      t_end = tab[t + 1].tile_begin;
    }
    if (T < t_begin) continue;              // cannot happen with a well-formed table
    const TensorDesc d = tab[t];
    body(d, (T - t_begin) * TILE, lane);
  }
}

// copy the codec tables from global memory into the workgroup's LDS
__device__ __forceinline__ void load_tables(CodecTables& dst, const CodecTables* __restrict__ src) {
  constexpr int N16 = sizeof(CodecTables) / 16;
  const gp<const u32x4> s = (gp<const u32x4>)src;
  u32x4* d = (u32x4*)&dst;
  for (int i = threadIdx.x; i < N16; i += blockDim.x) d[i] = s[i];
  __syncthreads();
}

// Each wave of a fused step keeps its own LDS copy of the codec tables, filled
// by six asynchronous buffer->LDS loads (64 lanes x 16 B each) issued before
// the tile's own loads: the copy's latency overlaps the tile's instead of
// preceding it, and no workgroup barrier is needed, because a wave reads only
// the copy it filled.  The buffer form (not the global one) keeps the vector
// memory counter in order, so the first table read waits for these six loads
// only and the tile's loads still retire progressively.  The scheduling
// barrier keeps them ahead of the tile's loads.
typedef __attribute__((address_space(3))) void lds_void;
constexpr int BUFFER_RSRC_WORD3 = 0x00020000;   // raw buffer, 32-bit data format
// With one wave per workgroup the wave's copy is the workgroup's only LDS
// allocation: its address is the constant 0, so table addresses fold into the
// LDS instructions' offsets.
template <int WPG>
__device__ __forceinline__ const CodecTables& wave_tables(CodecTables* lds, const CodecTables* __restrict__ src) {
  constexpr int CHUNKS = sizeof(CodecTables) / (16 * WAVE);
  const int wid = (WPG == 1) ? 0 : __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & (WAVE - 1);
  const __amdgpu_buffer_rsrc_t r =
      __builtin_amdgcn_make_buffer_rsrc((void*)src, 0, (int)sizeof(CodecTables), BUFFER_RSRC_WORD3);
  u32x4* d = (u32x4*)(lds + wid);
#pragma unroll
  for (int i = 0; i < CHUNKS; ++i)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)(d + i * WAVE), 16, lane * 16 + i * 16 * WAVE, 0, 0, 0);
  __builtin_amdgcn_sched_barrier(0);
  return lds[wid];
}

// ---------------------------------------------------------------------------
// launch table written from kernel arguments (allocation-free entry point)
// ---------------------------------------------------------------------------
// A chunk of the descriptor array travels by value in the kernel arguments
// (copied at launch, or into the node of a captured graph), so nothing on the
// host has to outlive the call.  TABLE_CHUNK keeps the arguments far below
// the 4-KiB kernel-argument limit together with the implicit arguments.
constexpr int TABLE_CHUNK = 3072;
struct alignas(16) TableChunk {
  uint8_t data[TABLE_CHUNK];
  uint32_t offset;   // byte offset of the chunk in the table
  uint32_t bytes;    // a multiple of 16, at most TABLE_CHUNK
};
__global__ void __launch_bounds__(WG) k_put_table(uint8_t* __restrict__ dst, TableChunk c) {
  const int i = threadIdx.x;                       // one 16-byte word per thread
  if ((uint32_t)i * 16u < c.bytes) {
    const u32x4 v = reinterpret_cast<const u32x4*>(c.data)[i];
    ((gp<u32x4>)(dst + c.offset))[i] = v;
  }
}
static_assert(WG * 16 >= TABLE_CHUNK, "one workgroup writes a whole chunk");

// Tile-bucket index of a descriptor table already on the device: entry b
// (0 <= b < nbk) is the last tensor whose first tile is at or before
// min(b << shift, tiles - 1), found by binary search over tile_begin.
__global__ void __launch_bounds__(WG) k_bucket_index(const TensorDesc* __restrict__ tab, int count, int shift,
                                                     int nbk, int64_t tiles, int32_t* __restrict__ buckets) {
  const int b = blockIdx.x * WG + threadIdx.x;
  if (b >= nbk) return;
  const int64_t first = min((int64_t)b << shift, tiles - 1);
  int lo = 0, hi = count - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (tab[mid].tile_begin <= first) lo = mid; else hi = mid - 1;
  }
  buckets[b] = lo;
}

__global__ void __launch_bounds__(WG) k_init_tables(CodecTables* out) {
  __shared__ float thr[127 + 7];
  build_tables((gp<CodecTables>)out, thr, threadIdx.x, blockDim.x);
}

// ECC8: three waves per SIMD (at most 168 VGPRs), the occupancy the stream
// needs.  ECC16 holds more registers; forcing three waves there spills, and
// two waves without spills run faster.
template <int WFMT, int ECC, int CODEC, bool L2>
__global__ void __launch_bounds__(WAVE * adamw_tile_waves<ECC>) __attribute__((amdgpu_waves_per_eu(ECC == 8 ? 3 : 1)))
k_fused_adamw(const TensorDesc* __restrict__ tab, int count, int64_t tile0, int64_t tile_end,
              const CodecTables* __restrict__ gtabs, AdamWConsts c) {
  __shared__ CodecTables wtabs[adamw_tile_waves<ECC>];
  const CodecTables& tabs = wave_tables<adamw_tile_waves<ECC>>(wtabs, gtabs);
  tile_loop<adamw_tile_waves<ECC>>(tab, count, tile0, tile_end, [&](const TensorDesc& d, int64_t e0, int lane) {
    if (e0 + TILE <= d.n) fused_tile<AdamWRule<L2>, WFMT, ECC, CODEC, true>(d, e0, lane, tabs, c);
    else fused_tile<AdamWRule<L2>, WFMT, ECC, CODEC, false>(d, e0, lane, tabs, c);
  });
}

template <int WFMT, int ECC, int CODEC>
__global__ void __launch_bounds__(WAVE * SGDM_TILE_WAVES) k_fused_sgdm(const TensorDesc* __restrict__ tab, int count,
                                                                 int64_t tile0, int64_t tile_end,
                                                                 const CodecTables* __restrict__ gtabs, SGDMConsts c) {
  __shared__ CodecTables wtabs[SGDM_TILE_WAVES];
  const CodecTables& tabs = wave_tables<SGDM_TILE_WAVES>(wtabs, gtabs);
  tile_loop<SGDM_TILE_WAVES>(tab, count, tile0, tile_end, [&](const TensorDesc& d, int64_t e0, int lane) {
    if (e0 + TILE <= d.n) fused_tile<SGDMRule, WFMT, ECC, CODEC, true>(d, e0, lane, tabs, c);
    else fused_tile<SGDMRule, WFMT, ECC, CODEC, false>(d, e0, lane, tabs, c);
  });
}

// same launch shape as the AdamW step it is compared with
template <int ECC>
__global__ void __launch_bounds__(WAVE * adamw_tile_waves<ECC>) k_stream_probe(const TensorDesc* __restrict__ tab, int count,
                                                                        int64_t tile0, int64_t tile_end, uint32_t key) {
  tile_loop<adamw_tile_waves<ECC>>(tab, count, tile0, tile_end, [&](const TensorDesc& d, int64_t e0, int lane) {
    if (e0 + TILE <= d.n) probe_tile<ECC, true>(d, e0, lane, key);
    else probe_tile<ECC, false>(d, e0, lane, key);
  });
}

// ---------------------------------------------------------------------------
// standalone element-wise kernels (8 elements per thread, grid-stride)
// ---------------------------------------------------------------------------
template <int WFMT, int ECC>
__global__ void __launch_bounds__(WG) k_split(const float* __restrict__ x, int64_t n,
                                              uint16_t* __restrict__ w16, uint8_t* __restrict__ ecc) {
  constexpr int EB = ECC / 8;
  const gp<const float> xs = (gp<const float>)x;
  const int64_t stride = (int64_t)gridDim.x * WG * EPL;
  // every lane of a wave iterates together (the stride is a multiple of 512),
  // so the wave-uniform branches inside split8 see whole waves
  for (int64_t i0 = (int64_t)blockIdx.x * WG * EPL; i0 < n; i0 += stride) {
    const int64_t i = i0 + threadIdx.x * EPL;
    const int cnt = (int)max((int64_t)0, min((int64_t)8, n - i));
    float v[8];
    if (cnt == 8) {
      const f32x4 a = *(gp<const f32x4>)(xs + i), b = *(gp<const f32x4>)(xs + i + 4);
      v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    } else {
#pragma unroll
      for (int k = 0; k < 8; ++k) v[k] = (k < cnt) ? xs[i + k] : 0.0f;
    }
    uint32_t wo[4], eo[ECC / 4];
    split8<WFMT, ECC>(v, wo, eo);
    if (cnt == 8) {
      store8<2, true>((gp<uint8_t>)w16 + i * 2, wo, 8);
      store8<EB, true>((gp<uint8_t>)ecc + i * EB, eo, 8);
    } else if (cnt > 0) {
      store8<2, false>((gp<uint8_t>)w16 + i * 2, wo, cnt);
      store8<EB, false>((gp<uint8_t>)ecc + i * EB, eo, cnt);
    }
  }
}

template <int WFMT, int ECC>
__global__ void __launch_bounds__(WG) k_reconstruct(const uint16_t* __restrict__ w16, const uint8_t* __restrict__ ecc,
                                                    int64_t n, float* __restrict__ out) {
  constexpr int EB = ECC / 8;
  const gp<float> o = (gp<float>)out;
  const int64_t stride = (int64_t)gridDim.x * WG * EPL;
  for (int64_t i = ((int64_t)blockIdx.x * WG + threadIdx.x) * EPL; i < n; i += stride) {
    const int cnt = (int)min((int64_t)8, n - i);
    DW<4> W;
    DW<2 * EB> E;
    const gp<const uint8_t> wp = (gp<const uint8_t>)w16 + i * 2;
    const gp<const uint8_t> ep = (gp<const uint8_t>)ecc + i * EB;
    if (cnt == 8) { W = load8<2, true>(wp, 8); E = load8<EB, true>(ep, 8); }
    else { W = load8<2, false>(wp, cnt); E = load8<EB, false>(ep, cnt); }
    float v[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) v[k] = ecc_decode<WFMT, ECC>(wid<WFMT>(W, k), rho_at<ECC>(E, k));
    if (cnt == 8) {
      *(gp<f32x4>)(o + i) = f32x4{v[0], v[1], v[2], v[3]};
      *(gp<f32x4>)(o + i + 4) = f32x4{v[4], v[5], v[6], v[7]};
    } else {
#pragma unroll
      for (int k = 0; k < 8; ++k) if (k < cnt) o[i + k] = v[k];
    }
  }
}

// KIND 0 = momentum (int8, or signed nibbles under COMPANDED4), 1 = variance
// (uint8, or nibbles).  A quad of lanes = one block.
template <int KIND, int CODEC>
__global__ void __launch_bounds__(WG) k_quantize(const float* __restrict__ x, int64_t n,
                                                 uint8_t* __restrict__ codes, uint16_t* __restrict__ scales,
                                                 const CodecTables* __restrict__ gtabs) {
  __shared__ CodecTables tabs;
  load_tables(tabs, gtabs);
  constexpr int CC = code_codec<CODEC>;
  const gp<const float> xs = (gp<const float>)x;
  const int64_t stride = (int64_t)gridDim.x * WG * EPL;
  // all lanes iterate together (stride multiple of 512), so the 4 lanes of a
  // block are active at the same time; lanes past n contribute NaN to the
  // block maximum (skipped by maxNum) and store nothing
  for (int64_t i0 = (int64_t)blockIdx.x * WG * EPL; i0 < n; i0 += stride) {
    const int64_t i = i0 + threadIdx.x * EPL;
    const int cnt = (int)max((int64_t)0, min((int64_t)8, n - i));
    float v[8];
    if (cnt == 8) {
      const f32x4 a = *(gp<const f32x4>)(xs + i), b = *(gp<const f32x4>)(xs + i + 4);
      v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    } else {
#pragma unroll
      for (int k = 0; k < 8; ++k) v[k] = (k < cnt) ? xs[i + k] : __builtin_nanf("");
    }
    float e[8];
    if (KIND == 1 && CC != LINEAR) {
      uint64_t slow = 0;
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        e[k] = sqrt_corrected(v[k]);
        slow |= __builtin_amdgcn_ballot_w64(sqrt_needs_scaling(v[k]));
      }
      if (slow) {
#pragma unroll
        for (int k = 0; k < 8; ++k) e[k] = __builtin_sqrtf(v[k]);
      }
    } else {
#pragma unroll
      for (int k = 0; k < 8; ++k) e[k] = v[k];
    }
    float mx = __builtin_nanf("");            // all-NaN block -> NaN scale
#pragma unroll
    for (int k = 0; k < 8; ++k) mx = fmaxf(mx, (KIND == 0) ? fabsf(e[k]) : e[k]);
    mx = quad_max(mx);
    const uint32_t sb = scale_bf16<CODEC> ? ru_bf16(mx) : ru_fp16((KIND == 1 && CC == LINEAR) ? __builtin_sqrtf(mx) : mx);
    if ((threadIdx.x & 3) == 0 && cnt > 0) ((gp<uint16_t>)scales)[i >> 5] = (uint16_t)sb;
    const float sf = scale_f32<CODEC>(sb);
    const float sdiv = (KIND == 1 && CC == LINEAR) ? sf * sf : sf;
    const float rdiv = 1.0f / sdiv;
    const bool sat = ((KIND == 0 || CC == COMPANDED4) ? (mx > 65504.0f) : (mx == __builtin_inff())) ||
                     (scale_bf16<CODEC> && !scale_in_fast_range(sf));
    const bool sat_wave = __builtin_amdgcn_ballot_w64(sat) != 0;
    constexpr int QW = code_words<CC>;
    uint32_t o[QW];
    encode_group<CC>(KIND == 0 ? MOMENTUM_STATE : VARIANCE_STATE, e, sdiv, rdiv, sat_wave, tabs, o);
    const gp<uint8_t> cp = (gp<uint8_t>)codes + i * QW / 2;
    if (cnt == 8) store_codes<CC, true>(cp, o, 8);
    else if (cnt > 0) store_codes<CC, false>(cp, o, cnt);
  }
}

template <int KIND, int CODEC>
__global__ void __launch_bounds__(WG) k_dequantize(const uint8_t* __restrict__ codes, const uint16_t* __restrict__ scales,
                                                   int64_t n, float* __restrict__ out,
                                                   const CodecTables* __restrict__ gtabs) {
  __shared__ CodecTables tabs;
  load_tables(tabs, gtabs);
  const gp<float> o = (gp<float>)out;
  const int64_t stride = (int64_t)gridDim.x * WG * EPL;
  constexpr int SK = (KIND == 0) ? MOMENTUM_STATE : VARIANCE_STATE;
  for (int64_t i = ((int64_t)blockIdx.x * WG + threadIdx.x) * EPL; i < n; i += stride) {
    const int cnt = (int)min((int64_t)8, n - i);
    constexpr int CC = code_codec<CODEC>;
    constexpr int QW = code_words<CC>;
    const gp<const uint8_t> cp = (gp<const uint8_t>)codes + i * QW / 2;
    const DW<QW> q = (cnt == 8) ? load_codes<CC, true>(cp, 8) : load_codes<CC, false>(cp, cnt);
    // the 8 elements of a thread lie in one 32-element block
    const float dm = decode_mult<SK, CODEC>(scale_f32<CODEC>(((gp<const uint16_t>)scales)[i >> 5]));
    float v[8];
    const auto qo = code_operand<CC>(q);
#pragma unroll
    for (int k = 0; k < 8; ++k) v[k] = decode_state<SK, CC>(qo, k, dm, tabs);
    if (cnt == 8) {
      *(gp<f32x4>)(o + i) = f32x4{v[0], v[1], v[2], v[3]};
      *(gp<f32x4>)(o + i + 4) = f32x4{v[4], v[5], v[6], v[7]};
    } else {
#pragma unroll
      for (int k = 0; k < 8; ++k) if (k < cnt) o[i + k] = v[k];
    }
  }
}

// ---------------------------------------------------------------------------
// self-test of the exact fast arithmetic (mismatch counters; not a hot path)
// ---------------------------------------------------------------------------
// what 0: rcp_refined vs IEEE 1/b on the f32 patterns [lo, lo+count)
// what 1: sqrt_corrected vs the IEEE square root
// what 2: v_cvt_pk_u8_f32 vs clamp(round_half_even(x), 0, 255), NaN -> 0
// what 3: div_refined(a, b, rcp_refined(b)) vs IEEE a/b on `count` pairs drawn
//         from a counter-based generator seeded by lo: b over every exponent of
//         the refined reciprocal's range, a over the dividend range of the
//         fast AdamW step (|a| in [2^-100, 2^101) or 0), quotient 0 or of
//         magnitude in [2^-125, 2^120) (pairs outside are skipped)
// what 4: the same division with b an fp16 value (a block scale) and |a| <= b
// what 5: as 3, but only pairs whose quotient is a nonzero subnormal: the
//         range the AdamW step's guard keeps out of the fast form
// what 6: sqrt_fast (from the successor's estimate) vs the IEEE square root
//         on the f32 patterns [lo, lo+count)
__device__ __forceinline__ uint64_t splitmix64(uint64_t x) {
  x += 0x9E3779B97F4A7C15ull;
  x = (x ^ (x >> 30)) * 0xBF58476D1CE4E5B9ull;
  x = (x ^ (x >> 27)) * 0x94D049BB133111EBull;
  return x ^ (x >> 31);
}
__global__ void __launch_bounds__(WG) k_selftest(int what, uint32_t lo, uint64_t count,
                                                 unsigned long long* __restrict__ bad) {
  const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  unsigned long long nb = 0;
  for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < count; i += stride) {
    bool ok;
    if (what <= 2 || what == 6) {
      const float x = u2f(lo + (uint32_t)i);
      if (what == 0) ok = f2u(rcp_refined(x)) == f2u(1.0f / x);
      else if (what == 1) ok = f2u(sqrt_corrected(x)) == f2u(__builtin_sqrtf(x));
      else if (what == 6) ok = f2u(sqrt_fast(x)) == f2u(__builtin_sqrtf(x));
      else {
        const uint32_t got = __builtin_amdgcn_cvt_pk_u8_f32(x, 0, 0u) & 0xFFu;
        const uint32_t ref = (x != x) ? 0u : (uint32_t)__builtin_rintf(fmaxf(fminf(x, 255.0f), 0.0f));
        ok = got == ref;
      }
    } else {
      const uint64_t h = splitmix64(((uint64_t)lo << 32) ^ i);
      float a, b;
      if (what != 4) {
        const uint32_t eb = 1u + (uint32_t)((h >> 23) % 252u);                  // b in [2^-126, 2^126)
        b = u2f((eb << 23) | (uint32_t)(h & 0x7FFFFFu));
        const uint32_t ea = 27u + (uint32_t)((h >> 31) % 201u);                 // |a| in [2^-100, 2^101)
        a = u2f(((uint32_t)(h >> 63) << 31) | (ea << 23) | (uint32_t)((h >> 40) & 0x7FFFFFu));
        if (((h >> 12) & 1023u) == 0u) a = 0.0f;
        const float q = fabsf(a / b);
        const bool fast_domain = q == 0.0f || (q >= 0x1p-125f && q < 0x1p120f);
        const bool subnormal = q > 0.0f && q < 0x1p-126f;
        if (what == 3 ? !fast_domain : !subnormal) continue;
      } else {
        b = h2f(1u + (uint32_t)((h >> 48) % 0x7BFFu));                          // positive finite fp16
        const float t = u2f((uint32_t)(h & 0x7FFFFFu) | 0x3F000000u) * 2.0f - 1.0f;   // [-1, 1)
        a = b * t;
      }
      ok = f2u(div_refined(a, b, rcp_refined(b))) == f2u(a / b);
    }
    nb += ok ? 0 : 1;
  }
  if (nb) atomicAdd(bad, nb);
}

}  // namespace fo
