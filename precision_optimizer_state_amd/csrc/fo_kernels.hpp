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
  float wd;       // coupled (L2) weight decay of Adam; unused by AdamW
  int fast_rcp;   // eps >= 2^-126: every denominator is a positive normal >= eps
};
struct SGDMConsts {
  float lr, mu, wd;
  float damp1;    // 1 - dampening
  int nesterov;
  int first;      // step 1: the buffer is set to the (decayed) gradient
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

// element k of a packed group
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
// shared pieces of the fused update
// ---------------------------------------------------------------------------
// w = sqrt(v) correctly rounded for 8 values (IEEE expansion when any lane of
// the wave needs scaling)
__device__ __forceinline__ void sqrt8(const float (&v)[EPL], float (&w)[EPL]) {
  uint64_t slow = 0;
#pragma unroll
  for (int k = 0; k < EPL; ++k) {
    w[k] = sqrt_corrected(v[k]);
    slow |= __builtin_amdgcn_ballot_w64(sqrt_needs_scaling(v[k]));
  }
  if (slow) {
#pragma unroll
    for (int k = 0; k < EPL; ++k) w[k] = __builtin_sqrtf(v[k]);
  }
}

// r = RN(1/d) for 8 denominators (IEEE division when any lane is outside the
// verified range, or when eps does not keep denominators normal)
__device__ __forceinline__ void rcp8(const float (&d)[EPL], float (&r)[EPL], int fast) {
  uint64_t slow = fast ? 0ull : ~0ull;
#pragma unroll
  for (int k = 0; k < EPL; ++k) {
    r[k] = rcp_refined(d[k]);
    slow |= __builtin_amdgcn_ballot_w64(!(d[k] < 0x1p126f));
  }
  if (slow) {
#pragma unroll
    for (int k = 0; k < EPL; ++k) r[k] = 1.0f / d[k];
  }
}

// ---------------------------------------------------------------------------
// fused AdamW: one wave tile
// ---------------------------------------------------------------------------
template <int WFMT, int ECC, int CODEC, bool L2, bool FULL>
__device__ __forceinline__ void adamw_tile(const TensorDesc& d, int64_t e0, int lane,
                                           const CodecTables& tabs, const AdamWConsts& c) {
  constexpr int EB = ECC / 8;                                  // ECC bytes per element
  const int Q = lane >> 2, p = lane & 3;
  const int64_t n = d.n;
  const gp<const uint8_t> grad = (gp<const uint8_t>)d.grad + e0 * 2;
  const gp<uint8_t> w16 = (gp<uint8_t>)d.w16 + e0 * 2;
  const gp<uint8_t> ecc = (gp<uint8_t>)d.ecc + e0 * EB;
  const gp<uint8_t> mq = (gp<uint8_t>)d.q1 + e0;
  const gp<uint8_t> vq = (gp<uint8_t>)d.q2 + e0;
  const gp<uint16_t> ms = (gp<uint16_t>)d.s1 + (e0 >> 5);
  const gp<uint16_t> vs = (gp<uint16_t>)d.s2 + (e0 >> 5);
  const int64_t rem = n - e0;                                  // valid elements from e0 on
  const int own = p * 16 + Q;                                  // owned block within the tile
  const bool own_ok = FULL || (int64_t)own * 32 < rem;

  // ---- issue every load of the tile -------------------------------------
  DW<4> G[NSUB], W[NSUB];
  DW<2 * EB> E[NSUB];
  DW<2> MQ[NSUB], VQ[NSUB];
  int cnt[NSUB];
#pragma unroll
  for (int j = 0; j < NSUB; ++j) {
    const int off = j * SUB + lane * EPL;
    cnt[j] = FULL ? 8 : (int)max((int64_t)0, min((int64_t)8, rem - off));
    G[j] = load8<2, FULL>(grad + off * 2, cnt[j]);
    W[j] = load8<2, FULL>(w16 + off * 2, cnt[j]);
    E[j] = load8<EB, FULL>(ecc + off * EB, cnt[j]);
    MQ[j] = load8<1, FULL>(mq + off, cnt[j]);
    VQ[j] = load8<1, FULL>(vq + off, cnt[j]);
  }
  const uint32_t sm_old = own_ok ? (uint32_t)__builtin_nontemporal_load(ms + own) : 0u;
  const uint32_t sv_old = own_ok ? (uint32_t)__builtin_nontemporal_load(vs + own) : 0u;

  // ---- per-block decode constants (owned block) -------------------------
  const float smf = h2f(sm_old), svf = h2f(sv_old);
  const float dm_own = (CODEC == COMPANDED) ? smf : smf * K127;
  const float dv_own = (CODEC == COMPANDED) ? svf * K255 : (svf * svf) * K255;

  float Mn[NSUB][EPL], Xn[NSUB][EPL];       // fresh m and (sqrt(v) | v) for re-encoding
  // block maxima start at NaN: IEEE maxNum returns any non-NaN element (the
  // zeros of a partial block included), so only an all-NaN block keeps NaN
  // and gets a NaN scale, which carries the NaN into the decoded state
  float own_mmax = 0.0f, own_xmax = 0.0f;

#pragma unroll
  for (int j = 0; j < NSUB; ++j) {
    const float dm = bcast_j(dm_own, j), dv = bcast_j(dv_own, j);
    float th[EPL], m[EPL], v[EPL], w[EPL], den[EPL], r[EPL];
#pragma unroll
    for (int k = 0; k < EPL; ++k) {
      float g = wid<WFMT>(G[j], k);
      th[k] = ecc_decode<WFMT, ECC>(wid<WFMT>(W[j], k), rho_at<ECC>(E[j], k));
      if constexpr (L2) g = g + c.wd * th[k];                  // Adam: decay folded into the gradient
      const int32_t qm = s8(MQ[j], k);
      const float mh = (CODEC == COMPANDED) ? dm * tabs.lut[qm + LUT_BIAS] : dm * (float)qm;
      const float tv = dv * (float)u8(VQ[j], k);
      const float vh = (CODEC == COMPANDED) ? tv * tv : tv;
      // update (fixed float32 order, one rounding per operation)
      m[k] = c.b1 * mh + c.omb1 * g;
      v[k] = c.b2 * vh + c.omb2 * (g * g);
      th[k] = th[k] * c.decay;
    }
    sqrt8(v, w);
#pragma unroll
    for (int k = 0; k < EPL; ++k) den[k] = w[k] * c.ibc2 + c.eps;
    rcp8(den, r, c.fast_rcp);
#pragma unroll
    for (int k = 0; k < EPL; ++k) th[k] = th[k] - c.step_size * (m[k] * r[k]);

    // split the new master and store it
    uint32_t wo[4], eo[ECC / 4];
    split8<WFMT, ECC>(th, wo, eo);
    const int off = j * SUB + lane * EPL;
    store8<2, FULL>(w16 + off * 2, wo, cnt[j]);
    store8<EB, FULL>(ecc + off * EB, eo, cnt[j]);

    float mmax = __builtin_nanf(""), xmax = __builtin_nanf("");
#pragma unroll
    for (int k = 0; k < EPL; ++k) {
      const float x = (CODEC == COMPANDED) ? w[k] : v[k];
      Mn[j][k] = m[k];
      Xn[j][k] = x;
      mmax = fmaxf(mmax, fabsf(m[k]));
      xmax = fmaxf(xmax, x);
    }
    mmax = quad_max(mmax);
    xmax = quad_max(xmax);
    own_mmax = (p == j) ? mmax : own_mmax;
    own_xmax = (p == j) ? xmax : own_xmax;
  }

  // ---- new block scales and encode constants (owned block) ---------------
  const uint32_t smb = ru_fp16(own_mmax);
  const uint32_t svb = ru_fp16((CODEC == COMPANDED) ? own_xmax : __builtin_sqrtf(own_xmax));
  if (own_ok) {
    __builtin_nontemporal_store((uint16_t)smb, ms + own);
    __builtin_nontemporal_store((uint16_t)svb, vs + own);
  }
  const float sm = h2f(smb), sv = h2f(svb);
  float cm_own, cv_own;
  if constexpr (CODEC == COMPANDED) {
    cm_own = (sm > 0.0f) ? 1.0f / sm : 0.0f;
    cv_own = (sv > 0.0f) ? 255.0f / sv : 0.0f;
  } else {
    const float sv2 = sv * sv;
    cm_own = (sm > 0.0f) ? 127.0f / sm : 0.0f;
    cv_own = (sv2 > 0.0f) ? 255.0f / sv2 : 0.0f;
  }

#pragma unroll
  for (int j = 0; j < NSUB; ++j) {
    const float cm = bcast_j(cm_own, j), cv = bcast_j(cv_own, j);
    uint32_t qm[EPL], vo[2] = {0u, 0u};
#pragma unroll
    for (int k = 0; k < EPL; ++k) {
      qm[k] = (uint32_t)((CODEC == COMPANDED) ? encode_m_companded(Mn[j][k], cm, tabs)
                                              : encode_m_linear(Mn[j][k], cm));
      vo[k >> 2] = encode_v_into(Xn[j][k], cv, k & 3, vo[k >> 2]);
    }
    const uint32_t mo[2] = {pack4_byte0(qm[0], qm[1], qm[2], qm[3]), pack4_byte0(qm[4], qm[5], qm[6], qm[7])};
    const int off = j * SUB + lane * EPL;
    store8<1, FULL>(mq + off, mo, cnt[j]);
    store8<1, FULL>(vq + off, vo, cnt[j]);
  }
}

// ---------------------------------------------------------------------------
// fused SGD with momentum: one wave tile
// ---------------------------------------------------------------------------
template <int WFMT, int ECC, int CODEC, bool FULL>
__device__ __forceinline__ void sgdm_tile(const TensorDesc& d, int64_t e0, int lane,
                                          const CodecTables& tabs, const SGDMConsts& c) {
  constexpr int EB = ECC / 8;
  const int Q = lane >> 2, p = lane & 3;
  const int64_t n = d.n;
  const gp<const uint8_t> grad = (gp<const uint8_t>)d.grad + e0 * 2;
  const gp<uint8_t> w16 = (gp<uint8_t>)d.w16 + e0 * 2;
  const gp<uint8_t> ecc = (gp<uint8_t>)d.ecc + e0 * EB;
  const gp<uint8_t> bq = (gp<uint8_t>)d.q1 + e0;
  const gp<uint16_t> bs = (gp<uint16_t>)d.s1 + (e0 >> 5);
  const int64_t rem = n - e0;
  const int own = p * 16 + Q;
  const bool own_ok = FULL || (int64_t)own * 32 < rem;

  DW<4> G[NSUB], W[NSUB];
  DW<2 * EB> E[NSUB];
  DW<2> BQ[NSUB];
  int cnt[NSUB];
#pragma unroll
  for (int j = 0; j < NSUB; ++j) {
    const int off = j * SUB + lane * EPL;
    cnt[j] = FULL ? 8 : (int)max((int64_t)0, min((int64_t)8, rem - off));
    G[j] = load8<2, FULL>(grad + off * 2, cnt[j]);
    W[j] = load8<2, FULL>(w16 + off * 2, cnt[j]);
    E[j] = load8<EB, FULL>(ecc + off * EB, cnt[j]);
    BQ[j] = load8<1, FULL>(bq + off, cnt[j]);
  }
  const uint32_t sb_old = own_ok ? (uint32_t)__builtin_nontemporal_load(bs + own) : 0u;
  const float sbf = h2f(sb_old);
  const float db_own = (CODEC == COMPANDED) ? sbf : sbf * K127;

  float Bn[NSUB][EPL];
  float own_bmax = 0.0f;
#pragma unroll
  for (int j = 0; j < NSUB; ++j) {
    const float db = bcast_j(db_own, j);
    float th[EPL], b[EPL];
    float bmax = __builtin_nanf("");          // all-NaN block -> NaN scale
#pragma unroll
    for (int k = 0; k < EPL; ++k) {
      const float g = wid<WFMT>(G[j], k);
      const float t0 = ecc_decode<WFMT, ECC>(wid<WFMT>(W[j], k), rho_at<ECC>(E[j], k));
      const int32_t qb = s8(BQ[j], k);
      const float bh = (CODEC == COMPANDED) ? db * tabs.lut[qb + LUT_BIAS] : db * (float)qb;
      const float dd = g + c.wd * t0;
      b[k] = c.first ? dd : c.mu * bh + c.damp1 * dd;
      const float u = c.nesterov ? dd + c.mu * b[k] : b[k];
      th[k] = t0 - c.lr * u;
      Bn[j][k] = b[k];
      bmax = fmaxf(bmax, fabsf(b[k]));
    }
    uint32_t wo[4], eo[ECC / 4];
    split8<WFMT, ECC>(th, wo, eo);
    const int off = j * SUB + lane * EPL;
    store8<2, FULL>(w16 + off * 2, wo, cnt[j]);
    store8<EB, FULL>(ecc + off * EB, eo, cnt[j]);
    bmax = quad_max(bmax);
    own_bmax = (p == j) ? bmax : own_bmax;
  }
  const uint32_t sbb = ru_fp16(own_bmax);
  if (own_ok) __builtin_nontemporal_store((uint16_t)sbb, bs + own);
  const float sb = h2f(sbb);
  const float cb_own = (sb > 0.0f) ? ((CODEC == COMPANDED) ? 1.0f : 127.0f) / sb : 0.0f;
#pragma unroll
  for (int j = 0; j < NSUB; ++j) {
    const float cb = bcast_j(cb_own, j);
    uint32_t q[EPL];
#pragma unroll
    for (int k = 0; k < EPL; ++k)
      q[k] = (uint32_t)((CODEC == COMPANDED) ? encode_m_companded(Bn[j][k], cb, tabs)
                                             : encode_m_linear(Bn[j][k], cb));
    const uint32_t bo[2] = {pack4_byte0(q[0], q[1], q[2], q[3]), pack4_byte0(q[4], q[5], q[6], q[7])};
    store8<1, FULL>(bq + j * SUB + lane * EPL, bo, cnt[j]);
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
#pragma unroll
  for (int j = 0; j < NSUB; ++j) {
    const int off = j * SUB + lane * EPL;
    cnt[j] = FULL ? 8 : (int)max((int64_t)0, min((int64_t)8, rem - off));
    G[j] = load8<2, FULL>(grad + off * 2, cnt[j]);
    W[j] = load8<2, FULL>(w16 + off * 2, cnt[j]);
    E[j] = load8<EB, FULL>(ecc + off * EB, cnt[j]);
    MQ[j] = load8<1, FULL>(mq + off, cnt[j]);
    VQ[j] = load8<1, FULL>(vq + off, cnt[j]);
  }
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
    const int off = j * SUB + lane * EPL;
    store8<2, FULL>(w16 + off * 2, W[j].w, cnt[j]);
    store8<EB, FULL>(ecc + off * EB, E[j].w, cnt[j]);
    store8<1, FULL>(mq + off, MQ[j].w, cnt[j]);
    store8<1, FULL>(vq + off, VQ[j].w, cnt[j]);
  }
  if (own_ok) { ms[own] = (uint16_t)(sm ^ key); vs[own] = (uint16_t)(sv ^ key); }
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
__device__ __forceinline__ const CodecTables& wave_tables(CodecTables* lds, const CodecTables* __restrict__ src) {
  constexpr int CHUNKS = sizeof(CodecTables) / (16 * WAVE);
  const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
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

__global__ void __launch_bounds__(WG) k_init_tables(CodecTables* out) {
  __shared__ float thr[128];
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
  const CodecTables& tabs = wave_tables(wtabs, gtabs);
  tile_loop<adamw_tile_waves<ECC>>(tab, count, tile0, tile_end, [&](const TensorDesc& d, int64_t e0, int lane) {
    if (e0 + TILE <= d.n) adamw_tile<WFMT, ECC, CODEC, L2, true>(d, e0, lane, tabs, c);
    else adamw_tile<WFMT, ECC, CODEC, L2, false>(d, e0, lane, tabs, c);
  });
}

template <int WFMT, int ECC, int CODEC>
__global__ void __launch_bounds__(WAVE * SGDM_TILE_WAVES) k_fused_sgdm(const TensorDesc* __restrict__ tab, int count,
                                                                 int64_t tile0, int64_t tile_end,
                                                                 const CodecTables* __restrict__ gtabs, SGDMConsts c) {
  __shared__ CodecTables wtabs[SGDM_TILE_WAVES];
  const CodecTables& tabs = wave_tables(wtabs, gtabs);
  tile_loop<SGDM_TILE_WAVES>(tab, count, tile0, tile_end, [&](const TensorDesc& d, int64_t e0, int lane) {
    if (e0 + TILE <= d.n) sgdm_tile<WFMT, ECC, CODEC, true>(d, e0, lane, tabs, c);
    else sgdm_tile<WFMT, ECC, CODEC, false>(d, e0, lane, tabs, c);
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

// KIND 0 = momentum (int8), 1 = variance (uint8).  A quad of lanes = one block.
template <int KIND, int CODEC>
__global__ void __launch_bounds__(WG) k_quantize(const float* __restrict__ x, int64_t n,
                                                 uint8_t* __restrict__ codes, uint16_t* __restrict__ scales,
                                                 const CodecTables* __restrict__ gtabs) {
  __shared__ CodecTables tabs;
  load_tables(tabs, gtabs);
  const gp<const float> xs = (gp<const float>)x;
  const int64_t stride = (int64_t)gridDim.x * WG * EPL;
  // all lanes iterate together (stride multiple of 512), so the 4 lanes of a
  // block are active at the same time; lanes past n contribute zeros
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
    float e[8];
    if (KIND == 1 && CODEC == COMPANDED) {
      sqrt8(v, e);
    } else {
#pragma unroll
      for (int k = 0; k < 8; ++k) e[k] = v[k];
    }
    float mx = __builtin_nanf("");            // all-NaN block -> NaN scale
#pragma unroll
    for (int k = 0; k < 8; ++k) mx = fmaxf(mx, (KIND == 0) ? fabsf(e[k]) : e[k]);
    mx = quad_max(mx);
    const uint32_t sb = ru_fp16((KIND == 1 && CODEC == LINEAR) ? __builtin_sqrtf(mx) : mx);
    if ((threadIdx.x & 3) == 0 && cnt > 0) ((gp<uint16_t>)scales)[i >> 5] = (uint16_t)sb;
    const float s = h2f(sb);
    float C;
    if (KIND == 0) C = (s > 0.0f) ? ((CODEC == COMPANDED) ? 1.0f : 127.0f) / s : 0.0f;
    else if (CODEC == COMPANDED) C = (s > 0.0f) ? 255.0f / s : 0.0f;
    else { const float s2 = s * s; C = (s2 > 0.0f) ? 255.0f / s2 : 0.0f; }
    uint32_t o[2];
    if (KIND == 0) {
      uint32_t q[8];
#pragma unroll
      for (int k = 0; k < 8; ++k)
        q[k] = (uint32_t)((CODEC == COMPANDED) ? encode_m_companded(e[k], C, tabs) : encode_m_linear(e[k], C));
      o[0] = pack4_byte0(q[0], q[1], q[2], q[3]);
      o[1] = pack4_byte0(q[4], q[5], q[6], q[7]);
    } else {
      o[0] = o[1] = 0u;
#pragma unroll
      for (int k = 0; k < 8; ++k) o[k >> 2] = encode_v_into(e[k], C, k & 3, o[k >> 2]);
    }
    if (cnt == 8) store8<1, true>((gp<uint8_t>)codes + i, o, 8);
    else if (cnt > 0) store8<1, false>((gp<uint8_t>)codes + i, o, cnt);
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
  for (int64_t i = ((int64_t)blockIdx.x * WG + threadIdx.x) * EPL; i < n; i += stride) {
    const int cnt = (int)min((int64_t)8, n - i);
    const gp<const uint8_t> cp = (gp<const uint8_t>)codes + i;
    const DW<2> q = (cnt == 8) ? load8<1, true>(cp, 8) : load8<1, false>(cp, cnt);
    const float s = h2f(((gp<const uint16_t>)scales)[i >> 5]);
    float v[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      if (KIND == 0) {
        const int32_t cq = s8(q, k);
        v[k] = (CODEC == COMPANDED) ? s * tabs.lut[cq + LUT_BIAS] : (s * K127) * (float)cq;
      } else {
        const float cq = (float)u8(q, k);
        if (CODEC == COMPANDED) { const float t = (s * K255) * cq; v[k] = t * t; }
        else v[k] = ((s * s) * K255) * cq;
      }
    }
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
// what 2: v_cvt_pk_u8_f32 vs clamp(round_half_even(x), 0, 255) (NaN skipped)
__global__ void __launch_bounds__(WG) k_selftest(int what, uint32_t lo, uint64_t count,
                                                 unsigned long long* __restrict__ bad) {
  const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  unsigned long long nb = 0;
  for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < count; i += stride) {
    const float x = u2f(lo + (uint32_t)i);
    bool ok;
    if (what == 0) ok = f2u(rcp_refined(x)) == f2u(1.0f / x);
    else if (what == 1) ok = f2u(sqrt_corrected(x)) == f2u(__builtin_sqrtf(x));
    else {
      const uint32_t got = __builtin_amdgcn_cvt_pk_u8_f32(x, 0, 0u) & 0xFFu;
      const uint32_t ref = (uint32_t)__builtin_rintf(fmaxf(fminf(x, 255.0f), 0.0f));
      ok = (x != x) || got == ref;
    }
    nb += ok ? 0 : 1;
  }
  if (nb) atomicAdd(bad, nb);
}

}  // namespace fo
