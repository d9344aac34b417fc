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
//   * Waves are persistent and stride over the global tile list of all
//     tensors of the step; a tile never crosses a tensor, and the last tile of
//     a tensor takes a masked path.
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
constexpr int WAVES_PER_WG = 4;
constexpr int WG = WAVE * WAVES_PER_WG;    // 256 threads

// Device copy of one tensor of a step (built by the host launcher).
struct alignas(16) TensorDesc {
  uint64_t w16, ecc, grad, q1, s1, q2, s2;  // q2/s2 unused by SGD-M
  int64_t n;
  int64_t tile_begin;                       // first global wave-tile index
};
static_assert(sizeof(TensorDesc) == 80, "descriptor layout");

struct AdamWConsts { float b1, b2, omb1, omb2, decay, step_size, ibc2, eps; };
struct SGDMConsts { float lr, mu, wd; };

// ---------------------------------------------------------------------------
// masked vector access for the last (partial) tile of a tensor
// ---------------------------------------------------------------------------
template <int NDW>
struct DW { uint32_t w[NDW]; };

// load 8 elements of ESZ bytes (NDW = 2*ESZ dwords) starting at element p[0]
template <int ESZ, bool FULL>
__device__ __forceinline__ DW<2 * ESZ> load8(const void* base, int cnt) {
  DW<2 * ESZ> r;
  if (FULL || cnt >= 8) {
    if constexpr (ESZ == 2) {
      const uint4 v = *(const uint4*)base;
      r.w[0] = v.x; r.w[1] = v.y; r.w[2] = v.z; r.w[3] = v.w;
    } else {
      const uint2 v = *(const uint2*)base;
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
      if constexpr (ESZ == 2) x = ((const uint16_t*)base)[k];
      else x = ((const uint8_t*)base)[k];
      r.w[(k * ESZ) >> 2] |= x << (8 * ((k * ESZ) & 3));
    }
  }
  return r;
}

template <int ESZ, bool FULL>
__device__ __forceinline__ void store8(void* base, const DW<2 * ESZ>& r, int cnt) {
  if (FULL || cnt >= 8) {
    if constexpr (ESZ == 2) *(uint4*)base = make_uint4(r.w[0], r.w[1], r.w[2], r.w[3]);
    else *(uint2*)base = make_uint2(r.w[0], r.w[1]);
    return;
  }
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    if (k < cnt) {
      const uint32_t x = r.w[(k * ESZ) >> 2] >> (8 * ((k * ESZ) & 3));
      if constexpr (ESZ == 2) ((uint16_t*)base)[k] = (uint16_t)x;
      else ((uint8_t*)base)[k] = (uint8_t)x;
    }
  }
}

// element k of a packed group
__device__ __forceinline__ uint32_t h16(const DW<4>& v, int k) { return (v.w[k >> 1] >> (16 * (k & 1))) & 0xFFFFu; }
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

// ---------------------------------------------------------------------------
// tile lookup
// ---------------------------------------------------------------------------
__device__ __forceinline__ int find_tensor(const TensorDesc* __restrict__ tab, int count, int64_t T) {
  int lo = 0, hi = count - 1;              // largest t with tile_begin <= T
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (tab[mid].tile_begin <= T) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// ---------------------------------------------------------------------------
// fused AdamW: one wave tile
// ---------------------------------------------------------------------------
template <int WFMT, int ECC, int CODEC, bool FULL>
__device__ __forceinline__ void adamw_tile(const TensorDesc& d, int64_t e0, int lane,
                                           const CodecTables& tabs, const AdamWConsts& c) {
  constexpr int EB = ECC / 8;                                  // ECC bytes per element
  const int Q = lane >> 2, p = lane & 3;
  const int64_t n = d.n;
  const uint16_t* __restrict__ grad = (const uint16_t*)d.grad + e0;
  uint16_t* __restrict__ w16 = (uint16_t*)d.w16 + e0;
  uint8_t* __restrict__ ecc = (uint8_t*)d.ecc + e0 * EB;
  int8_t* __restrict__ mq = (int8_t*)d.q1 + e0;
  uint8_t* __restrict__ vq = (uint8_t*)d.q2 + e0;
  uint16_t* __restrict__ ms = (uint16_t*)d.s1 + (e0 >> 5);
  uint16_t* __restrict__ vs = (uint16_t*)d.s2 + (e0 >> 5);
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
    G[j] = load8<2, FULL>(grad + off, cnt[j]);
    W[j] = load8<2, FULL>(w16 + off, cnt[j]);
    E[j] = load8<EB, FULL>(ecc + off * EB, cnt[j]);
    MQ[j] = load8<1, FULL>(mq + off, cnt[j]);
    VQ[j] = load8<1, FULL>(vq + off, cnt[j]);
  }
  const uint32_t sm_old = own_ok ? (uint32_t)ms[own] : 0u;
  const uint32_t sv_old = own_ok ? (uint32_t)vs[own] : 0u;

  // ---- per-block decode constants (owned block), then per sub-tile -------
  const float smf = h2f(sm_old), svf = h2f(sv_old);
  const float dm_own = (CODEC == COMPANDED) ? smf : smf * K127;
  const float dv_own = (CODEC == COMPANDED) ? svf * K255 : (svf * svf) * K255;

  float Mn[NSUB][EPL], Xn[NSUB][EPL];       // fresh m and (sqrt(v) | v) for re-encoding
  float own_mmax = 0.0f, own_xmax = 0.0f;

#pragma unroll
  for (int j = 0; j < NSUB; ++j) {
    float dm, dv;
    if (j == 0) { dm = quad_bcast<0>(dm_own); dv = quad_bcast<0>(dv_own); }
    if (j == 1) { dm = quad_bcast<1>(dm_own); dv = quad_bcast<1>(dv_own); }
    if (j == 2) { dm = quad_bcast<2>(dm_own); dv = quad_bcast<2>(dv_own); }
    if (j == 3) { dm = quad_bcast<3>(dm_own); dv = quad_bcast<3>(dv_own); }
    DW<4> Wo;
    DW<2 * EB> Eo;
#pragma unroll
    for (int i = 0; i < 2 * EB; ++i) Eo.w[i] = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) Wo.w[i] = 0;
    float mmax = 0.0f, xmax = 0.0f;
#pragma unroll
    for (int k = 0; k < EPL; ++k) {
      const float g = wid<WFMT>(G[j], k);
      int32_t rho;
      if constexpr (ECC == 8) rho = s8(E[j], k); else rho = s16(E[j], k);
      float th = ecc_decode<WFMT, ECC>(wid<WFMT>(W[j], k), rho);
      const int32_t qm = s8(MQ[j], k);
      float m = (CODEC == COMPANDED) ? dm * tabs.lut[qm + 127] : dm * (float)qm;
      const float tv = dv * (float)u8(VQ[j], k);
      float v = (CODEC == COMPANDED) ? tv * tv : tv;
      // update (fixed float32 order, one rounding per operation)
      m = c.b1 * m + c.omb1 * g;
      v = c.b2 * v + c.omb2 * (g * g);
      th = th * c.decay;
      const float w = __builtin_sqrtf(v);
      const float den = w * c.ibc2 + c.eps;
      th = th - c.step_size * (m / den);
      // split the new master
      const SplitOut so = ecc_encode<WFMT, ECC>(th);
      Wo.w[k >> 1] |= so.h << (16 * (k & 1));
      if constexpr (ECC == 8) Eo.w[k >> 2] |= ((uint32_t)so.rho & 0xFFu) << (8 * (k & 3));
      else Eo.w[k >> 1] |= ((uint32_t)so.rho & 0xFFFFu) << (16 * (k & 1));
      const float x = (CODEC == COMPANDED) ? w : v;
      Mn[j][k] = m;
      Xn[j][k] = x;
      mmax = fmaxf(mmax, fabsf(m));
      xmax = fmaxf(xmax, x);
    }
    const int off = j * SUB + lane * EPL;
    store8<2, FULL>(w16 + off, Wo, cnt[j]);
    store8<EB, FULL>(ecc + off * EB, Eo, cnt[j]);
    mmax = quad_max(mmax);
    xmax = quad_max(xmax);
    own_mmax = (p == j) ? mmax : own_mmax;
    own_xmax = (p == j) ? xmax : own_xmax;
  }

  // ---- new block scales and encode constants (owned block) ---------------
  const uint32_t smb = ru_fp16(own_mmax);
  const uint32_t svb = ru_fp16((CODEC == COMPANDED) ? own_xmax : __builtin_sqrtf(own_xmax));
  if (own_ok) { ms[own] = (uint16_t)smb; vs[own] = (uint16_t)svb; }
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
    float cm, cv;
    if (j == 0) { cm = quad_bcast<0>(cm_own); cv = quad_bcast<0>(cv_own); }
    if (j == 1) { cm = quad_bcast<1>(cm_own); cv = quad_bcast<1>(cv_own); }
    if (j == 2) { cm = quad_bcast<2>(cm_own); cv = quad_bcast<2>(cv_own); }
    if (j == 3) { cm = quad_bcast<3>(cm_own); cv = quad_bcast<3>(cv_own); }
    DW<2> Mo, Vo;
    Mo.w[0] = Mo.w[1] = Vo.w[0] = Vo.w[1] = 0;
#pragma unroll
    for (int k = 0; k < EPL; ++k) {
      const int32_t qm = (CODEC == COMPANDED) ? encode_m_companded(Mn[j][k], cm, tabs.thr)
                                              : encode_m_linear(Mn[j][k], cm);
      const uint32_t qv = encode_v(Xn[j][k], cv);
      Mo.w[k >> 2] |= ((uint32_t)qm & 0xFFu) << (8 * (k & 3));
      Vo.w[k >> 2] |= qv << (8 * (k & 3));
    }
    const int off = j * SUB + lane * EPL;
    store8<1, FULL>(mq + off, Mo, cnt[j]);
    store8<1, FULL>(vq + off, Vo, cnt[j]);
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
  const uint16_t* __restrict__ grad = (const uint16_t*)d.grad + e0;
  uint16_t* __restrict__ w16 = (uint16_t*)d.w16 + e0;
  uint8_t* __restrict__ ecc = (uint8_t*)d.ecc + e0 * EB;
  int8_t* __restrict__ bq = (int8_t*)d.q1 + e0;
  uint16_t* __restrict__ bs = (uint16_t*)d.s1 + (e0 >> 5);
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
    G[j] = load8<2, FULL>(grad + off, cnt[j]);
    W[j] = load8<2, FULL>(w16 + off, cnt[j]);
    E[j] = load8<EB, FULL>(ecc + off * EB, cnt[j]);
    BQ[j] = load8<1, FULL>(bq + off, cnt[j]);
  }
  const uint32_t sb_old = own_ok ? (uint32_t)bs[own] : 0u;
  const float sbf = h2f(sb_old);
  const float db_own = (CODEC == COMPANDED) ? sbf : sbf * K127;

  float Bn[NSUB][EPL];
  float own_bmax = 0.0f;
#pragma unroll
  for (int j = 0; j < NSUB; ++j) {
    float db;
    if (j == 0) db = quad_bcast<0>(db_own);
    if (j == 1) db = quad_bcast<1>(db_own);
    if (j == 2) db = quad_bcast<2>(db_own);
    if (j == 3) db = quad_bcast<3>(db_own);
    DW<4> Wo;
    DW<2 * EB> Eo;
#pragma unroll
    for (int i = 0; i < 2 * EB; ++i) Eo.w[i] = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) Wo.w[i] = 0;
    float bmax = 0.0f;
#pragma unroll
    for (int k = 0; k < EPL; ++k) {
      const float g = wid<WFMT>(G[j], k);
      int32_t rho;
      if constexpr (ECC == 8) rho = s8(E[j], k); else rho = s16(E[j], k);
      float th = ecc_decode<WFMT, ECC>(wid<WFMT>(W[j], k), rho);
      const int32_t qb = s8(BQ[j], k);
      float b = (CODEC == COMPANDED) ? db * tabs.lut[qb + 127] : db * (float)qb;
      const float dd = g + c.wd * th;
      b = c.mu * b + dd;
      th = th - c.lr * b;
      const SplitOut so = ecc_encode<WFMT, ECC>(th);
      Wo.w[k >> 1] |= so.h << (16 * (k & 1));
      if constexpr (ECC == 8) Eo.w[k >> 2] |= ((uint32_t)so.rho & 0xFFu) << (8 * (k & 3));
      else Eo.w[k >> 1] |= ((uint32_t)so.rho & 0xFFFFu) << (16 * (k & 1));
      Bn[j][k] = b;
      bmax = fmaxf(bmax, fabsf(b));
    }
    const int off = j * SUB + lane * EPL;
    store8<2, FULL>(w16 + off, Wo, cnt[j]);
    store8<EB, FULL>(ecc + off * EB, Eo, cnt[j]);
    bmax = quad_max(bmax);
    own_bmax = (p == j) ? bmax : own_bmax;
  }
  const uint32_t sbb = ru_fp16(own_bmax);
  if (own_ok) bs[own] = (uint16_t)sbb;
  const float sb = h2f(sbb);
  const float cb_own = (sb > 0.0f) ? ((CODEC == COMPANDED) ? 1.0f : 127.0f) / sb : 0.0f;
#pragma unroll
  for (int j = 0; j < NSUB; ++j) {
    float cb;
    if (j == 0) cb = quad_bcast<0>(cb_own);
    if (j == 1) cb = quad_bcast<1>(cb_own);
    if (j == 2) cb = quad_bcast<2>(cb_own);
    if (j == 3) cb = quad_bcast<3>(cb_own);
    DW<2> Bo;
    Bo.w[0] = Bo.w[1] = 0;
#pragma unroll
    for (int k = 0; k < EPL; ++k) {
      const int32_t q = (CODEC == COMPANDED) ? encode_m_companded(Bn[j][k], cb, tabs.thr)
                                             : encode_m_linear(Bn[j][k], cb);
      Bo.w[k >> 2] |= ((uint32_t)q & 0xFFu) << (8 * (k & 3));
    }
    store8<1, FULL>(bq + j * SUB + lane * EPL, Bo, cnt[j]);
  }
}

// ---------------------------------------------------------------------------
// stream probe: the byte streams of one fused AdamW tile, no arithmetic
// ---------------------------------------------------------------------------
template <int ECC, bool FULL>
__device__ __forceinline__ void probe_tile(const TensorDesc& d, int64_t e0, int lane, uint32_t key) {
  constexpr int EB = ECC / 8;
  const int Q = lane >> 2, p = lane & 3;
  const uint16_t* __restrict__ grad = (const uint16_t*)d.grad + e0;
  uint16_t* __restrict__ w16 = (uint16_t*)d.w16 + e0;
  uint8_t* __restrict__ ecc = (uint8_t*)d.ecc + e0 * EB;
  int8_t* __restrict__ mq = (int8_t*)d.q1 + e0;
  uint8_t* __restrict__ vq = (uint8_t*)d.q2 + e0;
  uint16_t* __restrict__ ms = (uint16_t*)d.s1 + (e0 >> 5);
  uint16_t* __restrict__ vs = (uint16_t*)d.s2 + (e0 >> 5);
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
    G[j] = load8<2, FULL>(grad + off, cnt[j]);
    W[j] = load8<2, FULL>(w16 + off, cnt[j]);
    E[j] = load8<EB, FULL>(ecc + off * EB, cnt[j]);
    MQ[j] = load8<1, FULL>(mq + off, cnt[j]);
    VQ[j] = load8<1, FULL>(vq + off, cnt[j]);
  }
  uint32_t sm = own_ok ? (uint32_t)ms[own] : 0u;
  uint32_t sv = own_ok ? (uint32_t)vs[own] : 0u;
#pragma unroll
  for (int j = 0; j < NSUB; ++j) {
    // fold the gradient into the key so it is really read
    uint32_t k2 = key & (G[j].w[0] ^ G[j].w[1] ^ G[j].w[2] ^ G[j].w[3]);
#pragma unroll
    for (int i = 0; i < 4; ++i) W[j].w[i] ^= k2;
#pragma unroll
    for (int i = 0; i < 2 * EB; ++i) E[j].w[i] ^= key;
    MQ[j].w[0] ^= key; MQ[j].w[1] ^= key; VQ[j].w[0] ^= key; VQ[j].w[1] ^= key;
    const int off = j * SUB + lane * EPL;
    store8<2, FULL>(w16 + off, W[j], cnt[j]);
    store8<EB, FULL>(ecc + off * EB, E[j], cnt[j]);
    store8<1, FULL>(mq + off, MQ[j], cnt[j]);
    store8<1, FULL>(vq + off, VQ[j], cnt[j]);
  }
  if (own_ok) { ms[own] = (uint16_t)(sm ^ key); vs[own] = (uint16_t)(sv ^ key); }
}

// ---------------------------------------------------------------------------
// persistent multi-tensor kernels
// ---------------------------------------------------------------------------
// Persistent waves stride over the global wave-tile list of the step.  The
// tensor of a tile is found by binary search over the descriptors' first-tile
// indices when a wave leaves its current tensor (tiles only move forward).
template <typename F>
__device__ __forceinline__ void tile_loop(const TensorDesc* __restrict__ tab, int count, int64_t total_tiles, F&& body) {
  const int lane = threadIdx.x & (WAVE - 1);
  const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t nwaves = (int64_t)gridDim.x * WAVES_PER_WG;
  int t = 0;
  int64_t t_begin = 0, t_end = -1;
  for (int64_t T = (int64_t)blockIdx.x * WAVES_PER_WG + wid; T < total_tiles; T += nwaves) {
    if (T >= t_end) {
      t = find_tensor(tab, count, T);
      t_begin = tab[t].tile_begin;
      t_end = tab[t + 1].tile_begin;
    }
    const TensorDesc d = tab[t];
    body(d, (T - t_begin) * TILE, lane);
  }
}

template <int WFMT, int ECC, int CODEC>
__global__ void __launch_bounds__(WG) k_fused_adamw(const TensorDesc* __restrict__ tab, int count,
                                                    int64_t total_tiles, AdamWConsts c) {
  __shared__ CodecTables tabs;
  init_tables(tabs, threadIdx.x, blockDim.x);
  __syncthreads();
  tile_loop(tab, count, total_tiles, [&](const TensorDesc& d, int64_t e0, int lane) {
    if (e0 + TILE <= d.n) adamw_tile<WFMT, ECC, CODEC, true>(d, e0, lane, tabs, c);
    else adamw_tile<WFMT, ECC, CODEC, false>(d, e0, lane, tabs, c);
  });
}

template <int WFMT, int ECC, int CODEC>
__global__ void __launch_bounds__(WG) k_fused_sgdm(const TensorDesc* __restrict__ tab, int count,
                                                   int64_t total_tiles, SGDMConsts c) {
  __shared__ CodecTables tabs;
  init_tables(tabs, threadIdx.x, blockDim.x);
  __syncthreads();
  tile_loop(tab, count, total_tiles, [&](const TensorDesc& d, int64_t e0, int lane) {
    if (e0 + TILE <= d.n) sgdm_tile<WFMT, ECC, CODEC, true>(d, e0, lane, tabs, c);
    else sgdm_tile<WFMT, ECC, CODEC, false>(d, e0, lane, tabs, c);
  });
}

template <int ECC>
__global__ void __launch_bounds__(WG) k_stream_probe(const TensorDesc* __restrict__ tab, int count,
                                                     int64_t total_tiles, uint32_t key) {
  tile_loop(tab, count, total_tiles, [&](const TensorDesc& d, int64_t e0, int lane) {
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
  const int64_t stride = (int64_t)gridDim.x * WG * EPL;
  for (int64_t i = ((int64_t)blockIdx.x * WG + threadIdx.x) * EPL; i < n; i += stride) {
    const int cnt = (int)min((int64_t)8, n - i);
    float v[8];
    if (cnt == 8) {
      const float4 a = *(const float4*)(x + i), b = *(const float4*)(x + i + 4);
      v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    } else {
#pragma unroll
      for (int k = 0; k < 8; ++k) v[k] = (k < cnt) ? x[i + k] : 0.0f;
    }
    DW<4> Wo;
    DW<2 * EB> Eo;
#pragma unroll
    for (int q = 0; q < 4; ++q) Wo.w[q] = 0;
#pragma unroll
    for (int q = 0; q < 2 * EB; ++q) Eo.w[q] = 0;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const SplitOut so = ecc_encode<WFMT, ECC>(v[k]);
      Wo.w[k >> 1] |= so.h << (16 * (k & 1));
      if constexpr (ECC == 8) Eo.w[k >> 2] |= ((uint32_t)so.rho & 0xFFu) << (8 * (k & 3));
      else Eo.w[k >> 1] |= ((uint32_t)so.rho & 0xFFFFu) << (16 * (k & 1));
    }
    if (cnt == 8) {
      store8<2, true>(w16 + i, Wo, 8);
      store8<EB, true>(ecc + i * EB, Eo, 8);
    } else {
      store8<2, false>(w16 + i, Wo, cnt);
      store8<EB, false>(ecc + i * EB, Eo, cnt);
    }
  }
}

template <int WFMT, int ECC>
__global__ void __launch_bounds__(WG) k_reconstruct(const uint16_t* __restrict__ w16, const uint8_t* __restrict__ ecc,
                                                    int64_t n, float* __restrict__ out) {
  constexpr int EB = ECC / 8;
  const int64_t stride = (int64_t)gridDim.x * WG * EPL;
  for (int64_t i = ((int64_t)blockIdx.x * WG + threadIdx.x) * EPL; i < n; i += stride) {
    const int cnt = (int)min((int64_t)8, n - i);
    DW<4> W;
    DW<2 * EB> E;
    if (cnt == 8) { W = load8<2, true>(w16 + i, 8); E = load8<EB, true>(ecc + i * EB, 8); }
    else { W = load8<2, false>(w16 + i, cnt); E = load8<EB, false>(ecc + i * EB, cnt); }
    float v[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      int32_t rho;
      if constexpr (ECC == 8) rho = s8(E, k); else rho = s16(E, k);
      v[k] = ecc_decode<WFMT, ECC>(wid<WFMT>(W, k), rho);
    }
    if (cnt == 8) {
      *(float4*)(out + i) = make_float4(v[0], v[1], v[2], v[3]);
      *(float4*)(out + i + 4) = make_float4(v[4], v[5], v[6], v[7]);
    } else {
#pragma unroll
      for (int k = 0; k < 8; ++k) if (k < cnt) out[i + k] = v[k];
    }
  }
}

// KIND 0 = momentum (int8), 1 = variance (uint8).  A quad of lanes = one block.
template <int KIND, int CODEC>
__global__ void __launch_bounds__(WG) k_quantize(const float* __restrict__ x, int64_t n,
                                                 uint8_t* __restrict__ codes, uint16_t* __restrict__ scales) {
  __shared__ CodecTables tabs;
  init_tables(tabs, threadIdx.x, blockDim.x);
  __syncthreads();
  const int64_t stride = (int64_t)gridDim.x * WG * EPL;
  for (int64_t i = ((int64_t)blockIdx.x * WG + threadIdx.x) * EPL; i < n + 0; i += stride) {
    // every lane of a wave iterates together (the stride is a multiple of 512),
    // so the 4 lanes of a block are always active at the same time
    const int cnt = (int)min((int64_t)8, n - i);
    float v[8];
    if (cnt == 8) {
      const float4 a = *(const float4*)(x + i), b = *(const float4*)(x + i + 4);
      v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    } else {
#pragma unroll
      for (int k = 0; k < 8; ++k) v[k] = (k < cnt) ? x[i + k] : 0.0f;
    }
    float e[8];
    float mx = 0.0f;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      e[k] = (KIND == 0) ? v[k] : ((CODEC == COMPANDED) ? __builtin_sqrtf(v[k]) : v[k]);
      mx = fmaxf(mx, (KIND == 0) ? fabsf(e[k]) : e[k]);
    }
    mx = quad_max(mx);
    const uint32_t sb = ru_fp16((KIND == 1 && CODEC == LINEAR) ? __builtin_sqrtf(mx) : mx);
    if ((threadIdx.x & 3) == 0) scales[i >> 5] = (uint16_t)sb;
    const float s = h2f(sb);
    float C;
    if (KIND == 0) C = (s > 0.0f) ? ((CODEC == COMPANDED) ? 1.0f : 127.0f) / s : 0.0f;
    else if (CODEC == COMPANDED) C = (s > 0.0f) ? 255.0f / s : 0.0f;
    else { const float s2 = s * s; C = (s2 > 0.0f) ? 255.0f / s2 : 0.0f; }
    DW<2> o;
    o.w[0] = o.w[1] = 0;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      uint32_t q;
      if (KIND == 0) q = (uint32_t)((CODEC == COMPANDED) ? encode_m_companded(e[k], C, tabs.thr)
                                                         : encode_m_linear(e[k], C)) & 0xFFu;
      else q = encode_v(e[k], C);
      o.w[k >> 2] |= q << (8 * (k & 3));
    }
    if (cnt == 8) store8<1, true>(codes + i, o, 8);
    else store8<1, false>(codes + i, o, cnt);
  }
}

template <int KIND, int CODEC>
__global__ void __launch_bounds__(WG) k_dequantize(const uint8_t* __restrict__ codes, const uint16_t* __restrict__ scales,
                                                   int64_t n, float* __restrict__ out) {
  __shared__ CodecTables tabs;
  init_tables(tabs, threadIdx.x, blockDim.x);
  __syncthreads();
  const int64_t stride = (int64_t)gridDim.x * WG * EPL;
  for (int64_t i = ((int64_t)blockIdx.x * WG + threadIdx.x) * EPL; i < n; i += stride) {
    const int cnt = (int)min((int64_t)8, n - i);
    DW<2> q = (cnt == 8) ? load8<1, true>(codes + i, 8) : load8<1, false>(codes + i, cnt);
    const float s = h2f(scales[i >> 5]);
    float v[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      if (KIND == 0) {
        const int32_t c = s8(q, k);
        v[k] = (CODEC == COMPANDED) ? s * tabs.lut[c + 127] : (s * K127) * (float)c;
      } else {
        const float c = (float)u8(q, k);
        if (CODEC == COMPANDED) { const float t = (s * K255) * c; v[k] = t * t; }
        else v[k] = ((s * s) * K255) * c;
      }
    }
    if (cnt == 8) {
      *(float4*)(out + i) = make_float4(v[0], v[1], v[2], v[3]);
      *(float4*)(out + i + 4) = make_float4(v[4], v[5], v[6], v[7]);
    } else {
#pragma unroll
      for (int k = 0; k < 8; ++k) if (k < cnt) out[i + k] = v[k];
    }
  }
}

}  // namespace fo
