// fo_lib.hip -- C ABI of the fused low-precision optimizer step (see
// include/foamd.h for the contract of every entry point).
//
// Host responsibilities: argument validation (before anything is launched),
// the per-step float32 constants (computed in double, rounded once), the
// multi-tensor launch table (cached per distinct tensor list and device), and
// the launches themselves (one wave per tile; long lists in tile ranges).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <functional>
#include <unordered_map>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/foamd.h"
#include "fo_kernels.hpp"
#include "fo_slots.hpp"
#include "fo_grad16.hpp"

using namespace fo;

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(FO_EHIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

bool fmt_ok(int wfmt, int ecc_bits) {
  return (wfmt == FO_BF16 && (ecc_bits == 8 || ecc_bits == 16)) || (wfmt == FO_FP16 && ecc_bits == 8);
}

// ---------------------------------------------------------------------------
// device properties and grid sizing
// ---------------------------------------------------------------------------
struct DevInfo { int cus = 0; CodecTables* tables = nullptr; };
std::mutex g_dev_mu;
std::vector<DevInfo> g_dev;

int current_device(int* dev) {
  hipError_t e = hipGetDevice(dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  return FO_OK;
}

int device_cus(int dev, int* cus) {
  std::lock_guard<std::mutex> lk(g_dev_mu);
  if ((int)g_dev.size() <= dev) g_dev.resize(dev + 1);
  if (g_dev[dev].cus == 0) {
    int v = 0;
    hipError_t e = hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return hip_fail(e, "hipDeviceGetAttribute");
    g_dev[dev].cus = v;
  }
  *cus = g_dev[dev].cus;
  return FO_OK;
}

// Codec tables of the device (momentum levels and the momentum-code interval
// table), built once by k_init_tables on the stream of the first call that
// needs them; later calls on any stream of the device are ordered after that
// build by the synchronisation below.
int device_tables(int dev, hipStream_t stream, const CodecTables** out) {
  std::lock_guard<std::mutex> lk(g_dev_mu);
  if ((int)g_dev.size() <= dev) g_dev.resize(dev + 1);
  if (!g_dev[dev].tables) {
    CodecTables* t = nullptr;
    hipError_t e = hipMalloc((void**)&t, sizeof(CodecTables));
    if (e != hipSuccess) return fail(FO_ENOMEM, "hipMalloc(codec tables): %s", hipGetErrorString(e));
    hipLaunchKernelGGL(k_init_tables, 1, WG, 0, stream, t);
    e = hipGetLastError();
    if (e == hipSuccess) e = hipStreamSynchronize(stream);
    if (e != hipSuccess) { (void)hipFree(t); return hip_fail(e, "codec table build"); }
    g_dev[dev].tables = t;
  }
  *out = g_dev[dev].tables;
  return FO_OK;
}

// One wave per wave tile: the flat grid measured faster on MI355X than
// persistent waves for this read/write mix (new workgroups keep the memory
// pipeline full while finished ones retire).
// A list is launched as consecutive ranges of at most kLaunchTiles wave
// tiles (2^29 elements), one kernel each, all reading the same table.  On the
// Llama-3.1-8B list (291 tensors, 3.9M tiles) one launch over every tile ran
// 7-9% slower than ranges; of the range sizes 2^16..2^20, 2^18 measured best
// (0.3-0.6% ahead of 2^17, 1-2% of 2^19, 3-4% of 2^20).  Lists up to that
// size are one launch.
constexpr int64_t kLaunchTiles = int64_t(1) << 18;

// waves per workgroup of the AdamW step and probe kernels (their launch bounds)
int adamw_waves(int ecc_bits) { return ecc_bits == 16 ? adamw_tile_waves<16> : adamw_tile_waves<8>; }

int tile_grid(int64_t total_tiles, int waves_per_wg, int* grid) {
  const int64_t want = (total_tiles + waves_per_wg - 1) / waves_per_wg;
  *grid = (int)std::max<int64_t>(1, std::min<int64_t>(want, (int64_t)INT32_MAX));
  return FO_OK;
}

int elementwise_grid(int dev, int64_t n, int* grid) {
  int cus = 0;
  int rc = device_cus(dev, &cus);
  if (rc) return rc;
  const int64_t want = (n + (int64_t)WG * EPL - 1) / ((int64_t)WG * EPL);
  *grid = (int)std::max<int64_t>(1, std::min<int64_t>(want, (int64_t)cus * 16));
  return FO_OK;
}

// ---------------------------------------------------------------------------
// launch-table cache: one device table per distinct (device, kind, list)
// ---------------------------------------------------------------------------
struct TableEntry {
  int dev = -1;
  TensorDesc* dptr = nullptr;
  TensorDesc* hptr = nullptr;   // pinned staging copy
  size_t cap = 0;               // bytes
  hipEvent_t ev = nullptr;      // the staging copy of the last fill (hptr -> dptr)
  bool ev_recorded = false;
  SlotUses uses;                // streams whose launches read dptr since the fill
  int count = 0;                // non-empty tensors
  int64_t total_tiles = 0;
};

// Enough slots for one list per parameter of a large model (gradient release
// can step parameters one by one or in small buckets), so such lists do not
// evict each other; the slot index makes a lookup O(1) in the number of
// slots.  Slots read by a captured HIP graph are pinned (fo_slots.hpp).
constexpr size_t kCacheEntries = 1024;
std::mutex g_tab_mu;
std::vector<TableEntry> g_tab(kCacheEntries);
SlotCache g_slots(kCacheEntries);

std::string index_key(int dev, const std::vector<uint8_t>& key) {
  std::string k(sizeof(int) + key.size(), '\0');
  std::memcpy(&k[0], &dev, sizeof(int));
  if (!key.empty()) std::memcpy(&k[sizeof(int)], key.data(), key.size());
  return k;
}

// caller holds g_tab_mu
TableEntry* find_entry(int dev, const std::vector<uint8_t>& key) {
  const long slot = g_slots.find(index_key(dev, key));
  return slot < 0 ? nullptr : &g_tab[(size_t)slot];
}

struct Range { uintptr_t lo, hi; };

int check_alias(Range* r, size_t n) {
  std::sort(r, r + n, [](const Range& a, const Range& b) { return a.lo < b.lo; });
  for (size_t i = 1; i < n; ++i)
    if (r[i].lo < r[i - 1].hi) return fail(FO_EALIAS, "arrays of the tensor list overlap (%p .. %p)",
                                            (void*)r[i - 1].lo, (void*)r[i].lo);
  return FO_OK;
}
int check_alias(std::vector<Range>& r) { return check_alias(r.data(), r.size()); }

// Wait for the device `dev` to finish all queued work (the current device is
// restored afterwards).
int sync_device(int dev) {
  int cur = -1;
  hipError_t he = hipGetDevice(&cur);
  if (he != hipSuccess) return hip_fail(he, "hipGetDevice");
  if (cur != dev && (he = hipSetDevice(dev)) != hipSuccess) return hip_fail(he, "hipSetDevice");
  const hipError_t hs = hipDeviceSynchronize();
  if (cur != dev && (he = hipSetDevice(cur)) != hipSuccess) return hip_fail(he, "hipSetDevice");
  return hs == hipSuccess ? FO_OK : hip_fail(hs, "hipDeviceSynchronize");
}

// Build (or fetch) the device table for `descs` (already validated, n > 0 only).
// On success *out stays the caller's while it holds g_tab_mu.  A miss fills a
// slot: that copies the table from pinned host memory and may wait for the
// slot's earlier users, neither of which a graph capture can hold, so a miss
// under capture is refused (the list must be stepped once before capture).
int get_table(int dev, const std::vector<uint8_t>& key, const std::vector<TensorDesc>& descs,
              const std::vector<int32_t>& buckets, int64_t total_tiles, hipStream_t stream, TableEntry** out) {
  if ((*out = find_entry(dev, key))) return FO_OK;
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  hipError_t he = hipStreamIsCapturing(stream, &cs);
  if (he != hipSuccess) return hip_fail(he, "hipStreamIsCapturing");
  if (cs != hipStreamCaptureStatusNone)
    return fail(FO_EINVAL, "this tensor list has no launch table yet: step it once outside HIP graph capture "
                           "before capturing it");
  // miss: refill the least recently used slot that no captured graph reads
  const long vi = g_slots.victim();
  if (vi < 0)
    return fail(FO_ENOMEM, "all %zu launch-table slots are held by captured HIP graphs", kCacheEntries);
  TableEntry& e = g_tab[(size_t)vi];
  g_slots.drop(vi);
  // device layout: descriptors (with the sentinel), then the tile-bucket index
  const size_t desc_bytes = descs.size() * sizeof(TensorDesc);
  const size_t need = desc_bytes + buckets.size() * sizeof(int32_t);
  const bool replace = (e.dev != dev || e.cap < need);
  // the slot's earlier readers: its last staging copy, then the launches
  if (e.ev_recorded) {
    he = hipEventSynchronize(e.ev);
    if (he != hipSuccess) return hip_fail(he, "hipEventSynchronize");
    e.ev_recorded = false;
  }
  int rc = FO_OK;
  switch (refill_wait(e.uses, stream, replace, e.dev == dev)) {
    case RefillWait::NONE: break;
    case RefillWait::STREAM:
      if ((he = hipStreamSynchronize(stream)) != hipSuccess) return hip_fail(he, "hipStreamSynchronize");
      break;
    case RefillWait::DEVICE:
      if ((rc = sync_device(e.dev))) return rc;
      break;
  }
  e.uses.clear();
  if (replace) {
    if (e.dptr) { (void)hipFree(e.dptr); e.dptr = nullptr; }
    if (e.hptr) { (void)hipHostFree(e.hptr); e.hptr = nullptr; }
    if (e.ev) { (void)hipEventDestroy(e.ev); e.ev = nullptr; }
    e.cap = 0;
    e.dev = -1;
    const size_t cap = std::max<size_t>(need, 64 * sizeof(TensorDesc));
    he = hipMalloc((void**)&e.dptr, cap);
    if (he != hipSuccess) { e.dptr = nullptr; return fail(FO_ENOMEM, "hipMalloc(launch table): %s", hipGetErrorString(he)); }
    he = hipHostMalloc((void**)&e.hptr, cap, hipHostMallocDefault);
    if (he != hipSuccess) { e.hptr = nullptr; return fail(FO_ENOMEM, "hipHostMalloc(launch table): %s", hipGetErrorString(he)); }
    he = hipEventCreateWithFlags(&e.ev, hipEventDisableTiming);
    if (he != hipSuccess) { e.ev = nullptr; return hip_fail(he, "hipEventCreate"); }
    e.cap = cap;
    e.dev = dev;
  }
  std::memcpy(e.hptr, descs.data(), desc_bytes);
  std::memcpy(reinterpret_cast<uint8_t*>(e.hptr) + desc_bytes, buckets.data(), buckets.size() * sizeof(int32_t));
  he = hipMemcpyAsync(e.dptr, e.hptr, need, hipMemcpyHostToDevice, stream);
  if (he != hipSuccess) return hip_fail(he, "hipMemcpyAsync(launch table)");
  // the next refill rewrites hptr from the host: it waits for this copy
  he = hipEventRecord(e.ev, stream);
  if (he != hipSuccess) return hip_fail(he, "hipEventRecord(launch table)");
  e.ev_recorded = true;
  g_slots.store(vi, index_key(dev, key));
  e.count = (int)descs.size() - 1;
  e.total_tiles = total_tiles;
  *out = &e;
  return FO_OK;
}

// After the launches that read `e`: note their stream (a later refill of the
// slot decides from the streams what it must wait for; no event is recorded
// per call, since an event between two steps holds the next step's launch
// back by several microseconds), or, when `stream` is being captured into a
// HIP graph, pin the slot, since the graph may replay them at any time.
int use_entry(TableEntry* e, hipStream_t stream) {
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  hipError_t he = hipStreamIsCapturing(stream, &cs);
  if (he != hipSuccess) return hip_fail(he, "hipStreamIsCapturing");
  if (cs != hipStreamCaptureStatusNone) {
    g_slots.pin((long)(e - g_tab.data()));
    return FO_OK;
  }
  e->uses.add(stream);
  return FO_OK;
}

// ---------------------------------------------------------------------------
// list validation -> device descriptors
// ---------------------------------------------------------------------------
// one array of a tensor: elem_bytes per element (per 32-element block when
// per_block); elem_bytes 0 means 4-bit codes, two per byte
struct ArraySpec { const void* p; size_t elem_bytes; bool per_block; const char* name; };
inline int64_t array_extent(const ArraySpec& s, int64_t n, int64_t nb) {
  if (s.per_block) return nb * (int64_t)s.elem_bytes;
  return s.elem_bytes == 0 ? (n + 1) / 2 : n * (int64_t)s.elem_bytes;
}
// bytes per element of a codec's code array (0 = two codes per byte)
inline size_t code_elem_bytes(int codec) { return codec == FO_COMPANDED4 ? 0 : 1; }
inline bool codec_ok(int codec) {
  return codec == FO_COMPANDED || codec == FO_LINEAR || codec == FO_COMPANDED4 || codec == FO_COMPANDED_BF16SCALE;
}

// Element counts above 2^56 cannot describe device memory; rejecting them
// keeps every byte-range computation below within int64 / uintptr_t.
constexpr int64_t kMaxElems = int64_t(1) << 56;

constexpr int kArraysPerTensor = 7;          // w16, ecc, grad, codes 1, scales 1, codes 2, scales 2
constexpr int kMaxBucketEntries = 65536 + 2;  // the index has (tiles >> shift) + 2 <= 65537 entries

// Launch table of a tensor list, built on caller storage: arrays[i * 7 + a]
// (a < na) and ns[i] describe tensor i < ntens; body holds ntens descriptors,
// ranges ntens * na, descs ntens + 1 (the non-empty tensors and the
// sentinel: *ndesc of them), buckets kMaxBucketEntries (*nbuckets used).
int build_descs_into(int ntens, int na, const ArraySpec* arrays, const int64_t* ns, TensorDesc* body, Range* ranges,
                     TensorDesc* descs, int* ndesc, int32_t* buckets, int* nbuckets, int64_t* total_tiles) {
  int nbody = 0;
  size_t nranges = 0;
  int64_t tiles = 0;
  for (int i = 0; i < ntens; ++i) {
    const int64_t n = ns[i];
    if (n < 0 || n > kMaxElems) return fail(FO_EINVAL, "tensor %d: n out of range (%lld)", i, (long long)n);
    if (n == 0) continue;
    const int64_t nb = (n + 31) / 32;
    uint64_t ptr[kArraysPerTensor] = {0, 0, 0, 0, 0, 0, 0};
    for (int a = 0; a < na; ++a) {
      const ArraySpec& s = arrays[(size_t)i * kArraysPerTensor + a];
      if (!s.p) return fail(FO_EINVAL, "tensor %d: %s is NULL", i, s.name);
      if (!aligned(s.p, s.per_block ? 2 : 16)) return fail(FO_EINVAL, "tensor %d: %s is not %d-byte aligned", i, s.name,
                                                            s.per_block ? 2 : 16);
      const uintptr_t lo = reinterpret_cast<uintptr_t>(s.p);
      ranges[nranges++] = {lo, lo + (uintptr_t)array_extent(s, n, nb)};
      ptr[a] = (uint64_t)lo;
    }
    TensorDesc d;
    d.w16 = ptr[0]; d.ecc = ptr[1]; d.grad = ptr[2]; d.q1 = ptr[3]; d.s1 = ptr[4]; d.q2 = ptr[5]; d.s2 = ptr[6];
    d.n = n;
    d.tile_begin = 0;
    body[nbody++] = d;
  }
  int rc = check_alias(ranges, nranges);
  if (rc) return rc;
  // Tile order: tensors whose last tile is partial come first, so their
  // masked tiles run in a launch's first wave round, where the other waves
  // hide their extra latency, instead of stretching its tail.  Tensors are
  // independent, so the order changes no result.
  int nd = 0;
  for (int pass = 0; pass < 2; ++pass) {
    for (int i = 0; i < nbody; ++i) {
      TensorDesc d = body[i];
      if ((d.n % TILE != 0) != (pass == 0)) continue;
      d.tile_begin = tiles;
      tiles += (d.n + TILE - 1) / TILE;
      descs[nd++] = d;
    }
  }
  // Tile-bucket index: bucket b (tiles [b << shift, (b + 1) << shift)) records
  // the tensor holding its first tile, so a wave searches only between two
  // adjacent entries.  At most 65536 buckets; the shift rides in the sentinel.
  int shift = TILE_BUCKET_SHIFT_MIN;
  while ((tiles >> shift) > 65535) ++shift;
  int nbk_entries = 0;
  if (tiles > 0) {
    const int64_t nbk = (tiles >> shift) + 1;
    nbk_entries = (int)nbk + 1;
    int t = 0;
    for (int64_t b = 0; b <= nbk; ++b) {
      const int64_t first = std::min<int64_t>(b << shift, tiles - 1);
      while (t + 1 < nd && descs[t + 1].tile_begin <= first) ++t;
      buckets[b] = t;
    }
  }
  TensorDesc sentinel;
  std::memset(&sentinel, 0, sizeof(sentinel));
  sentinel.tile_begin = tiles;
  sentinel.n = shift;
  descs[nd++] = sentinel;
  *ndesc = nd;
  *nbuckets = nbk_entries;
  *total_tiles = tiles;
  return FO_OK;
}

int build_descs(int ntens, int na, const std::vector<ArraySpec>& arrays, const std::vector<int64_t>& ns,
                std::vector<TensorDesc>* descs, std::vector<int32_t>* buckets, int64_t* total_tiles) {
  std::vector<TensorDesc> body((size_t)ntens);
  std::vector<Range> ranges((size_t)ntens * na);
  descs->resize((size_t)ntens + 1);
  buckets->resize(kMaxBucketEntries);
  int nd = 0, nbk = 0;
  const int rc = build_descs_into(ntens, na, arrays.data(), ns.data(), body.data(), ranges.data(), descs->data(), &nd,
                                  buckets->data(), &nbk, total_tiles);
  if (rc) return rc;
  descs->resize((size_t)nd);
  buckets->resize((size_t)nbk);
  return FO_OK;
}

hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

// ---------------------------------------------------------------------------
// kernel selection
// ---------------------------------------------------------------------------
#define FO_SELECT3(KERNEL, wfmt, ecc, codec, OUT)                                           \
  do {                                                                                      \
    if (wfmt == FO_BF16 && ecc == 8 && codec == FO_COMPANDED) OUT = KERNEL<BF16, 8, COMPANDED>; \
    else if (wfmt == FO_BF16 && ecc == 8 && codec == FO_LINEAR) OUT = KERNEL<BF16, 8, LINEAR>;  \
    else if (wfmt == FO_BF16 && ecc == 16 && codec == FO_COMPANDED) OUT = KERNEL<BF16, 16, COMPANDED>; \
    else if (wfmt == FO_BF16 && ecc == 16 && codec == FO_LINEAR) OUT = KERNEL<BF16, 16, LINEAR>; \
    else if (wfmt == FO_FP16 && ecc == 8 && codec == FO_COMPANDED) OUT = KERNEL<FP16, 8, COMPANDED>; \
    else if (wfmt == FO_FP16 && ecc == 8 && codec == FO_LINEAR) OUT = KERNEL<FP16, 8, LINEAR>;  \
    else if (wfmt == FO_BF16 && ecc == 8 && codec == FO_COMPANDED4) OUT = KERNEL<BF16, 8, COMPANDED4>; \
    else if (wfmt == FO_BF16 && ecc == 16 && codec == FO_COMPANDED4) OUT = KERNEL<BF16, 16, COMPANDED4>; \
    else if (wfmt == FO_FP16 && ecc == 8 && codec == FO_COMPANDED4) OUT = KERNEL<FP16, 8, COMPANDED4>; \
    else if (wfmt == FO_BF16 && ecc == 8 && codec == FO_COMPANDED_BF16SCALE) OUT = KERNEL<BF16, 8, COMPANDED_BF16S>; \
    else if (wfmt == FO_BF16 && ecc == 16 && codec == FO_COMPANDED_BF16SCALE) OUT = KERNEL<BF16, 16, COMPANDED_BF16S>; \
    else if (wfmt == FO_FP16 && ecc == 8 && codec == FO_COMPANDED_BF16SCALE) OUT = KERNEL<FP16, 8, COMPANDED_BF16S>; \
  } while (0)

// AdamW (decoupled decay) and Adam (L2 decay folded into the gradient)
template <int W, int E, int C>
constexpr auto k_fused_adamw_dec = k_fused_adamw<W, E, C, false>;
template <int W, int E, int C>
constexpr auto k_fused_adamw_l2 = k_fused_adamw<W, E, C, true>;

int launch_check(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e, what);
  return FO_OK;
}

// Range of (effective) gradients for which the fused AdamW step's fast
// arithmetic is exact: g = 0 or g_lo <= |g| <= g_hi (see AdamWConsts).  It
// follows from the f32 step constants and the ranges every finite stored
// state decodes into:
//   momentum |m_hat| in {0} u [2^-33, 66021]  (scale >= 2^-24: level >= 2^-24/253;
//                                              linear code -128: 128/127 * 65504)
//   variance  v_hat  in {0} u [2^-66, 2^33]
// Conditions, each with a margin for the rounding of the products:
//   v = b2*v_hat + (1-b2)*g*g outside (0, 2^-96) and at most 2^100 (the
//     square root from the successor's estimate is exact there) and so
//     small that den = sqrt(v)*ibc2 + eps <= 2^52;
//   a nonzero m = b1*m_hat + (1-b1)*g at least 2^-73: both terms are 0 or at
//     least 2^-50, and a sum of such floats that does not vanish is a nonzero
//     multiple of 2^-73;
//   so every nonzero quotient m/den is a normal number (>= 2^-125), and
//   |m/den| < 2^119 because den >= eps.
// That keeps rcp_refined, div_refined and sqrt_fast in their exact ranges.  When no such range exists (eps not a normal number, b1 or b2 tiny,
// ibc2 huge) every wave takes the IEEE form.
static void adamw_fast_range(AdamWConsts* c, int wfmt) {
  c->fast = 0;
  c->g_lo2 = 0xFFFFFFFEu;
  c->g_hi = 0.0f;
  c->g16_lo = 0xFFFFu;     // every nonzero pattern is below: no fast range
  c->g16_hi = 0u;
  const double b1 = c->b1, b2 = c->b2, omb1 = c->omb1, omb2 = c->omb2, eps = c->eps, ibc2 = c->ibc2;
  if (!(eps >= 0x1p-126) || !(omb1 > 0.0) || !(omb2 > 0.0) || !(ibc2 > 0.0 && ibc2 < 0x1p35)) return;
  if (b1 != 0.0 && b1 < 0x1p-17) return;
  if (b2 != 0.0 && b2 < 0x1p-29) return;
  const double v_hi = std::min(0x1p100, std::pow((0x1p52 - eps) / ibc2, 2.0)) * (1.0 - 0x1p-20);
  const double lo = std::max(std::sqrt(0x1p-95 / omb2), 0x1p-49 / omb1);
  const double hi = std::min(std::sqrt((v_hi - 0x1p34) / omb2), (0x1p119 * eps - 66021.0 * b1 - 1.0) / omb1);
  const float flo = std::nextafter((float)lo, INFINITY);        // rounded outwards: conservative
  const float fhi = std::nextafter((float)hi, 0.0f);
  if (!(flo > 0.0f) || !(fhi > flo) || !std::isfinite(fhi)) return;
  uint32_t blo;
  std::memcpy(&blo, &flo, 4);
  c->g_lo2 = 2u * blo - 2u;
  c->g_hi = fhi;
  c->g16_lo = grad16_last(wfmt == FO_BF16, flo, true);
  c->g16_hi = grad16_last(wfmt == FO_BF16, fhi, false);
  c->fast = 1;
}

}  // namespace

extern "C" {

int fo_abi_version(void) { return FO_ABI_VERSION; }

int fo_cache_pinned(void) {
  std::lock_guard<std::mutex> lk(g_tab_mu);
  return (int)g_slots.pinned_count();
}

const char* fo_last_error(void) { return g_err.c_str(); }

int fo_split_weights(const float* w32, int64_t n, int wfmt, int ecc_bits, void* w16_out, void* ecc_out,
                     void* stream) {
  g_err.clear();
  if (!fmt_ok(wfmt, ecc_bits)) return fail(FO_EINVAL, "unsupported format/ECC combination (%d, %d)", wfmt, ecc_bits);
  if (n < 0 || n > kMaxElems) return fail(FO_EINVAL, "n out of range (%lld)", (long long)n);
  if (n == 0) return FO_OK;
  if (!w32 || !w16_out || !ecc_out) return fail(FO_EINVAL, "NULL pointer");
  if (!aligned(w32, 16) || !aligned(w16_out, 16) || !aligned(ecc_out, 16)) return fail(FO_EINVAL, "pointer not 16-byte aligned");
  std::vector<Range> r = {{(uintptr_t)w32, (uintptr_t)w32 + n * 4}, {(uintptr_t)w16_out, (uintptr_t)w16_out + n * 2},
                          {(uintptr_t)ecc_out, (uintptr_t)ecc_out + n * (ecc_bits / 8)}};
  int rc = check_alias(r);
  if (rc) return rc;
  int dev, grid;
  if ((rc = current_device(&dev)) || (rc = elementwise_grid(dev, n, &grid))) return rc;
  auto* w = (uint16_t*)w16_out;
  auto* e = (uint8_t*)ecc_out;
  if (wfmt == FO_BF16 && ecc_bits == 8) hipLaunchKernelGGL((k_split<BF16, 8>), grid, WG, 0, as_stream(stream), w32, n, w, e);
  else if (wfmt == FO_BF16) hipLaunchKernelGGL((k_split<BF16, 16>), grid, WG, 0, as_stream(stream), w32, n, w, e);
  else hipLaunchKernelGGL((k_split<FP16, 8>), grid, WG, 0, as_stream(stream), w32, n, w, e);
  return launch_check("k_split launch");
}

int fo_reconstruct_weights(const void* w16, const void* ecc, int64_t n, int wfmt, int ecc_bits, float* w32_out,
                           void* stream) {
  g_err.clear();
  if (!fmt_ok(wfmt, ecc_bits)) return fail(FO_EINVAL, "unsupported format/ECC combination (%d, %d)", wfmt, ecc_bits);
  if (n < 0 || n > kMaxElems) return fail(FO_EINVAL, "n out of range (%lld)", (long long)n);
  if (n == 0) return FO_OK;
  if (!w16 || !ecc || !w32_out) return fail(FO_EINVAL, "NULL pointer");
  if (!aligned(w16, 16) || !aligned(ecc, 16) || !aligned(w32_out, 16)) return fail(FO_EINVAL, "pointer not 16-byte aligned");
  std::vector<Range> r = {{(uintptr_t)w32_out, (uintptr_t)w32_out + n * 4}, {(uintptr_t)w16, (uintptr_t)w16 + n * 2},
                          {(uintptr_t)ecc, (uintptr_t)ecc + n * (ecc_bits / 8)}};
  int rc = check_alias(r);
  if (rc) return rc;
  int dev, grid;
  if ((rc = current_device(&dev)) || (rc = elementwise_grid(dev, n, &grid))) return rc;
  auto* w = (const uint16_t*)w16;
  auto* e = (const uint8_t*)ecc;
  if (wfmt == FO_BF16 && ecc_bits == 8) hipLaunchKernelGGL((k_reconstruct<BF16, 8>), grid, WG, 0, as_stream(stream), w, e, n, w32_out);
  else if (wfmt == FO_BF16) hipLaunchKernelGGL((k_reconstruct<BF16, 16>), grid, WG, 0, as_stream(stream), w, e, n, w32_out);
  else hipLaunchKernelGGL((k_reconstruct<FP16, 8>), grid, WG, 0, as_stream(stream), w, e, n, w32_out);
  return launch_check("k_reconstruct launch");
}

int fo_companded_quantize(const float* x, int64_t n, int kind, int codec, void* codes_out, uint16_t* scales_out,
                          void* stream) {
  g_err.clear();
  if (kind != FO_MOMENTUM && kind != FO_VARIANCE) return fail(FO_EINVAL, "bad kind %d", kind);
  if (!codec_ok(codec)) return fail(FO_EINVAL, "bad codec %d", codec);
  if (n < 0 || n > kMaxElems) return fail(FO_EINVAL, "n out of range (%lld)", (long long)n);
  if (n == 0) return FO_OK;
  if (!x || !codes_out || !scales_out) return fail(FO_EINVAL, "NULL pointer");
  if (!aligned(x, 16) || !aligned(codes_out, 16) || !aligned(scales_out, 2)) return fail(FO_EINVAL, "misaligned pointer");
  const int64_t nb = (n + 31) / 32;
  const int64_t cb = array_extent({codes_out, code_elem_bytes(codec), false, "codes"}, n, nb);
  std::vector<Range> r = {{(uintptr_t)x, (uintptr_t)x + n * 4}, {(uintptr_t)codes_out, (uintptr_t)codes_out + cb},
                          {(uintptr_t)scales_out, (uintptr_t)scales_out + nb * 2}};
  int rc = check_alias(r);
  if (rc) return rc;
  int dev, grid;
  hipStream_t s = as_stream(stream);
  const CodecTables* tb = nullptr;
  if ((rc = current_device(&dev)) || (rc = elementwise_grid(dev, n, &grid)) || (rc = device_tables(dev, s, &tb))) return rc;
  auto* c = (uint8_t*)codes_out;
  void (*kern)(const float*, int64_t, uint8_t*, uint16_t*, const CodecTables*) =
      (kind == FO_MOMENTUM) ? (codec == FO_COMPANDED   ? k_quantize<0, COMPANDED>
                               : codec == FO_LINEAR    ? k_quantize<0, LINEAR>
                               : codec == FO_COMPANDED4 ? k_quantize<0, COMPANDED4>
                                                        : k_quantize<0, COMPANDED_BF16S>)
                            : (codec == FO_COMPANDED   ? k_quantize<1, COMPANDED>
                               : codec == FO_LINEAR    ? k_quantize<1, LINEAR>
                               : codec == FO_COMPANDED4 ? k_quantize<1, COMPANDED4>
                                                        : k_quantize<1, COMPANDED_BF16S>);
  hipLaunchKernelGGL(kern, grid, WG, 0, s, x, n, c, scales_out, tb);
  return launch_check("k_quantize launch");
}

int fo_dequantize(const void* codes, const uint16_t* scales, int64_t n, int kind, int codec, float* x_out, void* stream) {
  g_err.clear();
  if (kind != FO_MOMENTUM && kind != FO_VARIANCE) return fail(FO_EINVAL, "bad kind %d", kind);
  if (!codec_ok(codec)) return fail(FO_EINVAL, "bad codec %d", codec);
  if (n < 0 || n > kMaxElems) return fail(FO_EINVAL, "n out of range (%lld)", (long long)n);
  if (n == 0) return FO_OK;
  if (!codes || !scales || !x_out) return fail(FO_EINVAL, "NULL pointer");
  if (!aligned(codes, 16) || !aligned(scales, 2) || !aligned(x_out, 16)) return fail(FO_EINVAL, "misaligned pointer");
  const int64_t nb = (n + 31) / 32;
  const int64_t cb = array_extent({codes, code_elem_bytes(codec), false, "codes"}, n, nb);
  std::vector<Range> r = {{(uintptr_t)x_out, (uintptr_t)x_out + n * 4}, {(uintptr_t)codes, (uintptr_t)codes + cb},
                          {(uintptr_t)scales, (uintptr_t)scales + nb * 2}};
  int rc = check_alias(r);
  if (rc) return rc;
  int dev, grid;
  hipStream_t s = as_stream(stream);
  const CodecTables* tb = nullptr;
  if ((rc = current_device(&dev)) || (rc = elementwise_grid(dev, n, &grid)) || (rc = device_tables(dev, s, &tb))) return rc;
  auto* c = (const uint8_t*)codes;
  void (*kern)(const uint8_t*, const uint16_t*, int64_t, float*, const CodecTables*) =
      (kind == FO_MOMENTUM) ? (codec == FO_COMPANDED   ? k_dequantize<0, COMPANDED>
                               : codec == FO_LINEAR    ? k_dequantize<0, LINEAR>
                               : codec == FO_COMPANDED4 ? k_dequantize<0, COMPANDED4>
                                                        : k_dequantize<0, COMPANDED_BF16S>)
                            : (codec == FO_COMPANDED   ? k_dequantize<1, COMPANDED>
                               : codec == FO_LINEAR    ? k_dequantize<1, LINEAR>
                               : codec == FO_COMPANDED4 ? k_dequantize<1, COMPANDED4>
                                                        : k_dequantize<1, COMPANDED_BF16S>);
  hipLaunchKernelGGL(kern, grid, WG, 0, s, c, scales, n, x_out, tb);
  return launch_check("k_dequantize launch");
}

// Device table of a tensor list.  The cache is consulted first: an identical
// list was validated when it was stored.  On a miss the list is validated
// before any device error is returned, so argument errors are reported even
// where no device is usable.  `fill` describes each tensor's arrays.  The
// caller holds g_tab_mu; the entry stays the caller's until its use is
// recorded.
// fill(arrays, ns): arrays[i * kArraysPerTensor + a] for the `na` arrays of tensor i
using FillArrays = std::function<void(ArraySpec*, int64_t*)>;
static int list_table(const std::vector<uint8_t>& key, int32_t count, int na, const FillArrays& fill,
                      hipStream_t stream, TableEntry** entry) {
  int dev = -1;
  const int dev_rc = current_device(&dev);
  if (dev_rc == FO_OK && (*entry = find_entry(dev, key))) return FO_OK;
  std::vector<ArraySpec> arrays((size_t)count * kArraysPerTensor);
  std::vector<int64_t> ns(count);
  fill(arrays.data(), ns.data());
  std::vector<TensorDesc> descs;
  std::vector<int32_t> buckets;
  int64_t tiles = 0;
  const int rc = build_descs(count, na, arrays, ns, &descs, &buckets, &tiles);
  if (rc) return rc;
  if (tiles == 0) { *entry = nullptr; g_err.clear(); return FO_OK; }   // only empty tensors: nothing to do
  if (dev_rc) return dev_rc;                  // its message is still the current one
  return get_table(dev, key, descs, buckets, tiles, stream, entry);
}

static void fill_adamw_arrays(const fo_adamw_tensor* list, int32_t count, int ecc_bits, int codec, ArraySpec* arrays,
                              int64_t* ns) {
  const size_t eb = (size_t)ecc_bits / 8, qb = code_elem_bytes(codec);
  for (int i = 0; i < count; ++i) {
    const fo_adamw_tensor& t = list[i];
    ns[i] = t.n;
    ArraySpec* a = arrays + (size_t)i * kArraysPerTensor;
    a[0] = {t.w16, 2, false, "w16"}; a[1] = {t.ecc, eb, false, "ecc"}; a[2] = {t.grad, 2, false, "grad"};
    a[3] = {t.m_q, qb, false, "m_q"}; a[4] = {t.m_s, 2, true, "m_s"}; a[5] = {t.v_q, qb, false, "v_q"};
    a[6] = {t.v_s, 2, true, "v_s"};
  }
}

// The cache key holds what the validation depends on: the entry point, the
// formats (array extents) and the list itself.
static int adamw_like_table(const fo_adamw_tensor* list, int32_t count, int wfmt, int ecc_bits, int codec,
                            uint8_t tag, hipStream_t stream, TableEntry** entry) {
  const int32_t qb = (int32_t)code_elem_bytes(codec);
  std::vector<uint8_t> key(1 + sizeof(int32_t) * 3 + (size_t)count * sizeof(fo_adamw_tensor));
  key[0] = tag;
  std::memcpy(&key[1], &wfmt, 4);
  std::memcpy(&key[5], &ecc_bits, 4);
  std::memcpy(&key[9], &qb, 4);
  if (count) std::memcpy(&key[13], list, (size_t)count * sizeof(fo_adamw_tensor));
  return list_table(key, count, 7, [&](ArraySpec* arrays, int64_t* ns) {
    fill_adamw_arrays(list, count, ecc_bits, codec, arrays, ns);
  }, stream, entry);
}

// Argument checks, step constants, kernel choice and launches of the fused
// AdamW step, shared by fo_fused_adamw_step and fo_fused_adamw_step_noalloc.
static int adamw_check_args(const fo_adamw_tensor* list, int32_t count, const fo_adamw_hparams* hp) {
  if (!hp) return fail(FO_EINVAL, "hp is NULL");
  if (count < 0) return fail(FO_EINVAL, "count < 0");
  if (count > 0 && !list) return fail(FO_EINVAL, "list is NULL");
  if (!fmt_ok(hp->wfmt, hp->ecc_bits)) return fail(FO_EINVAL, "unsupported format/ECC combination (%d, %d)", hp->wfmt, hp->ecc_bits);
  if (!codec_ok(hp->codec)) return fail(FO_EINVAL, "bad codec %d", hp->codec);
  if (hp->step < 1) return fail(FO_EINVAL, "step must be >= 1");
  if (hp->l2_decay != 0 && hp->l2_decay != 1) return fail(FO_EINVAL, "l2_decay must be 0 or 1");
  if (!(hp->beta1 >= 0.0 && hp->beta1 < 1.0 && hp->beta2 >= 0.0 && hp->beta2 < 1.0))
    return fail(FO_EINVAL, "betas must lie in [0, 1)");
  if (!(hp->lr >= 0.0) || !(hp->eps >= 0.0) || !(hp->weight_decay >= 0.0))
    return fail(FO_EINVAL, "lr, eps and weight_decay must be >= 0");
  return FO_OK;
}

// per-step float32 constants: double arithmetic, one rounding each
static AdamWConsts adamw_consts(const fo_adamw_hparams* hp) {
  const double t = (double)hp->step;
  AdamWConsts c;
  c.b1 = (float)hp->beta1;
  c.b2 = (float)hp->beta2;
  c.omb1 = (float)(1.0 - hp->beta1);
  c.omb2 = (float)(1.0 - hp->beta2);
  c.decay = (float)(1.0 - hp->lr * hp->weight_decay);
  c.step_size = (float)(hp->lr / (1.0 - std::pow(hp->beta1, t)));
  c.ibc2 = (float)(1.0 / std::sqrt(1.0 - std::pow(hp->beta2, t)));
  c.eps = (float)hp->eps;
  c.wd = hp->l2_decay ? (float)hp->weight_decay : 0.0f;
  if (hp->l2_decay) c.decay = 1.0f;                 // Adam: no decoupled decay
  adamw_fast_range(&c, hp->wfmt);
  return c;
}

static int adamw_launch(const fo_adamw_hparams* hp, const TensorDesc* tab, int count, int64_t total_tiles,
                        const CodecTables* tables, hipStream_t s) {
  const AdamWConsts c = adamw_consts(hp);
  void (*kern)(const TensorDesc*, int, int64_t, int64_t, const CodecTables*, AdamWConsts) = nullptr;
  if (hp->l2_decay) FO_SELECT3(k_fused_adamw_l2, hp->wfmt, hp->ecc_bits, hp->codec, kern);
  else FO_SELECT3(k_fused_adamw_dec, hp->wfmt, hp->ecc_bits, hp->codec, kern);
  const int waves = adamw_waves(hp->ecc_bits);
  int grid, rc;
  for (int64_t t0 = 0; t0 < total_tiles; t0 += kLaunchTiles) {
    const int64_t t1 = std::min<int64_t>(t0 + kLaunchTiles, total_tiles);
    if ((rc = tile_grid(t1 - t0, waves, &grid))) return rc;
    hipLaunchKernelGGL(kern, grid, WAVE * waves, 0, s, tab, count, t0, t1, tables, c);
  }
  return launch_check("k_fused_adamw launch");
}

int fo_fused_adamw_step(const fo_adamw_tensor* list, int32_t count, const fo_adamw_hparams* hp, void* stream) {
  g_err.clear();
  int rc = adamw_check_args(list, count, hp);
  if (rc || count == 0) return rc;
  hipStream_t s = as_stream(stream);
  std::lock_guard<std::mutex> lk(g_tab_mu);   // table slot stays ours until the use is recorded
  TableEntry* e = nullptr;
  rc = adamw_like_table(list, count, hp->wfmt, hp->ecc_bits, hp->codec, 'A', s, &e);
  if (rc) return rc;
  if (!e || e->total_tiles == 0) return FO_OK;
  int dev;
  const CodecTables* tb = nullptr;
  if ((rc = current_device(&dev)) || (rc = device_tables(dev, s, &tb))) return rc;
  if ((rc = adamw_launch(hp, (const TensorDesc*)e->dptr, e->count, e->total_tiles, tb, s))) return rc;
  return use_entry(e, s);
}

// ---------------------------------------------------------------------------
// allocation-free AdamW step
// ---------------------------------------------------------------------------
// The library's device memory of this entry point is one file-scope device
// array per GPU, held until the process ends: the codec tables, then the
// launch table (descriptors, sentinel, tile-bucket index) of the current
// call.  The descriptors reach it as kernel arguments (k_put_table, in
// chunks) and the bucket index is computed there from them
// (k_bucket_index), so no host buffer is read after the call returns: the
// call neither allocates nor synchronises, and a captured call replays its
// own table.  The array's device address comes from hipGetSymbolAddress,
// taken once per device with that device current; host code uses only that
// address.
static constexpr int kNoAllocMaxTensors = 2048;
constexpr size_t kScratchDescOff = sizeof(CodecTables);                 // tables first
constexpr size_t kScratchTableBytes = (size_t)(kNoAllocMaxTensors + 1) * sizeof(TensorDesc) +
                                      (size_t)kMaxBucketEntries * sizeof(int32_t);
constexpr size_t kScratchBytes = kScratchDescOff + kScratchTableBytes;   // 438 KiB
static_assert(kScratchDescOff % 16 == 0, "descriptor alignment");
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kNoAllocMaxDevices = 64;
struct NoAllocDevice { uint8_t* ptr = nullptr; bool tables_built = false; };
static std::mutex g_na_mu;
static NoAllocDevice g_na_dev[kNoAllocMaxDevices];
static ArraySpec g_na_arrays[(size_t)kNoAllocMaxTensors * kArraysPerTensor];
static int64_t g_na_ns[kNoAllocMaxTensors];
static TensorDesc g_na_body[kNoAllocMaxTensors];
static Range g_na_ranges[(size_t)kNoAllocMaxTensors * kArraysPerTensor];
static TensorDesc g_na_descs[kNoAllocMaxTensors + 1];
static int32_t g_na_buckets[kMaxBucketEntries];
static TableChunk g_na_chunk;

// The device's scratch address (hipGetSymbolAddress on the first call on the
// device) and its codec tables (built into it by k_init_tables on the stream
// of that first call; the caller orders later calls on other streams after
// it).  Under graph capture the build becomes part of the graph and is made
// again by the next call outside capture.
static int noalloc_scratch(int dev, hipStream_t s, uint8_t** out) {
  if (dev < 0 || dev >= kNoAllocMaxDevices) return fail(FO_EINVAL, "device %d beyond the %d the library serves", dev,
                                                        kNoAllocMaxDevices);
  NoAllocDevice& d = g_na_dev[dev];
  if (!d.ptr) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    d.ptr = static_cast<uint8_t*>(p);
  }
  if (!d.tables_built) {
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    const hipError_t e = hipStreamIsCapturing(s, &cs);
    if (e != hipSuccess) return hip_fail(e, "hipStreamIsCapturing");
    hipLaunchKernelGGL(k_init_tables, 1, WG, 0, s, reinterpret_cast<CodecTables*>(d.ptr));
    const int rc = launch_check("k_init_tables launch");
    if (rc) return rc;
    d.tables_built = (cs == hipStreamCaptureStatusNone);
  }
  *out = d.ptr;
  return FO_OK;
}

int fo_fused_adamw_step_noalloc(const fo_adamw_tensor* list, int32_t count, const fo_adamw_hparams* hp,
                                void* stream) {
  g_err.clear();
  int rc = adamw_check_args(list, count, hp);
  if (rc || count == 0) return rc;
  if (count > kNoAllocMaxTensors)
    return fail(FO_EINVAL, "the allocation-free step takes at most %d tensors (got %d)", kNoAllocMaxTensors, count);
  hipStream_t s = as_stream(stream);
  std::lock_guard<std::mutex> lk(g_na_mu);
  fill_adamw_arrays(list, count, hp->ecc_bits, hp->codec, g_na_arrays, g_na_ns);
  int nd = 0, nbk = 0;
  int64_t tiles = 0;
  rc = build_descs_into(count, 7, g_na_arrays, g_na_ns, g_na_body, g_na_ranges, g_na_descs, &nd, g_na_buckets, &nbk,
                        &tiles);
  if (rc) return rc;
  if (tiles == 0) return FO_OK;
  int dev;
  uint8_t* ptr = nullptr;
  if ((rc = current_device(&dev)) || (rc = noalloc_scratch(dev, s, &ptr))) return rc;
  // descriptors (with the sentinel, which holds the bucket shift), then the
  // bucket index right after them, where the kernels look
  uint8_t* table = ptr + kScratchDescOff;
  const size_t desc_bytes = (size_t)nd * sizeof(TensorDesc);
  static_assert(sizeof(TensorDesc) % 16 == 0 && TABLE_CHUNK % 16 == 0, "16-byte chunk words");
  for (size_t off = 0; off < desc_bytes; off += TABLE_CHUNK) {
    const size_t b = std::min<size_t>(TABLE_CHUNK, desc_bytes - off);
    std::memcpy(g_na_chunk.data, reinterpret_cast<const uint8_t*>(g_na_descs) + off, b);
    g_na_chunk.offset = (uint32_t)off;
    g_na_chunk.bytes = (uint32_t)b;
    hipLaunchKernelGGL(k_put_table, 1, WG, 0, s, table, g_na_chunk);
  }
  const int shift = (int)g_na_descs[nd - 1].n;
  hipLaunchKernelGGL(k_bucket_index, (nbk + WG - 1) / WG, WG, 0, s, reinterpret_cast<const TensorDesc*>(table),
                     nd - 1, shift, nbk, tiles, reinterpret_cast<int32_t*>(table + desc_bytes));
  if ((rc = launch_check("launch-table kernels"))) return rc;
  return adamw_launch(hp, reinterpret_cast<const TensorDesc*>(table), nd - 1, tiles,
                      reinterpret_cast<const CodecTables*>(ptr), s);
}

int fo_stream_probe(const fo_adamw_tensor* list, int32_t count, int32_t wfmt, int32_t ecc_bits, uint32_t key,
                    void* stream) {
  g_err.clear();
  if (count < 0) return fail(FO_EINVAL, "count < 0");
  if (count > 0 && !list) return fail(FO_EINVAL, "list is NULL");
  if (!fmt_ok(wfmt, ecc_bits)) return fail(FO_EINVAL, "unsupported format/ECC combination (%d, %d)", wfmt, ecc_bits);
  if (count == 0) return FO_OK;
  hipStream_t s = as_stream(stream);
  std::lock_guard<std::mutex> lk(g_tab_mu);
  TableEntry* e = nullptr;
  int rc = adamw_like_table(list, count, wfmt, ecc_bits, FO_COMPANDED, 'A', s, &e);
  if (rc) return rc;
  if (!e || e->total_tiles == 0) return FO_OK;
  void (*kern)(const TensorDesc*, int, int64_t, int64_t, uint32_t) = (ecc_bits == 8) ? k_stream_probe<8> : k_stream_probe<16>;
  int grid;
  const int waves = adamw_waves(ecc_bits);
  for (int64_t t0 = 0; t0 < e->total_tiles; t0 += kLaunchTiles) {
    const int64_t t1 = std::min<int64_t>(t0 + kLaunchTiles, e->total_tiles);
    if ((rc = tile_grid(t1 - t0, waves, &grid))) return rc;
    hipLaunchKernelGGL(kern, grid, WAVE * waves, 0, s, (const TensorDesc*)e->dptr, e->count, t0, t1, key);
  }
  rc = launch_check("k_stream_probe launch");
  if (rc) return rc;
  return use_entry(e, s);
}

int fo_hbm_probe(void* dst, const void* src, int64_t bytes, int32_t mode, int32_t chunk_kib, uint32_t key,
                 void* stream) {
  g_err.clear();
  if (mode < 0 || mode > 3) return fail(FO_EINVAL, "bad probe mode %d", mode);
  if (chunk_kib != 1 && chunk_kib != 2 && chunk_kib != 4 && chunk_kib != 8)
    return fail(FO_EINVAL, "chunk must be 1, 2, 4 or 8 KiB (got %d)", chunk_kib);
  const int64_t chunk = 1024 * (int64_t)chunk_kib;
  if (bytes < 0 || bytes % chunk != 0) return fail(FO_EINVAL, "bytes must be a non-negative multiple of %lld",
                                                   (long long)chunk);
  if (bytes == 0) return FO_OK;
  if (mode == 3) src = dst;                                     // in place: dst is read and rewritten
  if (!dst || (mode != 1 && !src)) return fail(FO_EINVAL, "NULL pointer");
  if (!aligned(dst, 16) || (src && !aligned(src, 16))) return fail(FO_EINVAL, "pointer not 16-byte aligned");
  hipStream_t s = as_stream(stream);
  const int64_t chunks = bytes / chunk;
  auto* d = (uint8_t*)dst;
  auto* r = (const uint8_t*)src;
  for (int64_t c0 = 0; c0 < chunks; c0 += kLaunchTiles) {
    const int grid = (int)std::min<int64_t>(kLaunchTiles, chunks - c0);
    if (chunk_kib == 1) hipLaunchKernelGGL(k_hbm_probe<1>, grid, WAVE, 0, s, d, r, c0, (int)mode, key);
    else if (chunk_kib == 2) hipLaunchKernelGGL(k_hbm_probe<2>, grid, WAVE, 0, s, d, r, c0, (int)mode, key);
    else if (chunk_kib == 4) hipLaunchKernelGGL(k_hbm_probe<4>, grid, WAVE, 0, s, d, r, c0, (int)mode, key);
    else hipLaunchKernelGGL(k_hbm_probe<8>, grid, WAVE, 0, s, d, r, c0, (int)mode, key);
  }
  return launch_check("k_hbm_probe launch");
}

int fo_fused_sgdm_step(const fo_sgdm_tensor* list, int32_t count, const fo_sgdm_hparams* hp, void* stream) {
  g_err.clear();
  if (!hp) return fail(FO_EINVAL, "hp is NULL");
  if (count < 0) return fail(FO_EINVAL, "count < 0");
  if (count > 0 && !list) return fail(FO_EINVAL, "list is NULL");
  if (!fmt_ok(hp->wfmt, hp->ecc_bits)) return fail(FO_EINVAL, "unsupported format/ECC combination (%d, %d)", hp->wfmt, hp->ecc_bits);
  if (!codec_ok(hp->codec)) return fail(FO_EINVAL, "bad codec %d", hp->codec);
  if (hp->step < 1) return fail(FO_EINVAL, "step must be >= 1");
  if (!(hp->lr >= 0.0) || !(hp->momentum >= 0.0) || !(hp->weight_decay >= 0.0))
    return fail(FO_EINVAL, "lr, momentum and weight_decay must be >= 0");
  if (!(hp->dampening >= 0.0 && hp->dampening <= 1.0)) return fail(FO_EINVAL, "dampening must lie in [0, 1]");
  if (hp->nesterov != 0 && hp->nesterov != 1) return fail(FO_EINVAL, "nesterov must be 0 or 1");
  if (hp->nesterov && (hp->momentum <= 0.0 || hp->dampening != 0.0))
    return fail(FO_EINVAL, "Nesterov momentum needs momentum > 0 and dampening 0");
  if (count == 0) return FO_OK;
  hipStream_t s = as_stream(stream);
  const int32_t qb = (int32_t)code_elem_bytes(hp->codec);
  std::vector<uint8_t> key(1 + 12 + (size_t)count * sizeof(fo_sgdm_tensor));
  key[0] = 'S';
  std::memcpy(&key[1], &hp->wfmt, 4);
  std::memcpy(&key[5], &hp->ecc_bits, 4);
  std::memcpy(&key[9], &qb, 4);
  std::memcpy(&key[13], list, (size_t)count * sizeof(fo_sgdm_tensor));
  TableEntry* e = nullptr;
  std::lock_guard<std::mutex> lk(g_tab_mu);
  const size_t eb = (size_t)hp->ecc_bits / 8;
  int rc = list_table(key, count, 5, [&](ArraySpec* arrays, int64_t* ns) {
    for (int i = 0; i < count; ++i) {
      const fo_sgdm_tensor& t = list[i];
      ns[i] = t.n;
      ArraySpec* a = arrays + (size_t)i * kArraysPerTensor;
      a[0] = {t.w16, 2, false, "w16"}; a[1] = {t.ecc, eb, false, "ecc"}; a[2] = {t.grad, 2, false, "grad"};
      a[3] = {t.b_q, (size_t)qb, false, "b_q"}; a[4] = {t.b_s, 2, true, "b_s"};
    }
  }, s, &e);
  if (rc) return rc;
  if (!e || e->total_tiles == 0) return FO_OK;
  SGDMConsts c;
  c.lr = (float)hp->lr;
  c.mu = (float)hp->momentum;
  c.wd = (float)hp->weight_decay;
  c.damp1 = (float)(1.0 - hp->dampening);
  c.nesterov = hp->nesterov;
  // step 1 sets the buffer to d; with momentum 0 every step does (torch.optim.SGD
  // keeps no buffer then, so dampening has no effect)
  c.first = (hp->step == 1 || hp->momentum == 0.0) ? 1 : 0;
  void (*kern)(const TensorDesc*, int, int64_t, int64_t, const CodecTables*, SGDMConsts) = nullptr;
  FO_SELECT3(k_fused_sgdm, hp->wfmt, hp->ecc_bits, hp->codec, kern);
  int grid;
  const CodecTables* tb = nullptr;
  if ((rc = device_tables(e->dev, s, &tb))) return rc;
  for (int64_t t0 = 0; t0 < e->total_tiles; t0 += kLaunchTiles) {
    const int64_t t1 = std::min<int64_t>(t0 + kLaunchTiles, e->total_tiles);
    if ((rc = tile_grid(t1 - t0, SGDM_TILE_WAVES, &grid))) return rc;
    hipLaunchKernelGGL(kern, grid, WAVE * SGDM_TILE_WAVES, 0, s, (const TensorDesc*)e->dptr, e->count, t0, t1, tb, c);
  }
  rc = launch_check("k_fused_sgdm launch");
  if (rc) return rc;
  return use_entry(e, s);
}

int fo_selftest(int what, uint32_t lo, uint64_t count, uint64_t* mismatches, void* stream) {
  g_err.clear();
  if (what < 0 || what > 6) return fail(FO_EINVAL, "bad self-test %d", what);
  if (!mismatches) return fail(FO_EINVAL, "mismatches is NULL");
  if ((what <= 2 || what == 6) && count > (1ull << 32) - lo) return fail(FO_EINVAL, "range exceeds the f32 patterns");
  hipStream_t s = as_stream(stream);
  unsigned long long* d = nullptr;
  hipError_t e = hipMalloc((void**)&d, sizeof(*d));
  if (e != hipSuccess) return fail(FO_ENOMEM, "hipMalloc: %s", hipGetErrorString(e));
  unsigned long long h = 0;
  e = hipMemcpyAsync(d, &h, sizeof(h), hipMemcpyHostToDevice, s);
  if (e == hipSuccess) {
    hipLaunchKernelGGL(k_selftest, 4096, WG, 0, s, what, lo, count, d);
    e = hipGetLastError();
  }
  if (e == hipSuccess) e = hipMemcpyAsync(&h, d, sizeof(h), hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  (void)hipFree(d);
  if (e != hipSuccess) return hip_fail(e, "self-test");
  *mismatches = h;
  return FO_OK;
}

}  // extern "C"
