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
  std::vector<uint8_t> key;
  TensorDesc* dptr = nullptr;
  TensorDesc* hptr = nullptr;   // pinned staging copy
  size_t cap = 0;               // bytes
  hipEvent_t ev = nullptr;      // last stream-ordered use of dptr/hptr
  bool ev_recorded = false;
  uint64_t stamp = 0;
  int count = 0;                // non-empty tensors
  int64_t total_tiles = 0;
};

// Enough slots for one list per parameter of a large model (gradient release
// can step parameters one by one or in small buckets), so such lists do not
// evict each other; the index makes a lookup O(1) in the number of slots.
constexpr size_t kCacheEntries = 1024;
std::mutex g_tab_mu;
std::vector<TableEntry> g_tab(kCacheEntries);
std::unordered_map<std::string, size_t> g_index;   // (device, key) -> slot
uint64_t g_stamp = 0;

std::string index_key(int dev, const std::vector<uint8_t>& key) {
  std::string k(sizeof(int) + key.size(), '\0');
  std::memcpy(&k[0], &dev, sizeof(int));
  if (!key.empty()) std::memcpy(&k[sizeof(int)], key.data(), key.size());
  return k;
}

// caller holds g_tab_mu
TableEntry* find_entry(int dev, const std::vector<uint8_t>& key) {
  auto it = g_index.find(index_key(dev, key));
  if (it == g_index.end()) return nullptr;
  TableEntry& e = g_tab[it->second];
  e.stamp = ++g_stamp;
  return &e;
}

struct Range { uintptr_t lo, hi; };

int check_alias(std::vector<Range>& r) {
  std::sort(r.begin(), r.end(), [](const Range& a, const Range& b) { return a.lo < b.lo; });
  for (size_t i = 1; i < r.size(); ++i)
    if (r[i].lo < r[i - 1].hi) return fail(FO_EALIAS, "arrays of the tensor list overlap (%p .. %p)",
                                            (void*)r[i - 1].lo, (void*)r[i].lo);
  return FO_OK;
}

// Build (or fetch) the device table for `descs` (already validated, n > 0 only).
// On success *out stays the caller's while it holds g_tab_mu.
int get_table(int dev, const std::vector<uint8_t>& key, const std::vector<TensorDesc>& descs,
              const std::vector<int32_t>& buckets, int64_t total_tiles, hipStream_t stream, TableEntry** out) {
  if ((*out = find_entry(dev, key))) return FO_OK;
  // miss: evict the least recently used entry of the cache
  size_t vi = 0;
  for (size_t i = 1; i < g_tab.size(); ++i) if (g_tab[i].stamp < g_tab[vi].stamp) vi = i;
  TableEntry& e = g_tab[vi];
  if (!e.key.empty()) g_index.erase(index_key(e.dev, e.key));
  e.key.clear();
  hipError_t he;
  if (e.ev_recorded) {
    he = hipEventSynchronize(e.ev);           // previous users of this slot are done
    if (he != hipSuccess) return hip_fail(he, "hipEventSynchronize");
    e.ev_recorded = false;
  }
  // device layout: descriptors (with the sentinel), then the tile-bucket index
  const size_t desc_bytes = descs.size() * sizeof(TensorDesc);
  const size_t need = desc_bytes + buckets.size() * sizeof(int32_t);
  if (e.dev != dev || e.cap < need) {
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
  if (he != hipSuccess) { e.key.clear(); return hip_fail(he, "hipMemcpyAsync(launch table)"); }
  // the staging copy is in flight: mark the slot used now, so that a later
  // eviction waits for it even if the launch that follows fails
  he = hipEventRecord(e.ev, stream);
  if (he != hipSuccess) { e.key.clear(); return hip_fail(he, "hipEventRecord(launch table)"); }
  e.ev_recorded = true;
  e.key = key;
  g_index[index_key(dev, key)] = vi;
  e.count = (int)descs.size() - 1;
  e.total_tiles = total_tiles;
  e.stamp = ++g_stamp;
  *out = &e;
  return FO_OK;
}

int record_use(TableEntry* e, hipStream_t stream) {
  hipError_t he = hipEventRecord(e->ev, stream);
  if (he != hipSuccess) return hip_fail(he, "hipEventRecord");
  e->ev_recorded = true;
  return FO_OK;
}

// ---------------------------------------------------------------------------
// list validation -> device descriptors
// ---------------------------------------------------------------------------
struct ArraySpec { const void* p; size_t elem_bytes; bool per_block; const char* name; };

// Element counts above 2^56 cannot describe device memory; rejecting them
// keeps every byte-range computation below within int64 / uintptr_t.
constexpr int64_t kMaxElems = int64_t(1) << 56;

int build_descs(int ntens, const std::vector<std::vector<ArraySpec>>& arrays, const std::vector<int64_t>& ns,
                std::vector<TensorDesc>* descs, std::vector<int32_t>* buckets, int64_t* total_tiles) {
  std::vector<Range> ranges;
  std::vector<TensorDesc> body;
  descs->clear();
  int64_t tiles = 0;
  for (int i = 0; i < ntens; ++i) {
    const int64_t n = ns[i];
    if (n < 0 || n > kMaxElems) return fail(FO_EINVAL, "tensor %d: n out of range (%lld)", i, (long long)n);
    if (n == 0) continue;
    const int64_t nb = (n + 31) / 32;
    uint64_t ptr[7] = {0, 0, 0, 0, 0, 0, 0};
    for (size_t a = 0; a < arrays[i].size(); ++a) {
      const ArraySpec& s = arrays[i][a];
      if (!s.p) return fail(FO_EINVAL, "tensor %d: %s is NULL", i, s.name);
      if (!aligned(s.p, s.per_block ? 2 : 16)) return fail(FO_EINVAL, "tensor %d: %s is not %d-byte aligned", i, s.name,
                                                            s.per_block ? 2 : 16);
      const uintptr_t lo = reinterpret_cast<uintptr_t>(s.p);
      ranges.push_back({lo, lo + (uintptr_t)((s.per_block ? nb : n) * (int64_t)s.elem_bytes)});
      ptr[a] = (uint64_t)lo;
    }
    TensorDesc d;
    d.w16 = ptr[0]; d.ecc = ptr[1]; d.grad = ptr[2]; d.q1 = ptr[3]; d.s1 = ptr[4]; d.q2 = ptr[5]; d.s2 = ptr[6];
    d.n = n;
    body.push_back(d);
  }
  int rc = check_alias(ranges);
  if (rc) return rc;
  // Tile order: tensors whose last tile is partial come first, so their
  // masked tiles run in a launch's first wave round, where the other waves
  // hide their extra latency, instead of stretching its tail.  Tensors are
  // independent, so the order changes no result.
  for (int pass = 0; pass < 2; ++pass) {
    for (TensorDesc d : body) {
      if ((d.n % TILE != 0) != (pass == 0)) continue;
      d.tile_begin = tiles;
      tiles += (d.n + TILE - 1) / TILE;
      descs->push_back(d);
    }
  }
  // Tile-bucket index: bucket b (tiles [b << shift, (b + 1) << shift)) records
  // the tensor holding its first tile, so a wave searches only between two
  // adjacent entries.  At most 65536 buckets; the shift rides in the sentinel.
  int shift = TILE_BUCKET_SHIFT_MIN;
  while ((tiles >> shift) > 65535) ++shift;
  buckets->clear();
  if (tiles > 0) {
    const int64_t nbk = (tiles >> shift) + 1;
    buckets->resize((size_t)nbk + 1);
    int t = 0;
    const int ndesc = (int)descs->size();
    for (int64_t b = 0; b <= nbk; ++b) {
      const int64_t first = std::min<int64_t>(b << shift, tiles - 1);
      while (t + 1 < ndesc && (*descs)[t + 1].tile_begin <= first) ++t;
      (*buckets)[(size_t)b] = t;
    }
  }
  TensorDesc sentinel;
  std::memset(&sentinel, 0, sizeof(sentinel));
  sentinel.tile_begin = tiles;
  sentinel.n = shift;
  descs->push_back(sentinel);
  *total_tiles = tiles;
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

}  // namespace

extern "C" {

int fo_abi_version(void) { return FO_ABI_VERSION; }

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
  if (codec != FO_COMPANDED && codec != FO_LINEAR) return fail(FO_EINVAL, "bad codec %d", codec);
  if (n < 0 || n > kMaxElems) return fail(FO_EINVAL, "n out of range (%lld)", (long long)n);
  if (n == 0) return FO_OK;
  if (!x || !codes_out || !scales_out) return fail(FO_EINVAL, "NULL pointer");
  if (!aligned(x, 16) || !aligned(codes_out, 16) || !aligned(scales_out, 2)) return fail(FO_EINVAL, "misaligned pointer");
  const int64_t nb = (n + 31) / 32;
  std::vector<Range> r = {{(uintptr_t)x, (uintptr_t)x + n * 4}, {(uintptr_t)codes_out, (uintptr_t)codes_out + n},
                          {(uintptr_t)scales_out, (uintptr_t)scales_out + nb * 2}};
  int rc = check_alias(r);
  if (rc) return rc;
  int dev, grid;
  hipStream_t s = as_stream(stream);
  const CodecTables* tb = nullptr;
  if ((rc = current_device(&dev)) || (rc = elementwise_grid(dev, n, &grid)) || (rc = device_tables(dev, s, &tb))) return rc;
  auto* c = (uint8_t*)codes_out;
  if (kind == FO_MOMENTUM && codec == FO_COMPANDED) hipLaunchKernelGGL((k_quantize<0, COMPANDED>), grid, WG, 0, s, x, n, c, scales_out, tb);
  else if (kind == FO_MOMENTUM) hipLaunchKernelGGL((k_quantize<0, LINEAR>), grid, WG, 0, s, x, n, c, scales_out, tb);
  else if (codec == FO_COMPANDED) hipLaunchKernelGGL((k_quantize<1, COMPANDED>), grid, WG, 0, s, x, n, c, scales_out, tb);
  else hipLaunchKernelGGL((k_quantize<1, LINEAR>), grid, WG, 0, s, x, n, c, scales_out, tb);
  return launch_check("k_quantize launch");
}

int fo_dequantize(const void* codes, const uint16_t* scales, int64_t n, int kind, int codec, float* x_out, void* stream) {
  g_err.clear();
  if (kind != FO_MOMENTUM && kind != FO_VARIANCE) return fail(FO_EINVAL, "bad kind %d", kind);
  if (codec != FO_COMPANDED && codec != FO_LINEAR) return fail(FO_EINVAL, "bad codec %d", codec);
  if (n < 0 || n > kMaxElems) return fail(FO_EINVAL, "n out of range (%lld)", (long long)n);
  if (n == 0) return FO_OK;
  if (!codes || !scales || !x_out) return fail(FO_EINVAL, "NULL pointer");
  if (!aligned(codes, 16) || !aligned(scales, 2) || !aligned(x_out, 16)) return fail(FO_EINVAL, "misaligned pointer");
  const int64_t nb = (n + 31) / 32;
  std::vector<Range> r = {{(uintptr_t)x_out, (uintptr_t)x_out + n * 4}, {(uintptr_t)codes, (uintptr_t)codes + n},
                          {(uintptr_t)scales, (uintptr_t)scales + nb * 2}};
  int rc = check_alias(r);
  if (rc) return rc;
  int dev, grid;
  hipStream_t s = as_stream(stream);
  const CodecTables* tb = nullptr;
  if ((rc = current_device(&dev)) || (rc = elementwise_grid(dev, n, &grid)) || (rc = device_tables(dev, s, &tb))) return rc;
  auto* c = (const uint8_t*)codes;
  if (kind == FO_MOMENTUM && codec == FO_COMPANDED) hipLaunchKernelGGL((k_dequantize<0, COMPANDED>), grid, WG, 0, s, c, scales, n, x_out, tb);
  else if (kind == FO_MOMENTUM) hipLaunchKernelGGL((k_dequantize<0, LINEAR>), grid, WG, 0, s, c, scales, n, x_out, tb);
  else if (codec == FO_COMPANDED) hipLaunchKernelGGL((k_dequantize<1, COMPANDED>), grid, WG, 0, s, c, scales, n, x_out, tb);
  else hipLaunchKernelGGL((k_dequantize<1, LINEAR>), grid, WG, 0, s, c, scales, n, x_out, tb);
  return launch_check("k_dequantize launch");
}

// Device table of a tensor list.  The cache is consulted first: an identical
// list was validated when it was stored.  On a miss the list is validated
// before any device error is returned, so argument errors are reported even
// where no device is usable.  `fill` describes each tensor's arrays.  The
// caller holds g_tab_mu; the entry stays the caller's until its use is
// recorded.
using FillArrays = std::function<void(std::vector<std::vector<ArraySpec>>&, std::vector<int64_t>&)>;
static int list_table(const std::vector<uint8_t>& key, int32_t count, const FillArrays& fill, hipStream_t stream,
                      TableEntry** entry) {
  int dev = -1;
  const int dev_rc = current_device(&dev);
  if (dev_rc == FO_OK && (*entry = find_entry(dev, key))) return FO_OK;
  std::vector<std::vector<ArraySpec>> arrays(count);
  std::vector<int64_t> ns(count);
  fill(arrays, ns);
  std::vector<TensorDesc> descs;
  std::vector<int32_t> buckets;
  int64_t tiles = 0;
  const int rc = build_descs(count, arrays, ns, &descs, &buckets, &tiles);
  if (rc) return rc;
  if (tiles == 0) { *entry = nullptr; g_err.clear(); return FO_OK; }   // only empty tensors: nothing to do
  if (dev_rc) return dev_rc;                  // its message is still the current one
  return get_table(dev, key, descs, buckets, tiles, stream, entry);
}

static int adamw_like_table(const fo_adamw_tensor* list, int32_t count, int wfmt, int ecc_bits, uint8_t tag,
                            hipStream_t stream, TableEntry** entry) {
  std::vector<uint8_t> key(1 + sizeof(int32_t) * 2 + (size_t)count * sizeof(fo_adamw_tensor));
  key[0] = tag;
  std::memcpy(&key[1], &wfmt, 4);
  std::memcpy(&key[5], &ecc_bits, 4);
  if (count) std::memcpy(&key[9], list, (size_t)count * sizeof(fo_adamw_tensor));
  const size_t eb = (size_t)ecc_bits / 8;
  return list_table(key, count, [&](std::vector<std::vector<ArraySpec>>& arrays, std::vector<int64_t>& ns) {
    for (int i = 0; i < count; ++i) {
      const fo_adamw_tensor& t = list[i];
      ns[i] = t.n;
      arrays[i] = {{t.w16, 2, false, "w16"}, {t.ecc, eb, false, "ecc"}, {t.grad, 2, false, "grad"},
                   {t.m_q, 1, false, "m_q"}, {t.m_s, 2, true, "m_s"}, {t.v_q, 1, false, "v_q"},
                   {t.v_s, 2, true, "v_s"}};
    }
  }, stream, entry);
}

int fo_fused_adamw_step(const fo_adamw_tensor* list, int32_t count, const fo_adamw_hparams* hp, void* stream) {
  g_err.clear();
  if (!hp) return fail(FO_EINVAL, "hp is NULL");
  if (count < 0) return fail(FO_EINVAL, "count < 0");
  if (count > 0 && !list) return fail(FO_EINVAL, "list is NULL");
  if (!fmt_ok(hp->wfmt, hp->ecc_bits)) return fail(FO_EINVAL, "unsupported format/ECC combination (%d, %d)", hp->wfmt, hp->ecc_bits);
  if (hp->codec != FO_COMPANDED && hp->codec != FO_LINEAR) return fail(FO_EINVAL, "bad codec %d", hp->codec);
  if (hp->step < 1) return fail(FO_EINVAL, "step must be >= 1");
  if (hp->l2_decay != 0 && hp->l2_decay != 1) return fail(FO_EINVAL, "l2_decay must be 0 or 1");
  if (!(hp->beta1 >= 0.0 && hp->beta1 < 1.0 && hp->beta2 >= 0.0 && hp->beta2 < 1.0))
    return fail(FO_EINVAL, "betas must lie in [0, 1)");
  if (!(hp->lr >= 0.0) || !(hp->eps >= 0.0) || !(hp->weight_decay >= 0.0))
    return fail(FO_EINVAL, "lr, eps and weight_decay must be >= 0");
  if (count == 0) return FO_OK;
  hipStream_t s = as_stream(stream);
  std::lock_guard<std::mutex> lk(g_tab_mu);   // table slot stays ours until the use is recorded
  TableEntry* e = nullptr;
  int rc = adamw_like_table(list, count, hp->wfmt, hp->ecc_bits, 'A', s, &e);
  if (rc) return rc;
  if (!e || e->total_tiles == 0) return FO_OK;
  // per-step float32 constants: double arithmetic, one rounding each
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
  c.fast_rcp = (c.eps >= 0x1p-126f) ? 1 : 0;
  void (*kern)(const TensorDesc*, int, int64_t, int64_t, const CodecTables*, AdamWConsts) = nullptr;
  if (hp->l2_decay) FO_SELECT3(k_fused_adamw_l2, hp->wfmt, hp->ecc_bits, hp->codec, kern);
  else FO_SELECT3(k_fused_adamw_dec, hp->wfmt, hp->ecc_bits, hp->codec, kern);
  int dev, grid;
  const int waves = adamw_waves(hp->ecc_bits);
  const CodecTables* tb = nullptr;
  if ((rc = current_device(&dev)) || (rc = device_tables(dev, s, &tb))) return rc;
  for (int64_t t0 = 0; t0 < e->total_tiles; t0 += kLaunchTiles) {
    const int64_t t1 = std::min<int64_t>(t0 + kLaunchTiles, e->total_tiles);
    if ((rc = tile_grid(t1 - t0, waves, &grid))) return rc;
    hipLaunchKernelGGL(kern, grid, WAVE * waves, 0, s, (const TensorDesc*)e->dptr, e->count, t0, t1, tb, c);
  }
  rc = launch_check("k_fused_adamw launch");
  if (rc) return rc;
  return record_use(e, s);
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
  int rc = adamw_like_table(list, count, wfmt, ecc_bits, 'A', s, &e);
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
  return record_use(e, s);
}

int fo_fused_sgdm_step(const fo_sgdm_tensor* list, int32_t count, const fo_sgdm_hparams* hp, void* stream) {
  g_err.clear();
  if (!hp) return fail(FO_EINVAL, "hp is NULL");
  if (count < 0) return fail(FO_EINVAL, "count < 0");
  if (count > 0 && !list) return fail(FO_EINVAL, "list is NULL");
  if (!fmt_ok(hp->wfmt, hp->ecc_bits)) return fail(FO_EINVAL, "unsupported format/ECC combination (%d, %d)", hp->wfmt, hp->ecc_bits);
  if (hp->codec != FO_COMPANDED && hp->codec != FO_LINEAR) return fail(FO_EINVAL, "bad codec %d", hp->codec);
  if (hp->step < 1) return fail(FO_EINVAL, "step must be >= 1");
  if (!(hp->lr >= 0.0) || !(hp->momentum >= 0.0) || !(hp->weight_decay >= 0.0))
    return fail(FO_EINVAL, "lr, momentum and weight_decay must be >= 0");
  if (!(hp->dampening >= 0.0 && hp->dampening <= 1.0)) return fail(FO_EINVAL, "dampening must lie in [0, 1]");
  if (hp->nesterov != 0 && hp->nesterov != 1) return fail(FO_EINVAL, "nesterov must be 0 or 1");
  if (hp->nesterov && (hp->momentum <= 0.0 || hp->dampening != 0.0))
    return fail(FO_EINVAL, "Nesterov momentum needs momentum > 0 and dampening 0");
  if (count == 0) return FO_OK;
  hipStream_t s = as_stream(stream);
  std::vector<uint8_t> key(1 + 8 + (size_t)count * sizeof(fo_sgdm_tensor));
  key[0] = 'S';
  std::memcpy(&key[1], &hp->wfmt, 4);
  std::memcpy(&key[5], &hp->ecc_bits, 4);
  std::memcpy(&key[9], list, (size_t)count * sizeof(fo_sgdm_tensor));
  TableEntry* e = nullptr;
  std::lock_guard<std::mutex> lk(g_tab_mu);
  const size_t eb = (size_t)hp->ecc_bits / 8;
  int rc = list_table(key, count, [&](std::vector<std::vector<ArraySpec>>& arrays, std::vector<int64_t>& ns) {
    for (int i = 0; i < count; ++i) {
      const fo_sgdm_tensor& t = list[i];
      ns[i] = t.n;
      arrays[i] = {{t.w16, 2, false, "w16"}, {t.ecc, eb, false, "ecc"}, {t.grad, 2, false, "grad"},
                   {t.b_q, 1, false, "b_q"}, {t.b_s, 2, true, "b_s"}};
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
  c.first = (hp->step == 1) ? 1 : 0;
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
  return record_use(e, s);
}

int fo_selftest(int what, uint32_t lo, uint64_t count, uint64_t* mismatches, void* stream) {
  g_err.clear();
  if (what < 0 || what > 2) return fail(FO_EINVAL, "bad self-test %d", what);
  if (!mismatches) return fail(FO_EINVAL, "mismatches is NULL");
  if (count > (1ull << 32) - lo) return fail(FO_EINVAL, "range exceeds the f32 patterns");
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
