// Slot bookkeeping of the launch-table cache (host code only, no HIP): which
// slot holds which key, least-recently-used choice of the slot to refill,
// pinning, and what a refill must wait for.
//
// A slot is pinned once a HIP graph captures a launch that reads it: the
// graph holds the slot's device address and replays it at any later time, so
// a pinned slot is never chosen for refilling and its contents never change.
// Pins last until the process ends.  When every slot is pinned, victim()
// reports none and the caller fails the call instead of evicting.
#pragma once

#include <cstddef>
#include <cstdint>
#include <string>
#include <unordered_map>
#include <vector>

namespace fo {

// The streams that launched work reading a slot since it was last filled:
// none, exactly one (kept), or several.  Calls record no event per use; a
// refill decides from this what it must wait for (refill_wait).
struct SlotUses {
  const void* stream = nullptr;   // the stream when count == 1
  int count = 0;                  // 0, 1, or 2 for "two or more"
  void add(const void* s) {
    if (count == 0) { stream = s; count = 1; }
    else if (count == 1 && s != stream) count = 2;
  }
  void clear() { stream = nullptr; count = 0; }
};

// What refilling a slot from a call on stream `s` must wait for, besides the
// staging copy of the slot's previous fill (which has an event of its own):
//   NONE    no use since the fill, or every use was on `s` and the slot's
//           device memory is rewritten in place: the new copy is queued on
//           `s` behind them;
//   STREAM  every use was on `s` but the memory is freed and replaced, and
//           freeing is not ordered on any stream: wait for `s`;
//   DEVICE  a use on another stream, or the slot is on another device: no
//           stream orders those uses before the new copy, so wait for the
//           slot's device.
enum class RefillWait { NONE, STREAM, DEVICE };
inline RefillWait refill_wait(const SlotUses& u, const void* s, bool frees, bool same_device) {
  if (u.count == 0) return RefillWait::NONE;
  if (!same_device || u.count > 1 || u.stream != s) return RefillWait::DEVICE;
  return frees ? RefillWait::STREAM : RefillWait::NONE;
}

class SlotCache {
 public:
  explicit SlotCache(size_t slots) : key_(slots), stamp_(slots, 0), pinned_(slots, 0), used_(slots, 0) {}

  size_t size() const { return key_.size(); }

  // Slot holding `key`, or -1.  A hit makes the slot the most recently used.
  long find(const std::string& key) {
    const auto it = index_.find(key);
    if (it == index_.end()) return -1;
    stamp_[it->second] = ++clock_;
    return (long)it->second;
  }

  // The slot to refill: the least recently used slot that is not pinned
  // (empty slots first), or -1 when every slot is pinned.
  long victim() const {
    long v = -1;
    for (size_t i = 0; i < key_.size(); ++i)
      if (!pinned_[i] && (v < 0 || stamp_[i] < stamp_[(size_t)v])) v = (long)i;
    return v;
  }

  // Forget the key of `slot` (the slot becomes empty; its recency stays).
  void drop(long slot) {
    if (used_[(size_t)slot]) index_.erase(key_[(size_t)slot]);
    key_[(size_t)slot].clear();
    used_[(size_t)slot] = 0;
  }

  // `slot` now holds `key` (after drop); it becomes the most recently used.
  void store(long slot, const std::string& key) {
    key_[(size_t)slot] = key;
    used_[(size_t)slot] = 1;
    index_[key] = (size_t)slot;
    stamp_[(size_t)slot] = ++clock_;
  }

  void pin(long slot) { pinned_[(size_t)slot] = 1; }
  size_t pinned_count() const {
    size_t k = 0;
    for (uint8_t p : pinned_) k += p;
    return k;
  }
  bool pinned(long slot) const { return pinned_[(size_t)slot] != 0; }
  bool holds(long slot) const { return used_[(size_t)slot] != 0; }
  const std::string& key(long slot) const { return key_[(size_t)slot]; }

 private:
  std::vector<std::string> key_;
  std::vector<uint64_t> stamp_;
  std::vector<uint8_t> pinned_, used_;
  std::unordered_map<std::string, size_t> index_;
  uint64_t clock_ = 0;
};

}  // namespace fo
