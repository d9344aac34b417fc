// CPU check of the launch-table cache's slot bookkeeping (fo_slots.hpp):
// least-recently-used refill, pinned slots (read by captured HIP graphs)
// never refilled, the per-slot record of the streams that read a slot, and
// what a refill waits for.  Prints "ok" or the first failed condition and exits 1.
#include <cstdio>
#include <cstdlib>
#include <string>

#include "../../precision_optimizer_state_amd/csrc/fo_slots.hpp"

#define CHECK(c)                                              \
  do {                                                        \
    if (!(c)) {                                               \
      std::printf("failed at line %d: %s\n", __LINE__, #c);  \
      return 1;                                               \
    }                                                         \
  } while (0)

// One cache operation as the library performs it: a hit, or a refill of the
// victim slot.  Returns the slot, or -1 when every slot is pinned.
static long use(fo::SlotCache& c, const std::string& key) {
  long s = c.find(key);
  if (s >= 0) return s;
  s = c.victim();
  if (s < 0) return -1;
  c.drop(s);
  c.store(s, key);
  return s;
}

int main() {
  // plain LRU: empty slots fill first, then the least recently used goes
  {
    fo::SlotCache c(3);
    const long a = use(c, "a"), b = use(c, "b"), d = use(c, "c");
    CHECK(a != b && b != d && a != d);
    CHECK(use(c, "a") == a);                 // hit refreshes "a": "b" is now the oldest
    CHECK(use(c, "x") == b);
    CHECK(c.find("b") < 0 && c.find("x") == b && c.find("a") == a);
  }
  // a pinned slot is skipped by refills however old it is, and keeps its key
  {
    fo::SlotCache c(3);
    const long a = use(c, "a");
    c.pin(a);
    for (int i = 0; i < 100; ++i) {
      const long s = use(c, "k" + std::to_string(i));
      CHECK(s >= 0 && s != a);
      CHECK(c.holds(a) && c.pinned(a) && c.key(a) == "a");   // (find would refresh "a")
    }
    CHECK(use(c, "a") == a);                 // still a hit
  }
  // every slot pinned: no victim; hits still served
  {
    fo::SlotCache c(4);
    long s[4];
    for (int i = 0; i < 4; ++i) { s[i] = use(c, "p" + std::to_string(i)); c.pin(s[i]); }
    CHECK(c.victim() < 0 && c.pinned_count() == 4);
    CHECK(use(c, "new") < 0);
    for (int i = 0; i < 4; ++i) CHECK(use(c, "p" + std::to_string(i)) == s[i]);
  }
  // the cache's own size with capture-style pinning of every other list:
  // pinned lists survive any number of later refills
  {
    const size_t n = 1024;
    fo::SlotCache c(n);
    for (int i = 0; i < 512; ++i) c.pin(use(c, "g" + std::to_string(i)));
    for (int i = 0; i < 20000; ++i) CHECK(use(c, "e" + std::to_string(i)) >= 0);
    for (int i = 0; i < 512; ++i) {
      const long s = c.find("g" + std::to_string(i));
      CHECK(s >= 0 && c.pinned(s));
    }
    // the unpinned half keeps only the most recent 512 eager lists
    for (int i = 20000 - 512; i < 20000; ++i) CHECK(c.find("e" + std::to_string(i)) >= 0);
    CHECK(c.find("e" + std::to_string(20000 - 513)) < 0);
  }
  // drop leaves a slot empty and refillable; an empty slot is not a hit
  {
    fo::SlotCache c(2);
    const long a = use(c, "a");
    c.drop(a);
    CHECK(!c.holds(a) && c.find("a") < 0);
    CHECK(use(c, "b") >= 0);
  }
  // per-slot use tracking: none, one stream, or several
  {
    int A, B;                                 // two distinct stream handles
    fo::SlotUses u;
    CHECK(u.count == 0);
    u.add(&A);
    CHECK(u.count == 1 && u.stream == &A);
    u.add(&A);
    CHECK(u.count == 1 && u.stream == &A);   // the same stream again
    u.add(&B);
    CHECK(u.count == 2);
    u.add(&A);
    CHECK(u.count == 2);                      // several stays several
    u.clear();
    CHECK(u.count == 0 && u.stream == nullptr);
    u.add(nullptr);                           // the null stream is a stream like any other
    CHECK(u.count == 1 && u.stream == nullptr);
    u.add(&A);
    CHECK(u.count == 2);
  }
  // what a refill on stream S waits for
  {
    using fo::RefillWait;
    int S, T;
    fo::SlotUses none, onS, onT, both;
    onS.add(&S);
    onT.add(&T);
    both.add(&S);
    both.add(&T);
    for (bool frees : {false, true})
      for (bool same_dev : {false, true}) CHECK(fo::refill_wait(none, &S, frees, same_dev) == RefillWait::NONE);
    CHECK(fo::refill_wait(onS, &S, false, true) == RefillWait::NONE);     // queued behind them on S
    CHECK(fo::refill_wait(onS, &S, true, true) == RefillWait::STREAM);    // freeing is not stream-ordered
    CHECK(fo::refill_wait(onT, &S, false, true) == RefillWait::DEVICE);   // nothing orders T before S
    CHECK(fo::refill_wait(onT, &S, true, true) == RefillWait::DEVICE);
    CHECK(fo::refill_wait(both, &S, false, true) == RefillWait::DEVICE);  // uses on S and T
    CHECK(fo::refill_wait(both, &S, true, true) == RefillWait::DEVICE);
    CHECK(fo::refill_wait(onS, &S, false, false) == RefillWait::DEVICE);  // the slot's device is another
    CHECK(fo::refill_wait(onS, &S, true, false) == RefillWait::DEVICE);
  }
  std::printf("ok\n");
  return 0;
}
