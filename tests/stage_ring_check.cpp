// Host-only check of the staging ring's region bookkeeping (stage_ring.h):
// a simulated stream runs the enqueued table copies in order, a random number
// at a time, while the host keeps writing tables into the ring. Each region is
// filled with its table's tag when written; when the simulated copy runs, the
// region must still hold that tag. A region written over before its copy ran
// is the fault this bookkeeping exists to prevent.
//
// usage: stage_ring_check MODE SEED ITERS
//   MODE ring       the library's StageRing (expected: exit 0)
//   MODE frontonly  checks only the oldest listed use, as a ring that assumed
//                   its uses overlap new regions in list order (expected: exit 3)
//   MODE nocheck    writes without checking (expected: exit 3)
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <deque>
#include <random>
#include <string>
#include <type_traits>
#include <vector>

#include "stage_ring.h"

namespace {

struct Copy {
  size_t off, len;
  uint32_t tag;
  int ev;
  uint64_t seq;
};

// the bookkeeping that checks only the front of its list
struct FrontOnly {
  struct Use {
    size_t off, len;
    int ev;
  };
  size_t cap, head = 0;
  std::deque<Use> uses;
  explicit FrontOnly(size_t c) : cap(c) {}
  template <class Done>
  int acquire(size_t len, size_t& off, Done&& done) {
    if (head + len > cap) head = 0;
    while (!uses.empty()) {
      const Use& u = uses.front();
      if (!(u.off < head + len && head < u.off + u.len)) break;
      const int d = done(u.ev);
      if (d <= 0) return d;
      uses.pop_front();
    }
    off = head;
    return 1;
  }
  void commit(size_t off, size_t len, int ev) {
    uses.push_back({off, len, ev});
    head = off + len;
  }
};

struct NoCheck {
  size_t cap, head = 0;
  explicit NoCheck(size_t c) : cap(c) {}
  template <class Done>
  int acquire(size_t len, size_t& off, Done&&) {
    if (head + len > cap) head = 0;
    off = head;
    return 1;
  }
  void commit(size_t off, size_t len, int) { head = off + len; }
};

template <class Ring>
int run(Ring& ring, bool real, uint64_t seed, long iters) {
  const size_t cap = 64 * 1024;
  std::mt19937_64 rng(seed);
  std::vector<uint32_t> mem(cap / 4, 0);
  std::deque<Copy> stream;           // enqueued, not yet run
  std::vector<uint64_t> event_seq;   // copy sequence number each event was last recorded behind
  uint64_t next_seq = 0, ran = 0;    // copies enqueued / run so far
  long staged = 0, fallback = 0;
  uint32_t tag = 1;
  auto done = [&](int ev) { return event_seq[ev] < ran ? 1 : 0; };
  auto run_copies = [&](long n) -> bool {
    for (; n > 0 && !stream.empty(); --n) {
      const Copy c = stream.front();
      stream.pop_front();
      for (size_t i = c.off / 4; i < (c.off + c.len) / 4; ++i) {
        if (mem[i] != c.tag) {
          std::printf("copy %llu of [%zu, %zu) found its region written over\n",
                      static_cast<unsigned long long>(c.seq), c.off, c.off + c.len);
          return false;
        }
      }
      ++ran;
    }
    return true;
  };
  for (long it = 0; it < iters; ++it) {
    // table sizes: mostly small, some up to a third of the ring (tails get skipped)
    const int kind = static_cast<int>(rng() % 8);
    const size_t len = 256 * (kind < 5 ? 1 + rng() % 8 : 1 + rng() % (cap / 3 / 256));
    size_t off = 0;
    const int got = ring.acquire(len, off, done);
    if (got < 0) {
      std::printf("acquire failed\n");
      return 2;
    }
    if (got == 1) {
      if (off + len > cap) {
        std::printf("region [%zu, %zu) past the ring\n", off, off + len);
        return 2;
      }
      for (size_t i = off / 4; i < (off + len) / 4; ++i) mem[i] = tag;
      int ev = -1;
      if constexpr (std::is_same_v<Ring, lmlp::StageRing<int>>) {
        if (!ring.take_spare(ev)) {
          ev = static_cast<int>(event_seq.size());
          event_seq.push_back(0);
        }
      } else {
        ev = static_cast<int>(event_seq.size());
        event_seq.push_back(0);
      }
      event_seq[ev] = next_seq;
      stream.push_back({off, len, tag, ev, next_seq});
      ring.commit(off, len, ev);
      ++next_seq;
      ++tag;
      ++staged;
    } else {
      ++fallback;  // the copy kernels would write this table
    }
    // the stream runs 0..3 copies, now and then all of them
    const long n = (rng() % 64 == 0) ? static_cast<long>(stream.size()) : static_cast<long>(rng() % 4);
    if (!run_copies(n)) return 3;
    if constexpr (std::is_same_v<Ring, lmlp::StageRing<int>>) {
      if (real && ring.in_flight() > cap / 256) {
        std::printf("%zu uses listed for a ring of %zu regions\n", ring.in_flight(), cap / 256);
        return 2;
      }
      if (stream.empty()) {  // with nothing in flight every table must be taken
        size_t o2 = 0;
        const size_t l2 = 256 * (1 + rng() % (cap / 256));
        if (ring.acquire(l2, o2, done) != 1) {
          std::printf("idle ring refused %zu bytes\n", l2);
          return 2;
        }
      }
    }
  }
  if (!run_copies(static_cast<long>(stream.size()))) return 3;
  std::printf("ok staged %ld fallback %ld\n", staged, fallback);
  return 0;
}

}  // namespace

int main(int argc, char** argv) {
  if (argc != 4) return 64;
  const std::string mode = argv[1];
  const uint64_t seed = std::strtoull(argv[2], nullptr, 10);
  const long iters = std::strtol(argv[3], nullptr, 10);
  const size_t cap = 64 * 1024;
  if (mode == "ring") {
    lmlp::StageRing<int> r(cap);
    return run(r, true, seed, iters);
  }
  if (mode == "frontonly") {
    FrontOnly r(cap);
    return run(r, false, seed, iters);
  }
  if (mode == "nocheck") {
    NoCheck r(cap);
    return run(r, false, seed, iters);
  }
  return 64;
}
