// Region bookkeeping of the pinned host ring through which parameter tables
// reach the device (host code only, no HIP calls, so that it can be checked
// on its own).
//
// A table is written into a region of the ring and read into device memory
// by work enqueued on a stream, which then marks the use complete (an event,
// a completion slot). The region may be written again only once that read
// has run. Regions are handed out in ring order; a
// table that does not fit before the end starts again at offset 0 and leaves
// the tail unused, so a use listed earlier can lie anywhere in the ring: every
// listed use that overlaps a new region is checked, not only the oldest.
#pragma once

#include <cstddef>
#include <deque>
#include <vector>

namespace lmlp {

template <class Ev>
class StageRing {
 public:
  explicit StageRing(size_t capacity) : cap_(capacity) {}

  size_t capacity() const { return cap_; }
  size_t in_flight() const { return uses_.size(); }

  // Offers the region for a table of `len` bytes (0 < len <= capacity).
  // `done(ev)` tells whether the copy behind `ev` has run: 1 yes, 0 not yet,
  // below 0 an error. Returns 1 with `off` set when every listed use that
  // overlaps the region has run (those uses are then dropped and their events
  // kept for reuse), 0 when one has not (nothing changes), or the error.
  template <class Done>
  int acquire(size_t len, size_t& off, Done&& done) {
    if (len == 0 || len > cap_) return 0;
    const size_t at = head_ + len > cap_ ? 0 : head_;
    for (const Use& u : uses_) {
      if (!overlaps(u, at, len)) continue;
      const int d = done(u.ev);
      if (d <= 0) return d;
    }
    for (auto it = uses_.begin(); it != uses_.end();) {
      if (overlaps(*it, at, len)) {
        spare_.push_back(it->ev);
        it = uses_.erase(it);
      } else {
        ++it;
      }
    }
    off = at;
    return 1;
  }

  // Lists the copy enqueued from [off, off + len) behind `ev`; the next
  // region starts after it.
  void commit(size_t off, size_t len, Ev ev) {
    uses_.push_back({off, len, ev});
    head_ = off + len;
  }

  // An event of a use that has run, for the next copy; false when none.
  bool take_spare(Ev& ev) {
    if (spare_.empty()) return false;
    ev = spare_.back();
    spare_.pop_back();
    return true;
  }

 private:
  struct Use {
    size_t off, len;
    Ev ev;
  };
  static bool overlaps(const Use& u, size_t at, size_t len) { return u.off < at + len && at < u.off + u.len; }

  size_t cap_;
  size_t head_ = 0;
  std::deque<Use> uses_;
  std::vector<Ev> spare_;
};

}  // namespace lmlp
