// block_manager.h — host-side physical block manager for the paged pools
// (plain C++; no device code), lock-free.
//
// "PagedAttention: The Cache Was Storing Nothing", §2.2: the cache is cut
// into fixed-size blocks, every request has a block table mapping its
// logical blocks to physical ones, and because every free block has the
// same size any free block will do (no external fragmentation; only a
// request's last block is partly filled).  §2.3: tables may point at the
// same physical blocks (shared prompts, beam search), and a block is copied
// only when a sequence diverges and writes into it.  "Paged Attention Meets
// FlexAttention", "What carries the argument": the page manager hands out
// pages in constant time without locks, from a bump pointer and a free list.
//
// Ids come from a bump pointer (never-used blocks, in id order) and a
// free-list stack (released blocks, most recent first); every block carries
// a reference count: the number of table entries pointing at it.  All of it
// is lock-free, so any number of threads may call into one manager:
//   * the bump pointer is an atomic counter advanced by compare-exchange
//     below num_blocks;
//   * the free list is a Treiber stack: a 64-bit head holding the top id
//     and a tag that every successful exchange increments (so a head read
//     before another thread popped and pushed the same id again cannot be
//     installed: no ABA), with the link of each id in an atomic array;
//   * reference counts are atomic and change by compare-exchange, so a
//     block at zero cannot be shared again and is pushed exactly once;
//   * `avail_` counts the blocks that may still be handed out (stack plus
//     bump range minus reservations).  A caller reserves n blocks by one
//     compare-exchange on it before taking any, so a multi-block request is
//     all or nothing and every reserved take finds a block (blocks only
//     leave the stack and the bump range through reserved takes, and a
//     released block is pushed before it is counted back in).
// Called from one thread, the ids handed out are exactly those of the
// plain model (oracle/block_manager.py).
//
// The manager does not touch device memory: prepare_append returns the
// copy-on-write pairs and the write positions that paged_kv_copy_blocks and
// paged_kv_append then carry out on the pools.
#pragma once

#include <stdint.h>

#include <atomic>
#include <memory>

namespace pa {

// Exponential back-off after a failed compare-exchange on a shared word:
// under contention, retrying at once keeps the cache line bouncing between
// cores and every thread's exchange failing (single-block calls from eight
// threads ran about six times slower in total without it).
struct Backoff {
  int spins = 1;
  void operator()() {
    for (int i = 0; i < spins; ++i) __builtin_ia32_pause();
    if (spins < 64) spins <<= 1;
  }
};

class BlockManager {
 public:
  BlockManager(int32_t num_blocks, int32_t block_size)
      : nb_(num_blocks),
        bs_(block_size),
        ref_(new std::atomic<int32_t>[num_blocks]),
        link_(new std::atomic<int32_t>[num_blocks]),
        avail_(num_blocks) {
    for (int32_t i = 0; i < num_blocks; ++i) {
      ref_[i].store(0, std::memory_order_relaxed);
      link_[i].store(0, std::memory_order_relaxed);
    }
  }
  int32_t num_blocks() const { return nb_; }
  int32_t block_size() const { return bs_; }
  // Blocks that can be handed out now (exact when no call is in flight).
  int32_t num_free() const { return avail_.load(std::memory_order_acquire); }
  int32_t refcount(int32_t id) const {
    return id >= 0 && id < nb_ ? ref_[id].load(std::memory_order_acquire) : -1;
  }

  // Reserve n blocks for later take_reserved() calls; false (nothing
  // reserved) when fewer than n can be handed out.
  bool reserve(int32_t n) {
    int32_t a = avail_.load(std::memory_order_relaxed);
    for (Backoff wait;; wait()) {
      if (a < n) return false;
      if (avail_.compare_exchange_weak(a, a - n, std::memory_order_acq_rel,
                                       std::memory_order_relaxed))
        return true;
    }
  }
  // One fresh block (refcount 1) for a reservation the caller holds: the
  // most recently released block, else the next never-used one.
  int32_t take_reserved() {
    int32_t id = -1;
    take_reserved_n(1, &id);
    return id;
  }
  // n fresh blocks into ids[0..n) for a reservation of n the caller holds:
  // the ids that n take_reserved() calls in a row would give, taken as one
  // chain off the free list and one range of the bump pointer.
  void take_reserved_n(int32_t n, int32_t* ids) {
    int32_t k = 0;
    while (k < n) {
      k += pop_chain(n - k, ids + k);
      if (k < n) k += bump_range(n - k, ids + k);
      // a reserved block is always on the stack or in the bump range: if
      // both looked short, they were seen at two different instants, with a
      // block pushed in between, so look again
    }
    for (int32_t i = 0; i < n; ++i) ref_[ids[i]].store(1, std::memory_order_release);
  }
  // One fresh block, or -1 when none is free.
  int32_t take() { return reserve(1) ? take_reserved() : -1; }

  // Drop one reference of each of ids[0..n) in order; the blocks that reach
  // zero return to the free list as one chain, the last one released on top
  // (as n single drops would leave them).  Returns n, or the index of the
  // first id that is out of range or holds no reference (the ones before it
  // are dropped).
  int32_t drop_n(const int32_t* ids, int32_t n) {
    int32_t top = -1, bottom = -1, freed = 0, i = 0;
    for (; i < n; ++i) {
      const int32_t id = ids[i];
      const int32_t before = dec(id);
      if (before <= 0) break;
      if (before > 1) continue;
      // at zero nobody else can reach the block until it is pushed, so
      // its link is ours to set: it goes above the chain built so far
      link_[id].store(top + 1, std::memory_order_relaxed);
      if (bottom < 0) bottom = id;
      top = id;
      ++freed;
    }
    if (freed) {
      push_chain(top, bottom);
      avail_.fetch_add(freed, std::memory_order_acq_rel);
    }
    return i;
  }
  // Drop one reference; false if the block is out of range or holds none.
  bool drop(int32_t id) { return drop_n(&id, 1) == 1; }
  // Add a reference to a block in use; false if it is free or out of range.
  bool share(int32_t id) {
    if (id < 0 || id >= nb_) return false;
    int32_t r = ref_[id].load(std::memory_order_relaxed);
    do {
      if (r <= 0) return false;
    } while (!ref_[id].compare_exchange_weak(r, r + 1, std::memory_order_acq_rel,
                                             std::memory_order_relaxed));
    return true;
  }

 private:
  static constexpr uint64_t kIdMask = 0xffffffffull;

  // One reference less: the count before, or 0 when the id is out of range
  // or the block is free (nothing changed then).
  int32_t dec(int32_t id) {
    if (id < 0 || id >= nb_) return 0;
    int32_t r = ref_[id].load(std::memory_order_relaxed);
    do {
      if (r <= 0) return 0;
    } while (!ref_[id].compare_exchange_weak(r, r - 1, std::memory_order_acq_rel,
                                             std::memory_order_relaxed));
    return r;
  }

  // Free-list stack: head = (tag << 32) | (top id + 1), 0 in the low half
  // when empty; link_[id] = (id below it) + 1.  Every exchange adds one to
  // the tag.
  static uint64_t next_head(uint64_t h, int32_t top_plus_1) {
    return (((h >> 32) + 1) << 32) | (uint64_t)(uint32_t)top_plus_1;
  }
  // Push the chain top -> ... -> bottom (linked through link_) at once.
  void push_chain(int32_t top, int32_t bottom) {
    uint64_t h = head_.load(std::memory_order_acquire);
    for (Backoff wait;; wait()) {
      link_[bottom].store((int32_t)(h & kIdMask), std::memory_order_relaxed);
      if (head_.compare_exchange_weak(h, next_head(h, top + 1), std::memory_order_release,
                                      std::memory_order_acquire))
        return;
    }
  }
  // Pop up to n ids (top first) into ids; returns how many.  The links are
  // read before the exchange; if it succeeds the head (and its tag) did not
  // change in between, so no block was popped or pushed meanwhile and the
  // links read were those of the stack as it stood.  A link read while the
  // stack changed may be stale, but always names an id in range (or the
  // end), and the exchange then fails.
  int32_t pop_chain(int32_t n, int32_t* ids) {
    uint64_t h = head_.load(std::memory_order_acquire);
    for (Backoff wait;; wait()) {
      int32_t k = 0, x = (int32_t)(h & kIdMask);
      while (k < n && x != 0) {
        ids[k++] = x - 1;
        x = link_[x - 1].load(std::memory_order_relaxed);
      }
      if (k == 0) return 0;
      if (head_.compare_exchange_weak(h, next_head(h, x), std::memory_order_acquire,
                                      std::memory_order_acquire))
        return k;
    }
  }
  // Up to n never-used ids, in id order; returns how many.
  int32_t bump_range(int32_t n, int32_t* ids) {
    int32_t b = next_.load(std::memory_order_relaxed);
    for (Backoff wait;; wait()) {
      const int32_t k = nb_ - b < n ? nb_ - b : n;
      if (k <= 0) return 0;
      if (next_.compare_exchange_weak(b, b + k, std::memory_order_acq_rel,
                                      std::memory_order_relaxed)) {
        for (int32_t i = 0; i < k; ++i) ids[i] = b + i;
        return k;
      }
    }
  }

  int32_t nb_, bs_;
  std::unique_ptr<std::atomic<int32_t>[]> ref_;   // references per block
  std::unique_ptr<std::atomic<int32_t>[]> link_;  // free-list links
  // the three shared words on cache lines of their own
  alignas(64) std::atomic<uint64_t> head_{0};     // free-list top and tag
  alignas(64) std::atomic<int32_t> next_{0};      // bump pointer: [next_, nb_) never used
  alignas(64) std::atomic<int32_t> avail_;        // blocks not yet handed out or reserved
};

}  // namespace pa
