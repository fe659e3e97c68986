// block_manager.h — host-side physical block manager for the paged pools
// (plain C++; no device code).
//
// "PagedAttention: The Cache Was Storing Nothing", §2.2: the cache is cut
// into fixed-size blocks, every request has a block table mapping its
// logical blocks to physical ones, and because every free block has the
// same size any free block will do (no external fragmentation; only a
// request's last block is partly filled).  §2.3: tables may point at the
// same physical blocks (shared prompts, beam search), and a block is copied
// only when a sequence diverges and writes into it.
//
// Ids come from a bump pointer (never-used blocks, in id order) and a LIFO
// free list (released blocks, most recent first); both O(1).  Every block
// carries a reference count: the number of table entries pointing at it.
// The manager does not touch device memory: prepare_append returns the
// copy-on-write pairs and the write positions that paged_kv_copy_blocks and
// paged_kv_append then carry out on the pools.
//
// Not thread-safe: calls on one manager must be serialised by the caller
// (a serving loop's scheduler thread).
#pragma once

#include <stdint.h>

#include <vector>

namespace pa {

class BlockManager {
 public:
  BlockManager(int32_t num_blocks, int32_t block_size)
      : nb_(num_blocks), bs_(block_size), ref_(num_blocks, 0) {
    free_.reserve(num_blocks);
  }
  int32_t num_blocks() const { return nb_; }
  int32_t block_size() const { return bs_; }
  int32_t num_free() const { return nb_ - next_ + (int32_t)free_.size(); }
  int32_t refcount(int32_t id) const { return id >= 0 && id < nb_ ? ref_[id] : -1; }

  // One fresh block (refcount 1), or -1 when none is free.
  int32_t take() {
    int32_t id;
    if (!free_.empty()) {
      id = free_.back();
      free_.pop_back();
    } else if (next_ < nb_) {
      id = next_++;
    } else {
      return -1;
    }
    ref_[id] = 1;
    return id;
  }
  // Drop one reference; the block returns to the free list at zero.
  // false if the block is out of range or holds no reference.
  bool drop(int32_t id) {
    if (id < 0 || id >= nb_ || ref_[id] <= 0) return false;
    if (--ref_[id] == 0) free_.push_back(id);
    return true;
  }
  // Add a reference to a block in use; false if it is free or out of range.
  bool share(int32_t id) {
    if (id < 0 || id >= nb_ || ref_[id] <= 0) return false;
    ++ref_[id];
    return true;
  }

 private:
  int32_t nb_, bs_;
  int32_t next_ = 0;           // bump pointer: blocks [next_, nb_) never used
  std::vector<int32_t> ref_;   // references per block
  std::vector<int32_t> free_;  // released blocks, LIFO
};

}  // namespace pa
