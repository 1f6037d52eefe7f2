// Host block pool: free list, refcounts, per-sequence block tables.
//
// "PagedAttention Internals", sections "Fixed-Size KV Blocks" and "The Block
// Table Map"; "pagedattention" topic page, paragraphs three and four.  The
// placement policy (free-list head on allocation, tail on release, lazy
// allocation when a token lands at a block boundary, copy-on-write for the
// writer of a shared partial block, sharers served in call order) is fixed so
// that two independent implementations agree bit for bit.
#pragma once

#include <cstdint>
#include <vector>

namespace pkv {

struct CowPair {
  int32_t src, dst;
};

class BlockPool {
 public:
  BlockPool(int32_t num_blocks, int32_t block_size, const int32_t* free_order);

  int32_t num_blocks() const { return num_blocks_; }
  int32_t block_size() const { return block_size_; }

  int64_t create();
  // All-or-nothing append; returns a PKV status code.
  int append(const int64_t* seqs, const int32_t* n_new, int32_t n_seqs, int32_t* slots,
             int64_t slot_cap, int32_t* cow, int32_t cow_cap, int32_t* n_cow);
  int fork(int64_t parent, int64_t* child);
  int release(int64_t seq);
  int set_table(int64_t seq, const int32_t* phys, int32_t n, int64_t length);

  bool live(int64_t seq) const {
    return seq >= 0 && seq < (int64_t)seqs_.size() && seqs_[seq].live;
  }
  const std::vector<int32_t>& table(int64_t seq) const { return seqs_[seq].table; }
  int64_t length(int64_t seq) const { return seqs_[seq].length; }
  // bumped whenever an existing table entry is replaced (copy-on-write)
  uint32_t epoch(int64_t seq) const { return seqs_[seq].epoch; }

  int64_t free_count() const { return free_count_; }
  int64_t live_tokens() const { return live_tokens_; }
  int64_t live_seqs() const { return live_seqs_; }
  void export_state(int32_t* free_out, int32_t* ref_out) const;

 private:
  struct Seq {
    bool live = false;
    int64_t length = 0;
    uint32_t epoch = 0;
    std::vector<int32_t> table;
  };

  int32_t pop_free();
  void push_free(int32_t blk);

  int32_t num_blocks_, block_size_;
  // free list: ring buffer, head at free_head_, free_count_ entries
  std::vector<int32_t> ring_;
  int64_t free_head_ = 0, free_count_ = 0;
  std::vector<int32_t> ref_;   // references per block
  std::vector<int32_t> fill_;  // tokens stored per block (0..block_size)
  std::vector<Seq> seqs_;
  int64_t live_tokens_ = 0;    // sum of fill_ over blocks in use
  int64_t live_seqs_ = 0;
};

}  // namespace pkv
