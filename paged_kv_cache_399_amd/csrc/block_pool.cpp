#include "block_pool.hpp"

#include <algorithm>
#include <climits>
#include <stdexcept>
#include <unordered_map>

#include "internal.hpp"

namespace pkv {

namespace {
// floor(a / b) for b > 0 and any sign of a
inline int64_t floor_div(int64_t a, int64_t b) { return a >= 0 ? a / b : -((-a + b - 1) / b); }
}  // namespace

BlockPool::BlockPool(int32_t num_blocks, int32_t block_size, const int32_t* free_order)
    : num_blocks_(num_blocks), block_size_(block_size) {
  ring_.resize(num_blocks);
  ref_.assign(num_blocks, 0);
  fill_.assign(num_blocks, 0);
  for (int32_t i = 0; i < num_blocks; ++i) ring_[i] = free_order ? free_order[i] : i;
  free_head_ = 0;
  free_count_ = num_blocks;
}

int32_t BlockPool::pop_free() {
  int32_t blk = ring_[free_head_];
  free_head_ = (free_head_ + 1) % num_blocks_;
  --free_count_;
  return blk;
}

void BlockPool::push_free(int32_t blk) {
  ring_[(free_head_ + free_count_) % num_blocks_] = blk;
  ++free_count_;
}

int64_t BlockPool::create() {
  seqs_.emplace_back();
  seqs_.back().live = true;
  ++live_seqs_;
  return (int64_t)seqs_.size() - 1;
}

int BlockPool::append(const int64_t* seqs, const int32_t* n_new, int32_t n_seqs, int32_t* slots,
                      int64_t slot_cap, int32_t* cow, int32_t cow_cap, int32_t* n_cow) {
  if (n_seqs < 0) return fail(PKV_ERR_INVALID_ARG, "n_seqs < 0");
  if (n_seqs > 0 && (!seqs || !n_new)) return fail(PKV_ERR_INVALID_ARG, "NULL seqs / n_new");
  const int64_t P = block_size_;
  int64_t total = 0;
  for (int32_t i = 0; i < n_seqs; ++i) {
    if (!live(seqs[i])) return fail(PKV_ERR_BAD_SEQ, "sequence %lld is not live", (long long)seqs[i]);
    if (n_new[i] < 0) return fail(PKV_ERR_INVALID_ARG, "negative token count for entry %d", i);
    total += n_new[i];
  }
  {
    std::vector<int64_t> ids(seqs, seqs + n_seqs);
    std::sort(ids.begin(), ids.end());
    if (std::adjacent_find(ids.begin(), ids.end()) != ids.end())
      return fail(PKV_ERR_INVALID_ARG, "a sequence appears twice in one call");
  }
  if (total > slot_cap) return fail(PKV_ERR_CAPACITY, "%lld slots do not fit slot_cap %lld",
                                    (long long)total, (long long)slot_cap);
  if (total > 0 && !slots) return fail(PKV_ERR_INVALID_ARG, "NULL slot_mapping_out");

  // Dry run: blocks and copies the call needs, with the copy-on-write
  // reference drops of earlier sharers in this same call taken into account.
  int64_t need = 0, ncow = 0;
  std::unordered_map<int32_t, int32_t> dropped;
  for (int32_t i = 0; i < n_seqs; ++i) {
    const Seq& s = seqs_[seqs[i]];
    const int64_t n = n_new[i];
    if (n == 0) continue;
    const int64_t L = s.length;
    if (L % P != 0) {
      const int32_t last = s.table.back();
      int32_t& d = dropped[last];
      if (ref_[last] - d > 1) {
        ++need;
        ++ncow;
        ++d;
      }
    }
    // positions L .. L+n-1 that start a block
    need += floor_div(L + n - 1, P) - floor_div(L - 1, P);
  }
  if (need > free_count_)
    return fail(PKV_ERR_NO_BLOCKS, "call needs %lld blocks, %lld free", (long long)need,
                (long long)free_count_);
  if (ncow > cow_cap)
    return fail(PKV_ERR_CAPACITY, "%lld copy-on-write pairs do not fit cow_cap %d",
                (long long)ncow, cow_cap);
  if (ncow > 0 && !cow) return fail(PKV_ERR_INVALID_ARG, "NULL cow_pairs_out");

  int64_t k = 0;
  int32_t c = 0;
  for (int32_t i = 0; i < n_seqs; ++i) {
    Seq& s = seqs_[seqs[i]];
    const int32_t n = n_new[i];
    for (int32_t j = 0; j < n; ++j) {
      const int64_t L = s.length;
      const int32_t off = (int32_t)(L % P);
      if (off == 0) {
        const int32_t blk = pop_free();
        ref_[blk] = 1;
        fill_[blk] = 0;
        s.table.push_back(blk);
      } else if (ref_[s.table.back()] > 1) {
        const int32_t src = s.table.back();
        const int32_t dst = pop_free();
        --ref_[src];
        ref_[dst] = 1;
        fill_[dst] = fill_[src];
        live_tokens_ += fill_[src];
        cow[2 * c] = src;
        cow[2 * c + 1] = dst;
        ++c;
        s.table.back() = dst;
        ++s.epoch;
      }
      const int32_t blk = s.table[L / P];
      slots[k++] = blk * (int32_t)P + off;
      ++fill_[blk];
      ++live_tokens_;
      s.length = L + 1;
    }
  }
  if (n_cow) *n_cow = c;
  return PKV_OK;
}

int BlockPool::fork(int64_t parent, int64_t* child) {
  if (!live(parent)) return fail(PKV_ERR_BAD_SEQ, "sequence %lld is not live", (long long)parent);
  const int64_t id = create();
  Seq& c = seqs_[id];
  const Seq& p = seqs_[parent];
  c.table = p.table;
  c.length = p.length;
  for (int32_t blk : c.table) ++ref_[blk];
  *child = id;
  return PKV_OK;
}

int BlockPool::release(int64_t seq) {
  if (!live(seq)) return fail(PKV_ERR_BAD_SEQ, "sequence %lld is not live", (long long)seq);
  Seq& s = seqs_[seq];
  for (int32_t blk : s.table) {
    if (--ref_[blk] == 0) {
      live_tokens_ -= fill_[blk];
      fill_[blk] = 0;
      push_free(blk);
    }
  }
  std::vector<int32_t>().swap(s.table);
  s.live = false;
  s.length = 0;
  --live_seqs_;
  return PKV_OK;
}

int BlockPool::set_table(int64_t seq, const int32_t* phys, int32_t n, int64_t length) {
  if (!live(seq)) return fail(PKV_ERR_BAD_SEQ, "sequence %lld is not live", (long long)seq);
  Seq& s = seqs_[seq];
  if (!s.table.empty() || s.length != 0) return fail(PKV_ERR_INVALID_ARG, "set_table needs an empty sequence");
  if (n < 0 || (n > 0 && !phys)) return fail(PKV_ERR_INVALID_ARG, "bad block list");
  if (length < 0 || ceil_div(length, block_size_) != n)
    return fail(PKV_ERR_INVALID_ARG, "length %lld does not match %d blocks", (long long)length, n);
  std::vector<char> seen(num_blocks_, 0);
  for (int32_t j = 0; j < n; ++j) {
    const int32_t blk = phys[j];
    if (blk < 0 || blk >= num_blocks_ || ref_[blk] != 0 || seen[blk])
      return fail(PKV_ERR_INVALID_ARG, "block %d is not a distinct free block", blk);
    seen[blk] = 1;
  }
  // drop the chosen blocks from the free list, keeping the others' order
  std::vector<int32_t> rest;
  rest.reserve(free_count_);
  for (int64_t i = 0; i < free_count_; ++i) {
    const int32_t blk = ring_[(free_head_ + i) % num_blocks_];
    if (!seen[blk]) rest.push_back(blk);
  }
  free_head_ = 0;
  free_count_ = (int64_t)rest.size();
  std::copy(rest.begin(), rest.end(), ring_.begin());
  s.table.assign(phys, phys + n);
  for (int32_t j = 0; j < n; ++j) {
    ref_[phys[j]] = 1;
    fill_[phys[j]] = (int32_t)std::min<int64_t>(block_size_, length - (int64_t)j * block_size_);
  }
  s.length = length;
  live_tokens_ += length;
  return PKV_OK;
}

void BlockPool::export_state(int32_t* free_out, int32_t* ref_out) const {
  if (free_out)
    for (int64_t i = 0; i < free_count_; ++i) free_out[i] = ring_[(free_head_ + i) % num_blocks_];
  if (ref_out) std::copy(ref_.begin(), ref_.end(), ref_out);
}

}  // namespace pkv
