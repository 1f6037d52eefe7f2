// C ABI of the host block pool and of the block-table upload.
#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <climits>
#include <cstddef>
#include <cstdio>
#include <cstring>
#include <new>
#include <string>
#include <unordered_map>
#include <vector>

#include "block_pool.hpp"
#include "internal.hpp"

namespace pkv {

namespace {
thread_local std::string g_last_error;
}

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

}  // namespace pkv

// Pool handle: the host pool plus two pinned staging buffers for uploads.
struct pkv_pool {
  struct Stage {
    void* host = nullptr;
    size_t bytes = 0;
    hipEvent_t done = nullptr;  // recorded after the copies that read `host`
    bool pending = false;
  };
  // What the last upload wrote into one row of a device table.
  struct RowRecord {
    int64_t seq = -1;
    int32_t blocks = 0;   // entries [0, blocks) hold the sequence's table
    uint32_t epoch = 0;   // the sequence's copy-on-write epoch at that time
  };
  struct TableRecord {
    int32_t max_blocks = 0;
    std::vector<RowRecord> rows;
    const int32_t* shared_dev = nullptr;  // shared-token array written with this table
    std::vector<int32_t> shared_sent;     // what it holds
  };
  pkv::BlockPool pool;
  Stage stage[2];
  int next = 0;
  std::unordered_map<const void*, TableRecord> tables;  // keyed by device table address
  std::vector<int32_t> build;  // cacheable host buffer for full tables

  pkv_pool(int32_t nb, int32_t p, const int32_t* order) : pool(nb, p, order) {}
  ~pkv_pool() {
    for (Stage& s : stage) {
      if (s.pending) (void)hipEventSynchronize(s.done);
      if (s.done) (void)hipEventDestroy(s.done);
      if (s.host) (void)hipHostFree(s.host);
    }
  }
};

using pkv::fail;

extern "C" {

const char* pkv_last_error(void) { return pkv::g_last_error.c_str(); }

const char* pkv_version(void) { return "pkv 0.1 gfx950"; }

int pkv_pool_create(int32_t num_blocks, int32_t block_size, const int32_t* free_order,
                    pkv_pool** out) {
  PKV_TRY_BEGIN
  if (!out) return fail(PKV_ERR_INVALID_ARG, "out is NULL");
  if (num_blocks <= 0 || block_size <= 0)
    return fail(PKV_ERR_INVALID_ARG, "num_blocks and block_size must be positive");
  if ((int64_t)num_blocks * block_size > INT32_MAX)
    return fail(PKV_ERR_INVALID_ARG, "num_blocks * block_size exceeds int32 slot range");
  if (free_order) {
    std::vector<char> seen(num_blocks, 0);
    for (int32_t i = 0; i < num_blocks; ++i) {
      const int32_t b = free_order[i];
      if (b < 0 || b >= num_blocks || seen[b])
        return fail(PKV_ERR_INVALID_ARG, "free_order is not a permutation of 0..num_blocks-1");
      seen[b] = 1;
    }
  }
  *out = new pkv_pool(num_blocks, block_size, free_order);
  return PKV_OK;
  PKV_TRY_END
}

int pkv_pool_destroy(pkv_pool* pool) {
  PKV_TRY_BEGIN
  delete pool;
  return PKV_OK;
  PKV_TRY_END
}

int pkv_seq_create(pkv_pool* pool, int64_t* seq_out) {
  PKV_TRY_BEGIN
  if (!pool || !seq_out) return fail(PKV_ERR_INVALID_ARG, "NULL argument");
  *seq_out = pool->pool.create();
  return PKV_OK;
  PKV_TRY_END
}

int pkv_seq_append_slots(pkv_pool* pool, const int64_t* seqs, const int32_t* n_new,
                         int32_t n_seqs, int32_t* slot_mapping_out, int64_t slot_cap,
                         int32_t* cow_pairs_out, int32_t cow_cap, int32_t* n_cow_out) {
  PKV_TRY_BEGIN
  if (!pool) return fail(PKV_ERR_INVALID_ARG, "NULL pool");
  if (cow_cap < 0) return fail(PKV_ERR_INVALID_ARG, "cow_cap < 0");
  return pool->pool.append(seqs, n_new, n_seqs, slot_mapping_out, slot_cap, cow_pairs_out,
                           cow_cap, n_cow_out);
  PKV_TRY_END
}

int pkv_seq_fork(pkv_pool* pool, int64_t parent, int64_t* child_out) {
  PKV_TRY_BEGIN
  if (!pool || !child_out) return fail(PKV_ERR_INVALID_ARG, "NULL argument");
  return pool->pool.fork(parent, child_out);
  PKV_TRY_END
}

int pkv_seq_free(pkv_pool* pool, int64_t seq) {
  PKV_TRY_BEGIN
  if (!pool) return fail(PKV_ERR_INVALID_ARG, "NULL pool");
  return pool->pool.release(seq);
  PKV_TRY_END
}

int pkv_seq_set_table(pkv_pool* pool, int64_t seq, const int32_t* phys, int32_t n_blocks,
                      int64_t length) {
  PKV_TRY_BEGIN
  if (!pool) return fail(PKV_ERR_INVALID_ARG, "NULL pool");
  return pool->pool.set_table(seq, phys, n_blocks, length);
  PKV_TRY_END
}

int pkv_seq_get_table(pkv_pool* pool, int64_t seq, int32_t* phys_out, int32_t cap,
                      int32_t* n_out, int64_t* len_out) {
  PKV_TRY_BEGIN
  if (!pool) return fail(PKV_ERR_INVALID_ARG, "NULL pool");
  if (!pool->pool.live(seq)) return fail(PKV_ERR_BAD_SEQ, "sequence %lld is not live", (long long)seq);
  const std::vector<int32_t>& t = pool->pool.table(seq);
  if ((int64_t)t.size() > cap)
    return fail(PKV_ERR_CAPACITY, "table of %zu blocks does not fit cap %d", t.size(), cap);
  if (!t.empty() && !phys_out) return fail(PKV_ERR_INVALID_ARG, "NULL phys_out");
  std::copy(t.begin(), t.end(), phys_out);
  if (n_out) *n_out = (int32_t)t.size();
  if (len_out) *len_out = pool->pool.length(seq);
  return PKV_OK;
  PKV_TRY_END
}

int pkv_pool_stats(pkv_pool* pool, pkv_stats* out) {
  PKV_TRY_BEGIN
  if (!pool || !out) return fail(PKV_ERR_INVALID_ARG, "NULL argument");
  const pkv::BlockPool& p = pool->pool;
  out->num_blocks = p.num_blocks();
  out->free_blocks = p.free_count();
  out->used_blocks = p.num_blocks() - p.free_count();
  out->allocated_slots = out->used_blocks * p.block_size();
  out->live_tokens = p.live_tokens();
  out->wasted_slots = out->allocated_slots - out->live_tokens;
  out->num_seqs = p.live_seqs();
  out->fragmentation =
      out->allocated_slots ? (double)out->wasted_slots / (double)out->allocated_slots : 0.0;
  return PKV_OK;
  PKV_TRY_END
}

int pkv_pool_export(pkv_pool* pool, int32_t* free_order_out, int32_t* refcount_out,
                    int32_t* n_free_out) {
  PKV_TRY_BEGIN
  if (!pool) return fail(PKV_ERR_INVALID_ARG, "NULL pool");
  pool->pool.export_state(free_order_out, refcount_out);
  if (n_free_out) *n_free_out = (int32_t)pool->pool.free_count();
  return PKV_OK;
  PKV_TRY_END
}

}  // extern "C"

namespace {

// Tokens sequence b holds in the same physical blocks as sequence a: the
// leading table entries they have in common, limited to both lengths (equal
// block ids mean the same slots, so those tokens are the same bytes).
int32_t shared_tokens(const pkv::BlockPool& bp, int64_t a, int64_t b) {
  const std::vector<int32_t>& ta = bp.table(a);
  const std::vector<int32_t>& tb = bp.table(b);
  const size_t n = std::min(ta.size(), tb.size());
  const size_t k = (size_t)(std::mismatch(ta.begin(), ta.begin() + n, tb.begin()).first - ta.begin());
  return (int32_t)std::min<int64_t>({(int64_t)k * bp.block_size(), bp.length(a), bp.length(b)});
}

}  // namespace

extern "C" {

int pkv_seq_shared_prefix(pkv_pool* pool, const int64_t* seqs, int32_t n_seqs, int32_t* shared_out,
                          int64_t* unshared_tokens_out) {
  PKV_TRY_BEGIN
  if (!pool) return fail(PKV_ERR_INVALID_ARG, "NULL pool");
  if (n_seqs < 0) return fail(PKV_ERR_INVALID_ARG, "negative size");
  if (n_seqs > 0 && !seqs) return fail(PKV_ERR_INVALID_ARG, "NULL sequence list");
  const pkv::BlockPool& bp = pool->pool;
  for (int32_t i = 0; i < n_seqs; ++i)
    if (!bp.live(seqs[i])) return fail(PKV_ERR_BAD_SEQ, "sequence %lld is not live", (long long)seqs[i]);
  int64_t unshared = 0;
  for (int32_t i = 0; i < n_seqs; ++i) {
    const int32_t sh = i ? shared_tokens(bp, seqs[i - 1], seqs[i]) : 0;
    if (shared_out) shared_out[i] = sh;
    unshared += bp.length(seqs[i]) - sh;
  }
  if (unshared_tokens_out) *unshared_tokens_out = unshared;
  return PKV_OK;
  PKV_TRY_END
}

}  // extern "C"

namespace {

// Full upload: the padded table, the lengths, the shared-token counts and the
// slot mapping through one pinned staging round (double-buffered, reused after
// its copies finished).
int upload_full(pkv_pool* pool, const int64_t* seqs, int32_t n_seqs, int32_t max_blocks,
                int32_t* d_table, int32_t* d_lens, int32_t* d_shared, const int32_t* shared,
                const int32_t* slot_mapping, int32_t* d_slots, int32_t n_slots, hipStream_t st) {
  const pkv::BlockPool& bp = pool->pool;
  const size_t table_words = (size_t)n_seqs * max_blocks;
  const size_t n_sh = d_shared ? (size_t)n_seqs : 0;
  const size_t need = (table_words + n_seqs + n_sh + n_slots) * sizeof(int32_t);
  if (need == 0) return PKV_OK;
  pkv_pool::Stage& sg = pool->stage[pool->next];
  if (sg.pending) {
    if (hipEventSynchronize(sg.done) != hipSuccess)
      return fail(PKV_ERR_HIP, "waiting for a previous upload failed");
    sg.pending = false;
  }
  if (sg.bytes < need) {
    if (sg.host) (void)hipHostFree(sg.host);
    sg.host = nullptr;
    sg.bytes = 0;
    const size_t cap = std::max<size_t>(need, 4096);
    if (hipHostMalloc(&sg.host, cap, hipHostMallocDefault) != hipSuccess)
      return fail(PKV_ERR_HIP, "pinned staging allocation of %zu bytes failed", cap);
    sg.bytes = cap;
  }
  if (!sg.done && hipEventCreateWithFlags(&sg.done, hipEventDisableTiming) != hipSuccess)
    return fail(PKV_ERR_HIP, "event creation failed");
  // rows are assembled in ordinary cached memory, then moved to pinned memory
  // in one bulk copy (word-by-word writes to pinned memory are slow)
  std::vector<int32_t>& b = pool->build;
  b.resize(table_words + n_seqs);
  for (int32_t i = 0; i < n_seqs; ++i) {
    const std::vector<int32_t>& t = bp.table(seqs[i]);
    int32_t* row = b.data() + (size_t)i * max_blocks;
    std::copy(t.begin(), t.end(), row);
    std::fill(row + t.size(), row + max_blocks, -1);
    b[table_words + i] = (int32_t)bp.length(seqs[i]);
  }
  int32_t* tab = (int32_t*)sg.host;
  int32_t* lens = tab + table_words;
  int32_t* sh = lens + n_seqs;
  int32_t* slots = sh + n_sh;
  std::memcpy(tab, b.data(), (table_words + n_seqs) * sizeof(int32_t));
  if (n_sh) std::memcpy(sh, shared, n_sh * sizeof(int32_t));
  if (n_slots) std::memcpy(slots, slot_mapping, (size_t)n_slots * sizeof(int32_t));
  hipError_t e = hipSuccess;
  if (table_words) e = hipMemcpyAsync(d_table, tab, table_words * 4, hipMemcpyHostToDevice, st);
  if (e == hipSuccess && n_seqs)
    e = hipMemcpyAsync(d_lens, lens, (size_t)n_seqs * 4, hipMemcpyHostToDevice, st);
  if (e == hipSuccess && n_sh) e = hipMemcpyAsync(d_shared, sh, n_sh * 4, hipMemcpyHostToDevice, st);
  if (e == hipSuccess && n_slots)
    e = hipMemcpyAsync(d_slots, slots, (size_t)n_slots * 4, hipMemcpyHostToDevice, st);
  if (e == hipSuccess) e = hipEventRecord(sg.done, st);
  if (e != hipSuccess) return fail(PKV_ERR_HIP, "upload failed: %s", hipGetErrorString(e));
  sg.pending = true;
  pool->next ^= 1;
  return PKV_OK;
}

// Largest incremental patch sent as kernel-argument patches; anything bigger
// goes through the full upload.
constexpr size_t kMaxPatchLaunches = 16;

}  // namespace

extern "C" {

int pkv_block_table_upload(pkv_pool* pool, const int64_t* seqs, int32_t n_seqs,
                           int32_t max_blocks_per_seq, int32_t* d_block_table,
                           int32_t* d_context_lens, int32_t* d_shared_prev,
                           const int32_t* slot_mapping,
                           int32_t* d_slot_mapping, int32_t n_slots,
                           int32_t* max_context_len_out, int64_t* total_tokens_out,
                           int32_t flags, void* stream) {
  PKV_TRY_BEGIN
  if (!pool) return fail(PKV_ERR_INVALID_ARG, "NULL pool");
  if (n_seqs < 0 || max_blocks_per_seq < 0 || n_slots < 0)
    return fail(PKV_ERR_INVALID_ARG, "negative size");
  if (flags & ~PKV_UPLOAD_INCREMENTAL) return fail(PKV_ERR_INVALID_ARG, "unknown flags 0x%x", flags);
  if (n_seqs > 0 && (!seqs || !d_context_lens || (max_blocks_per_seq > 0 && !d_block_table)))
    return fail(PKV_ERR_INVALID_ARG, "NULL table / length pointer");
  if (n_slots > 0 && (!slot_mapping || !d_slot_mapping))
    return fail(PKV_ERR_INVALID_ARG, "NULL slot mapping pointer");
  const pkv::BlockPool& bp = pool->pool;
  int64_t total = 0;
  int32_t longest = 0;
  for (int32_t i = 0; i < n_seqs; ++i) {
    if (!bp.live(seqs[i])) return fail(PKV_ERR_BAD_SEQ, "sequence %lld is not live", (long long)seqs[i]);
    if ((int64_t)bp.table(seqs[i]).size() > max_blocks_per_seq)
      return fail(PKV_ERR_CAPACITY, "sequence %lld holds %zu blocks > max_blocks_per_seq %d",
                  (long long)seqs[i], bp.table(seqs[i]).size(), max_blocks_per_seq);
    const int64_t L = bp.length(seqs[i]);
    if (L > INT32_MAX) return fail(PKV_ERR_UNSUPPORTED, "context length exceeds int32");
    total += L;
    longest = std::max<int32_t>(longest, (int32_t)L);
  }
  hipStream_t st = (hipStream_t)stream;
  std::vector<int32_t> shared;
  if (d_shared_prev) {
    shared.assign(n_seqs, 0);
    for (int32_t i = 1; i < n_seqs; ++i) shared[i] = shared_tokens(bp, seqs[i - 1], seqs[i]);
  }

  // Incremental: rows whose record names the same sequence at the same
  // copy-on-write epoch get only their new entries; other rows are rewritten
  // (entries plus -1 padding).  Lengths and slots are always sent, the
  // shared-token counts when they differ from what this array last received.
  bool full = !(flags & PKV_UPLOAD_INCREMENTAL) || n_seqs == 0;
  std::vector<int32_t> ent, rst;
  auto rec_it = pool->tables.find(d_block_table);
  if (!full && (rec_it == pool->tables.end() || rec_it->second.max_blocks != max_blocks_per_seq))
    full = true;
  bool send_shared = d_shared_prev != nullptr;
  if (!full && send_shared && rec_it->second.shared_dev == d_shared_prev &&
      rec_it->second.shared_sent == shared)
    send_shared = false;
  if (!full) {
    const std::vector<pkv_pool::RowRecord>& rows = rec_it->second.rows;
    const size_t budget = kMaxPatchLaunches * pkv::kPatchWords;
    size_t words = (size_t)n_seqs + n_slots + (send_shared ? n_seqs : 0);
    for (int32_t i = 0; i < n_seqs && !full; ++i) {
      const std::vector<int32_t>& t = bp.table(seqs[i]);
      const int32_t n = (int32_t)t.size();
      int32_t from = 0;
      if (i < (int32_t)rows.size() && rows[i].seq == seqs[i] && rows[i].epoch == bp.epoch(seqs[i]) &&
          rows[i].blocks <= n) {
        from = rows[i].blocks;
      } else {
        rst.push_back(i);
        rst.push_back(n);
        words += 2;
      }
      for (int32_t j = from; j < n; ++j) {
        ent.push_back(i);
        ent.push_back(j);
        ent.push_back(t[j]);
      }
      words += 3 * (size_t)(n - from);
      if (words > budget) full = true;
    }
  }
  if (full) {
    int rc = upload_full(pool, seqs, n_seqs, max_blocks_per_seq, d_block_table, d_context_lens,
                         d_shared_prev, shared.data(), slot_mapping, d_slot_mapping, n_slots, st);
    if (rc) return rc;
  } else {
    // pack lengths, slots, entries and resets into kernel-argument patches
    pkv::TablePatchArgs a;
    const int32_t n_ent = (int32_t)(ent.size() / 3), n_rst = (int32_t)(rst.size() / 2);
    const int32_t n_sh = send_shared ? n_seqs : 0;
    int32_t li = 0, hi = 0, si = 0, ei = 0, ri = 0;
    while (li < n_seqs || hi < n_sh || si < n_slots || ei < n_ent || ri < n_rst) {
      std::memset(&a, 0, offsetof(pkv::TablePatchArgs, w));
      a.table = d_block_table;
      a.lens = d_context_lens;
      a.slots = d_slot_mapping;
      a.shared = d_shared_prev;
      a.max_blocks = max_blocks_per_seq;
      int32_t room = pkv::kPatchWords;
      a.len0 = li;
      a.n_len = std::min(room, n_seqs - li);
      for (int32_t k = 0; k < a.n_len; ++k) a.w[k] = (int32_t)bp.length(seqs[li + k]);
      li += a.n_len;
      room -= a.n_len;
      a.sh0 = hi;
      a.n_sh = std::min(room, n_sh - hi);
      if (a.n_sh) std::memcpy(a.w + a.n_len, shared.data() + hi, (size_t)a.n_sh * 4);
      hi += a.n_sh;
      room -= a.n_sh;
      a.slot0 = si;
      a.n_slot = std::min(room, n_slots - si);
      if (a.n_slot) std::memcpy(a.w + a.n_len + a.n_sh, slot_mapping + si, (size_t)a.n_slot * 4);
      si += a.n_slot;
      room -= a.n_slot;
      int32_t* e = a.w + a.n_len + a.n_sh + a.n_slot;
      a.n_ent = std::min(room / 3, n_ent - ei);
      if (a.n_ent) std::memcpy(e, ent.data() + 3 * (size_t)ei, (size_t)a.n_ent * 12);
      ei += a.n_ent;
      room -= 3 * a.n_ent;
      a.n_reset = std::min(room / 2, n_rst - ri);
      if (a.n_reset) std::memcpy(e + 3 * a.n_ent, rst.data() + 2 * (size_t)ri, (size_t)a.n_reset * 8);
      ri += a.n_reset;
      int rc = pkv::launch_table_patch(a, stream);
      if (rc) return rc;
    }
  }
  // remember what every row of this device table now holds
  if (n_seqs > 0 && max_blocks_per_seq > 0) {
    pkv_pool::TableRecord& tr = pool->tables[d_block_table];
    tr.max_blocks = max_blocks_per_seq;
    tr.rows.resize(n_seqs);
    for (int32_t i = 0; i < n_seqs; ++i) {
      tr.rows[i].seq = seqs[i];
      tr.rows[i].blocks = (int32_t)bp.table(seqs[i]).size();
      tr.rows[i].epoch = bp.epoch(seqs[i]);
    }
    if (d_shared_prev) {
      tr.shared_dev = d_shared_prev;
      tr.shared_sent = shared;
    }
  }
  if (max_context_len_out) *max_context_len_out = longest;
  if (total_tokens_out) *total_tokens_out = total;
  return PKV_OK;
  PKV_TRY_END
}

}  // extern "C"
