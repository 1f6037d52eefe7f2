// Host-only stress driver for the block pool, built with AddressSanitizer and
// UndefinedBehaviorSanitizer (g++, no device code): random create / append /
// fork / release / set_table sequences against the pool class, with the
// bookkeeping identities checked after every operation and the all-or-nothing
// rule checked on every refused call.
#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <random>
#include <set>
#include <vector>

#include "block_pool.hpp"
#include "internal.hpp"

namespace pkv {
int fail(int code, const char*, ...) { return code; }
}  // namespace pkv

#define CHECK(c)                                                      \
  do {                                                                \
    if (!(c)) {                                                       \
      std::fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #c); \
      std::exit(1);                                                   \
    }                                                                 \
  } while (0)

struct Snapshot {
  std::vector<int32_t> free_list, ref;
  bool operator==(const Snapshot& o) const { return free_list == o.free_list && ref == o.ref; }
};

static Snapshot snap(const pkv::BlockPool& p) {
  Snapshot s;
  std::vector<int32_t> f(p.num_blocks()), r(p.num_blocks());
  p.export_state(f.data(), r.data());
  f.resize(p.free_count());
  s.free_list = f;
  s.ref = r;
  return s;
}

static void check_invariants(const pkv::BlockPool& p, const std::vector<int64_t>& live) {
  const int32_t nb = p.num_blocks(), bs = p.block_size();
  Snapshot s = snap(p);
  // the free list holds each unreferenced block exactly once
  std::set<int32_t> fr(s.free_list.begin(), s.free_list.end());
  CHECK((int64_t)fr.size() == p.free_count());
  for (int32_t b = 0; b < nb; ++b) CHECK((s.ref[b] == 0) == (fr.count(b) == 1));
  // references equal table entries over live sequences; tables fit lengths
  std::vector<int64_t> refs(nb, 0);
  int64_t tokens = 0;
  for (int64_t q : live) {
    CHECK(p.live(q));
    const auto& t = p.table(q);
    const int64_t len = p.length(q);
    CHECK((int64_t)t.size() == (len + bs - 1) / bs);
    std::set<int32_t> own(t.begin(), t.end());
    CHECK(own.size() == t.size());  // no block twice in one table
    for (int32_t b : t) {
      CHECK(b >= 0 && b < nb);
      ++refs[b];
    }
    tokens += len;
  }
  for (int32_t b = 0; b < nb; ++b) CHECK(refs[b] == s.ref[b]);
  CHECK(p.live_seqs() == (int64_t)live.size());
  CHECK(p.live_tokens() <= tokens);  // shared tokens count once
}

int main(int argc, char** argv) {
  const int iters = argc > 1 ? std::atoi(argv[1]) : 20000;
  for (int32_t bs : {1, 2, 16}) {
    for (uint32_t seed = 1; seed <= 3; ++seed) {
      std::mt19937 rng(seed * 7919u + bs);
      const int32_t nb = 48;
      std::vector<int32_t> order(nb);
      for (int32_t i = 0; i < nb; ++i) order[i] = i;
      std::shuffle(order.begin(), order.end(), rng);
      pkv::BlockPool pool(nb, bs, order.data());
      std::vector<int64_t> live;
      for (int it = 0; it < iters; ++it) {
        const int op = (int)(rng() % 10);
        if (op <= 1 || live.empty()) {
          live.push_back(pool.create());
        } else if (op <= 5) {
          // append to up to 4 distinct live sequences
          std::vector<int64_t> seqs;
          std::vector<int32_t> n;
          for (int k = 0; k < 4 && k < (int)live.size(); ++k) {
            const int64_t q = live[rng() % live.size()];
            bool dup = false;
            for (int64_t x : seqs) dup |= x == q;
            if (dup) continue;
            seqs.push_back(q);
            n.push_back((int32_t)(rng() % (3 * bs + 2)));
          }
          int64_t total = 0;
          for (int32_t x : n) total += x;
          std::vector<int32_t> slots(total + 1), cow(2 * seqs.size() + 2);
          int32_t ncow = 0;
          const Snapshot before = snap(pool);
          const int rc = pool.append(seqs.data(), n.data(), (int32_t)seqs.size(), slots.data(),
                                     total, cow.data(), (int32_t)seqs.size() + 1, &ncow);
          if (rc != PKV_OK) {
            CHECK(rc == PKV_ERR_NO_BLOCKS);
            CHECK(snap(pool) == before);  // all or nothing
          } else {
            for (int64_t i = 0; i < total; ++i) CHECK(slots[i] >= 0 && slots[i] < nb * bs);
            for (int32_t i = 0; i < ncow; ++i) CHECK(cow[2 * i] != cow[2 * i + 1]);
          }
        } else if (op <= 6) {
          int64_t child = -1;
          CHECK(pool.fork(live[rng() % live.size()], &child) == PKV_OK);
          live.push_back(child);
        } else if (op <= 8) {
          const size_t i = rng() % live.size();
          CHECK(pool.release(live[i]) == PKV_OK);
          live.erase(live.begin() + (long)i);
        } else {
          // explicit placement on a fresh sequence from currently free blocks
          const Snapshot s = snap(pool);
          if (!s.free_list.empty()) {
            const int32_t k = 1 + (int32_t)(rng() % std::min<size_t>(3, s.free_list.size()));
            std::vector<int32_t> phys(s.free_list.begin(), s.free_list.begin() + k);
            const int64_t q = pool.create();
            const int64_t len = (int64_t)(k - 1) * bs + 1 + (int64_t)(rng() % bs);
            const int rc = pool.set_table(q, phys.data(), k, len);
            CHECK(rc == PKV_OK);
            live.push_back(q);
          }
        }
        // released ids must be refused
        CHECK(pool.release(-1) != PKV_OK);
        check_invariants(pool, live);
      }
    }
  }
  std::printf("pool stress: ok\n");
  return 0;
}
