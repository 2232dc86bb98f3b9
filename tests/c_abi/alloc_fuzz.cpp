// The block allocator (pa_alloc.cpp, the library's host code) driven by
// random operations, built together with it under AddressSanitizer and
// UndefinedBehaviorSanitizer by the CPU test suite. Every batch is run the
// way a caller queues it on one stream (all copies read their sources, then
// write; then the batch's cache writes land) on a model of the pool that
// holds token ids, and every live sequence must read back its own tokens
// through its table. Also exercises every error path. Prints
// "alloc_fuzz ok <ops> <refused>" and exits 0; any sanitizer report or
// failed check ends it with a non-zero status.
#include <cstdio>
#include <cstdlib>
#include <map>
#include <set>
#include <vector>

#include "pagedattn.h"

#define CHECK(c)                                                     \
  do {                                                               \
    if (!(c)) {                                                      \
      std::printf("FAIL line %d: %s\n", __LINE__, #c);               \
      std::exit(1);                                                  \
    }                                                                \
  } while (0)

static uint64_t rng_state = 391;
static uint32_t rnd(uint32_t n) {  // xorshift64*, test data only
  rng_state ^= rng_state >> 12;
  rng_state ^= rng_state << 25;
  rng_state ^= rng_state >> 27;
  return (uint32_t)((rng_state * 2685821657736338717ull) >> 33) % n;
}

int main(int argc, char** argv) {
  const int ops = argc > 1 ? std::atoi(argv[1]) : 20000;
  long refused = 0;
  for (int bs : {1, 4, 16}) {
    const int nb = 48;
    pa_allocator* a = nullptr;
    CHECK(pa_allocator_create(nb, bs, &a) == PA_OK);
    std::vector<std::vector<long>> content(nb, std::vector<long>(bs, -1));
    std::map<int32_t, std::vector<long>> tokens;
    std::vector<std::pair<int32_t, long>> writes;
    long next_tok = 0;
    std::vector<int32_t> table(nb + 1), slots(4 * bs + 2), pairs(2 * nb + 2);

    auto close = [&]() {
      int32_t n = -1;
      CHECK(pa_allocator_take_copies(a, pairs.data(), nb + 1, &n) == PA_OK && n >= 0);
      std::set<int32_t> dst, src;
      for (int i = 0; i < n; ++i) {
        CHECK(dst.insert(pairs[2 * i + 1]).second);
        src.insert(pairs[2 * i]);
      }
      for (int32_t d : dst) CHECK(!src.count(d));
      std::vector<std::vector<long>> snap(n);
      for (int i = 0; i < n; ++i) snap[i] = content[pairs[2 * i]];
      for (int i = 0; i < n; ++i) content[pairs[2 * i + 1]] = snap[i];
      std::set<int32_t> seen;
      for (auto& w : writes) {
        CHECK(seen.insert(w.first).second);
        content[w.first / bs][w.first % bs] = w.second;
      }
      writes.clear();
      for (auto& kv : tokens) {
        int32_t m = 0;
        CHECK(pa_allocator_block_table(a, kv.first, table.data(), nb + 1, &m) == PA_OK);
        for (size_t t = 0; t < kv.second.size(); ++t) CHECK(content[table[t / bs]][t % bs] == kv.second[t]);
      }
    };

    for (int i = 0; i < ops; ++i) {
      const uint32_t op = rnd(8);
      if (op == 0 || tokens.empty()) {
        int32_t s = -1;
        CHECK(pa_allocator_new_sequence(a, &s) == PA_OK);
        tokens[s] = {};
        continue;
      }
      auto it = tokens.begin();
      std::advance(it, rnd((uint32_t)tokens.size()));
      const int32_t sid = it->first;
      if (op <= 3 || op == 4) {
        int32_t target = sid;
        if (op == 4) {  // fork, then the child's first token at once
          CHECK(pa_allocator_fork(a, sid, &target) == PA_OK);
          tokens[target] = tokens[sid];
        }
        const int n = op == 4 ? 1 : 1 + (int)rnd(2 * bs + 1);
        const int32_t free_before = pa_allocator_num_free(a);
        const int32_t len_before = pa_allocator_sequence_length(a, target);
        const pa_status st = pa_allocator_append(a, target, n, slots.data());
        if (st != PA_OK) {
          CHECK(st == PA_ERR_NO_BLOCKS || st == PA_ERR_PENDING_WRITES);
          CHECK(pa_allocator_num_free(a) == free_before && pa_allocator_sequence_length(a, target) == len_before);
          refused += st == PA_ERR_PENDING_WRITES;
          continue;
        }
        for (int k = 0; k < n; ++k) {
          writes.push_back({slots[k], next_tok});
          tokens[target].push_back(next_tok++);
        }
      } else if (op == 5) {
        CHECK(pa_allocator_free_sequence(a, sid) == PA_OK);
        tokens.erase(sid);
      } else {
        close();
      }
    }
    close();
    long refs = 0, entries = 0;
    for (int b = 0; b < nb; ++b) refs += pa_allocator_refcount(a, b);
    for (auto& kv : tokens) {
      int32_t m = 0;
      CHECK(pa_allocator_block_table(a, kv.first, nullptr, 0, &m) == PA_OK);
      entries += m;
    }
    CHECK(refs == entries);
    // error paths
    int32_t m = 0, dummy = 0;
    CHECK(pa_allocator_append(a, -1, 1, nullptr) == PA_ERR_INVALID_ARG);
    CHECK(pa_allocator_append(a, 1 << 30, 1, nullptr) == PA_ERR_INVALID_ARG);
    CHECK(pa_allocator_fork(a, -5, &dummy) == PA_ERR_INVALID_ARG);
    CHECK(pa_allocator_free_sequence(a, 1 << 30) == PA_ERR_INVALID_ARG);
    CHECK(pa_allocator_take_copies(a, nullptr, 3, &m) == PA_ERR_INVALID_ARG);
    CHECK(pa_allocator_take_copies(nullptr, pairs.data(), 3, &m) == PA_ERR_INVALID_ARG);
    CHECK(pa_allocator_refcount(a, nb) == -1 && pa_allocator_refcount(a, -1) == -1);
    CHECK(pa_allocator_num_free(nullptr) == -1);
    if (!tokens.empty()) {
      const int32_t s = tokens.begin()->first;
      CHECK(pa_allocator_block_table(a, s, nullptr, 0, &m) == PA_OK);
      if (m > 1) CHECK(pa_allocator_block_table(a, s, table.data(), m - 1, &m) == PA_ERR_INVALID_ARG);
    }
    for (auto& kv : tokens) CHECK(pa_allocator_free_sequence(a, kv.first) == PA_OK);
    tokens.clear();
    close();
    CHECK(pa_allocator_num_free(a) == nb);
    pa_allocator_destroy(a);
  }
  pa_allocator* bad = nullptr;
  CHECK(pa_allocator_create(0, 16, &bad) == PA_ERR_INVALID_ARG && bad == nullptr);
  CHECK(pa_allocator_create(1 << 28, 16, &bad) == PA_ERR_INVALID_ARG);
  CHECK(pa_allocator_create(4, 16, nullptr) == PA_ERR_INVALID_ARG);
  std::printf("alloc_fuzz ok %d %ld\n", ops, refused);
  return 0;
}
