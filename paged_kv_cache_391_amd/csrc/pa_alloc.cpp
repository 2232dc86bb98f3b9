// Host-side manager of the physical KV blocks: allocation on demand,
// reference counts for blocks shared by forked sequences, copy-on-write and
// reclamation.
//
// The scheme follows the pages: the cache is cut into fixed-size blocks that
// are handed out as a sequence grows and returned when it finishes
// (devpress.csdn.net page, workflow step on memory reclamation; betteryeah.com
// page, section 2.2); each sequence keeps a table from its logical blocks to
// physical ones; parallel samples share the prompt's blocks through their
// tables, with a reference count per block and a copy made before a sharer
// writes into a shared block (aidocs.cortexgrid.cn page, FAQ answer on
// parallel sampling). Only a sequence's last block can be partly filled, so
// only that block is ever copied on write.
//
// Pure host bookkeeping: no device memory is touched. The copies it decides
// on are queued as (src, dst) block pairs that the caller hands to
// pa_copy_blocks before writing the new tokens with pa_reshape_and_cache.
// Free blocks are a LIFO stack that first hands out block 0, 1, 2, ...
//
// Batches. The allocator's calls of one scheduler step form a batch that
// take_copies closes once it has handed out every pending pair; the caller
// then queues the batch's copies and, after them, its cache writes. Within a
// batch the copies run concurrently and before any of the batch's writes, so
// the allocator keeps two rules that make every batch safe to run that way:
//   * a block that received slots in the current batch (its new tokens are
//     not written yet, or it is a copy destination) is never a copy source:
//     an append that would copy it returns PA_ERR_PENDING_WRITES and changes
//     nothing (close the batch, queue its work, then append again);
//   * a block whose count drops to 0 while it received slots or is a copy
//     source in the current batch returns to the pool only when the batch
//     closes, so it is neither a destination of the same batch's copies nor
//     handed a second set of slots in the same batch.
// Together: a batch's destinations are distinct fresh blocks, none is a
// source, and every source holds its final contents when the copies run.
#include <limits.h>

#include <new>
#include <vector>

#include "../../include/pagedattn.h"

struct pa_allocator {
  struct Seq {
    std::vector<int32_t> table;  // physical block of each logical block
    int32_t length = 0;          // tokens stored
    bool live = false;
  };
  int32_t num_blocks = 0;
  int32_t block_size = 0;
  std::vector<int32_t> free_stack;  // back() is handed out next
  std::vector<int32_t> refcount;
  std::vector<Seq> seqs;
  std::vector<int32_t> copies;      // pending (src, dst) pairs, flattened
  int64_t batch = 0;                // number of the open batch
  std::vector<int64_t> filled_in;   // batch in which the block last received slots (-1: never)
  std::vector<int64_t> source_in;   // batch in which the block was last a copy source (-1: never)
  std::vector<int32_t> deferred;    // blocks freed in the open batch, returned when it closes
};

namespace {

bool seq_ok(const pa_allocator* a, int32_t seq) {
  return a && seq >= 0 && seq < (int32_t)a->seqs.size() && a->seqs[seq].live;
}

int32_t take_block(pa_allocator* a) {
  const int32_t b = a->free_stack.back();
  a->free_stack.pop_back();
  a->refcount[b] = 1;
  return b;
}

void release_block(pa_allocator* a, int32_t b) {
  if (--a->refcount[b] != 0) return;
  if (a->filled_in[b] == a->batch || a->source_in[b] == a->batch)
    a->deferred.push_back(b);  // the open batch still writes or reads it
  else
    a->free_stack.push_back(b);
}

// Close the open batch: blocks freed during it return to the pool (in the
// order they were freed), and every block becomes a valid copy source.
void close_batch(pa_allocator* a) {
  for (int32_t b : a->deferred) a->free_stack.push_back(b);
  a->deferred.clear();
  ++a->batch;
}

// Blocks an append of n tokens to s takes from the pool: fresh blocks for
// the tokens that do not fit in the last block, plus one copy when the last
// block is partly filled and shared.
int64_t blocks_needed(const pa_allocator* a, const pa_allocator::Seq& s, int32_t n) {
  if (n <= 0) return 0;
  const int32_t bs = a->block_size;
  const int32_t off = s.length % bs;
  int64_t need = 0;
  int64_t rest = n;
  if (off != 0) {
    if (a->refcount[s.table.back()] > 1) need += 1;
    rest -= bs - off;
  }
  if (rest > 0) need += (rest + bs - 1) / bs;
  return need;
}

}  // namespace

extern "C" {

pa_status pa_allocator_create(int32_t num_blocks, int32_t block_size, pa_allocator** out) {
  if (!out) return PA_ERR_INVALID_ARG;
  *out = nullptr;
  if (num_blocks <= 0 || block_size <= 0 || (int64_t)num_blocks * block_size > INT32_MAX)
    return PA_ERR_INVALID_ARG;
  pa_allocator* a = new (std::nothrow) pa_allocator();
  if (!a) return PA_ERR_NO_MEMORY;
  try {
    a->num_blocks = num_blocks;
    a->block_size = block_size;
    a->refcount.assign(num_blocks, 0);
    a->filled_in.assign(num_blocks, -1);
    a->source_in.assign(num_blocks, -1);
    a->deferred.reserve(num_blocks);  // close_batch and release_block never allocate
    a->free_stack.reserve(num_blocks);
    a->free_stack.resize(num_blocks);
    for (int32_t i = 0; i < num_blocks; ++i) a->free_stack[i] = num_blocks - 1 - i;
  } catch (const std::bad_alloc&) {
    delete a;
    return PA_ERR_NO_MEMORY;
  }
  *out = a;
  return PA_OK;
}

void pa_allocator_destroy(pa_allocator* a) { delete a; }

int32_t pa_allocator_num_free(const pa_allocator* a) { return a ? (int32_t)a->free_stack.size() : -1; }

int32_t pa_allocator_refcount(const pa_allocator* a, int32_t block) {
  if (!a || block < 0 || block >= a->num_blocks) return -1;
  return a->refcount[block];
}

pa_status pa_allocator_new_sequence(pa_allocator* a, int32_t* seq) {
  if (!a || !seq) return PA_ERR_INVALID_ARG;
  if (a->seqs.size() >= (size_t)INT32_MAX) return PA_ERR_NO_MEMORY;
  try {
    a->seqs.emplace_back();
  } catch (const std::bad_alloc&) {
    return PA_ERR_NO_MEMORY;
  }
  a->seqs.back().live = true;
  *seq = (int32_t)a->seqs.size() - 1;
  return PA_OK;
}

pa_status pa_allocator_fork(pa_allocator* a, int32_t parent, int32_t* child) {
  if (!seq_ok(a, parent) || !child) return PA_ERR_INVALID_ARG;
  if (a->seqs.size() >= (size_t)INT32_MAX) return PA_ERR_NO_MEMORY;
  try {
    pa_allocator::Seq c;
    c.table = a->seqs[parent].table;
    c.length = a->seqs[parent].length;
    c.live = true;
    a->seqs.push_back(std::move(c));
  } catch (const std::bad_alloc&) {
    return PA_ERR_NO_MEMORY;
  }
  for (int32_t b : a->seqs.back().table) ++a->refcount[b];
  *child = (int32_t)a->seqs.size() - 1;
  return PA_OK;
}

pa_status pa_allocator_append(pa_allocator* a, int32_t seq, int32_t num_tokens, int32_t* slots) {
  if (!seq_ok(a, seq) || num_tokens < 0) return PA_ERR_INVALID_ARG;
  pa_allocator::Seq& s = a->seqs[seq];
  if ((int64_t)s.length + num_tokens > INT32_MAX) return PA_ERR_INVALID_ARG;
  const int32_t bs = a->block_size;
  // a shared, partly filled last block is copied first: not while the open
  // batch still has writes into it (they would run after the copy)
  if (num_tokens > 0 && s.length % bs != 0 && a->refcount[s.table.back()] > 1 &&
      a->filled_in[s.table.back()] == a->batch)
    return PA_ERR_PENDING_WRITES;  // nothing changed
  const int64_t need = blocks_needed(a, s, num_tokens);
  if (need > (int64_t)a->free_stack.size()) return PA_ERR_NO_BLOCKS;  // nothing changed
  try {
    s.table.reserve(s.table.size() + (size_t)need);
    a->copies.reserve(a->copies.size() + 2);
  } catch (const std::bad_alloc&) {
    return PA_ERR_NO_MEMORY;
  }
  for (int32_t i = 0; i < num_tokens; ++i) {
    const int32_t off = s.length % bs;
    if (off == 0) {
      s.table.push_back(take_block(a));
    } else if (a->refcount[s.table.back()] > 1) {  // shared, partly filled: copy before writing
      const int32_t old = s.table.back();
      const int32_t fresh = take_block(a);
      a->copies.push_back(old);
      a->copies.push_back(fresh);
      a->source_in[old] = a->batch;
      release_block(a, old);
      s.table.back() = fresh;
    }
    a->filled_in[s.table.back()] = a->batch;
    if (slots) slots[i] = s.table.back() * bs + off;
    ++s.length;
  }
  return PA_OK;
}

pa_status pa_allocator_free_sequence(pa_allocator* a, int32_t seq) {
  if (!seq_ok(a, seq)) return PA_ERR_INVALID_ARG;
  pa_allocator::Seq& s = a->seqs[seq];
  for (int32_t b : s.table) release_block(a, b);
  std::vector<int32_t>().swap(s.table);
  s.length = 0;
  s.live = false;
  return PA_OK;
}

int32_t pa_allocator_sequence_length(const pa_allocator* a, int32_t seq) {
  return seq_ok(a, seq) ? a->seqs[seq].length : -1;
}

pa_status pa_allocator_block_table(const pa_allocator* a, int32_t seq, int32_t* table, int32_t capacity,
                                   int32_t* num_blocks) {
  if (!seq_ok(a, seq) || !num_blocks || capacity < 0 || (capacity > 0 && !table)) return PA_ERR_INVALID_ARG;
  const pa_allocator::Seq& s = a->seqs[seq];
  *num_blocks = (int32_t)s.table.size();
  if ((int64_t)capacity < (int64_t)s.table.size()) return capacity == 0 ? PA_OK : PA_ERR_INVALID_ARG;
  for (size_t i = 0; i < s.table.size(); ++i) table[i] = s.table[i];
  return PA_OK;
}

pa_status pa_allocator_take_copies(pa_allocator* a, int32_t* pairs, int32_t capacity, int32_t* num_pairs) {
  if (!a || !num_pairs || capacity < 0 || (capacity > 0 && !pairs)) return PA_ERR_INVALID_ARG;
  const int64_t pending = (int64_t)a->copies.size() / 2;
  if (capacity == 0) {  // query only
    *num_pairs = (int32_t)pending;
    return PA_OK;
  }
  const int64_t n = pending < capacity ? pending : capacity;
  for (int64_t i = 0; i < 2 * n; ++i) pairs[i] = a->copies[i];
  a->copies.erase(a->copies.begin(), a->copies.begin() + 2 * n);
  *num_pairs = (int32_t)n;
  if (a->copies.empty()) close_batch(a);
  return PA_OK;
}

}  // extern "C"
