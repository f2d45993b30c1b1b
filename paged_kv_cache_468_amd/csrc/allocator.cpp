// Host block allocator with reference counts.
//
// From the pages: blocks are fixed-size and handed out as a sequence grows
// ("Scaling LLM serving", "Managing the cache: PagedAttention"; "Module 23:
// Serving", 23.4); a sequence wastes at most one partly filled block
// ("Module 23: Serving", Exercises); sequences sharing a prefix point at the
// same physical blocks and a shared block is copied when one of them writes
// into it ("Designing an LLM serving system", "Paged attention"); a finished
// sequence gives its blocks back before new requests are admitted (same
// page, "Continuous batching"); the occupancy of the cache is the capacity
// signal (same page, "Autoscaling").
//
// Data structure: a refcount per block and a LIFO stack of free ids, so
// alloc / free are O(1) and a freshly freed block (likely still in cache) is
// reused first. Host memory only; one scheduler thread owns an allocator.
#include <stdint.h>

#include <new>
#include <unordered_map>
#include <vector>

#include "pkv.h"

struct pkv_allocator {
  std::vector<int32_t> refcount;
  std::vector<int32_t> free_stack;   // top = back()
};

namespace {

bool live(const pkv_allocator* a, int32_t id) {
  return id >= 0 && id < (int32_t)a->refcount.size() && a->refcount[id] > 0;
}

void push_free(pkv_allocator* a, int32_t id) { a->free_stack.push_back(id); }

}  // namespace

extern "C" int pkv_allocator_create(int32_t num_blocks, pkv_allocator** out) {
  if (!out || num_blocks < 1) return PKV_EINVAL;
  *out = nullptr;
  pkv_allocator* a = new (std::nothrow) pkv_allocator;
  if (!a) return PKV_ENOMEM;
  try {
    a->refcount.assign((size_t)num_blocks, 0);
    a->free_stack.reserve((size_t)num_blocks);
    for (int32_t b = num_blocks - 1; b >= 0; --b) a->free_stack.push_back(b);
  } catch (...) {
    delete a;
    return PKV_ENOMEM;
  }
  *out = a;
  return PKV_OK;
}

extern "C" void pkv_allocator_destroy(pkv_allocator* a) { delete a; }

extern "C" int pkv_block_alloc(pkv_allocator* a, int32_t* id) {
  if (!a || !id) return PKV_EINVAL;
  if (a->free_stack.empty()) return PKV_ENOMEM;
  const int32_t b = a->free_stack.back();
  a->free_stack.pop_back();
  a->refcount[b] = 1;
  *id = b;
  return PKV_OK;
}

extern "C" int pkv_block_incref(pkv_allocator* a, int32_t id) {
  if (!a || !live(a, id)) return PKV_EINVAL;
  ++a->refcount[id];
  return PKV_OK;
}

extern "C" int pkv_block_decref(pkv_allocator* a, int32_t id) {
  if (!a || !live(a, id)) return PKV_EINVAL;
  if (--a->refcount[id] == 0) push_free(a, id);
  return PKV_OK;
}

extern "C" int32_t pkv_block_refcount(const pkv_allocator* a, int32_t id) {
  if (!a || id < 0 || id >= (int32_t)a->refcount.size()) return -1;
  return a->refcount[id];
}

extern "C" int32_t pkv_num_free(const pkv_allocator* a) {
  return a ? (int32_t)a->free_stack.size() : -1;
}

extern "C" int32_t pkv_num_blocks(const pkv_allocator* a) {
  return a ? (int32_t)a->refcount.size() : -1;
}

extern "C" int pkv_seq_grow(pkv_allocator* a, int32_t* table, int32_t* n_blocks,
                            int32_t max_blocks, int32_t new_context_len, int32_t* cow_src,
                            int32_t* cow_dst) {
  if (!a || !table || !n_blocks || !cow_src || !cow_dst) return PKV_EINVAL;
  if (max_blocks < 1 || *n_blocks < 0 || *n_blocks > max_blocks) return PKV_EINVAL;
  if (new_context_len < 1 || (int64_t)new_context_len > (int64_t)PKV_BLOCK_TOKENS * max_blocks)
    return PKV_EINVAL;
  for (int32_t b = 0; b < *n_blocks; ++b)
    if (!live(a, table[b])) return PKV_EINVAL;
  *cow_src = -1;
  *cow_dst = -1;
  const int32_t need = (new_context_len + PKV_BLOCK_TOKENS - 1) / PKV_BLOCK_TOKENS;
  while (*n_blocks < need) {
    int32_t id;
    if (pkv_block_alloc(a, &id) != PKV_OK) return PKV_ENOMEM;
    table[(*n_blocks)++] = id;
  }
  const int32_t idx = (new_context_len - 1) / PKV_BLOCK_TOKENS;
  const int32_t old = table[idx];
  if (a->refcount[old] > 1) {
    int32_t fresh;
    if (pkv_block_alloc(a, &fresh) != PKV_OK) return PKV_ENOMEM;
    --a->refcount[old];   // > 0 still: never freed here
    table[idx] = fresh;
    *cow_src = old;
    *cow_dst = fresh;
  }
  return PKV_OK;
}

namespace {

// Check, without changing any state, that the n_blocks entries of `table`
// are live blocks and, when releasing, that every block's refcount covers
// the number of times it appears (so a release can never free a block
// twice).
int check_table(const pkv_allocator* a, const int32_t* table, int32_t n_blocks, bool releasing) {
  if (!a || n_blocks < 0 || (n_blocks > 0 && !table)) return PKV_EINVAL;
  std::unordered_map<int32_t, int32_t> count;
  for (int32_t b = 0; b < n_blocks; ++b) {
    if (!live(a, table[b])) return PKV_EINVAL;
    ++count[table[b]];
  }
  if (releasing)
    for (const auto& kv : count)
      if (a->refcount[kv.first] < kv.second) return PKV_EINVAL;
  return PKV_OK;
}

}  // namespace

extern "C" int pkv_seq_fork(pkv_allocator* a, const int32_t* table, int32_t n_blocks) {
  const int rc = check_table(a, table, n_blocks, false);
  if (rc != PKV_OK) return rc;
  for (int32_t b = 0; b < n_blocks; ++b) ++a->refcount[table[b]];
  return PKV_OK;
}

extern "C" int pkv_seq_release(pkv_allocator* a, const int32_t* table, int32_t n_blocks) {
  const int rc = check_table(a, table, n_blocks, true);
  if (rc != PKV_OK) return rc;
  for (int32_t b = 0; b < n_blocks; ++b) pkv_block_decref(a, table[b]);
  return PKV_OK;
}
