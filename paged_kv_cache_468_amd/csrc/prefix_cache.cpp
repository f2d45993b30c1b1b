// Prefix cache over the block allocator, host only: a radix tree from token
// prefixes to the cached KV blocks that hold them.
//
// From the pages: "Scaling LLM serving", "Reuse shared prefixes" (requests
// that begin the same way have the same KV cache for that start; cached
// prefixes are kept in a tree so a new request picks up the cache of its
// longest cached prefix instead of recomputing it) and "Caching and
// shortcuts" (with paged attention, prefix caching is block sharing);
// "Designing an LLM serving system", "Paged attention" (sequences point at
// the same physical blocks, copy on write at divergence).
//
// Granularity is the 16-token block: only whole blocks are cached, since a
// block's contents are fixed once all 16 of its positions are written. A
// node holds a run of whole blocks (its tokens are a multiple of 16 long);
// its children are keyed by the first 16 tokens of their run. Invariants:
//   * every block in the tree holds exactly one reference owned by the tree
//     (callers that use a cached block hold references of their own);
//   * within a node, block i's parent in the prefix order is block i - 1,
//     so the blocks without a cached extension are exactly the last blocks
//     of leaf nodes;
//   * each block carries the tick of the last match or insert that reached
//     it. Eviction frees, one block at a time, the least recently reached
//     block without a cached extension whose only reference is the tree's
//     (ties by block id).
#include <stdint.h>

#include <algorithm>
#include <array>
#include <functional>
#include <map>
#include <memory>
#include <new>
#include <vector>

#include "pkv.h"

namespace {

using Key = std::array<int32_t, PKV_BLOCK_TOKENS>;

struct Node {
  Node* parent = nullptr;
  std::vector<int32_t> tokens;   // 16 * blocks.size()
  std::vector<int32_t> blocks;
  std::vector<uint64_t> ticks;   // per block: last match or insert that reached it
  std::map<Key, std::unique_ptr<Node>> children;
};

Key key_at(const int32_t* tokens) {
  Key k;
  for (int i = 0; i < PKV_BLOCK_TOKENS; ++i) k[i] = tokens[i];
  return k;
}

bool block_equal(const int32_t* a, const int32_t* b) {
  for (int i = 0; i < PKV_BLOCK_TOKENS; ++i)
    if (a[i] != b[i]) return false;
  return true;
}

}  // namespace

struct pkv_prefix_cache {
  pkv_allocator* alloc = nullptr;
  Node root;
  uint64_t tick = 0;
  int32_t n_blocks = 0;
};

namespace {

// Split node c after its first k blocks (0 < k < c->blocks.size()): c keeps
// the first k, a new child takes the rest and c's children.
void split(Node* c, size_t k) {
  std::unique_ptr<Node> tail(new Node);
  tail->parent = c;
  tail->tokens.assign(c->tokens.begin() + k * PKV_BLOCK_TOKENS, c->tokens.end());
  tail->blocks.assign(c->blocks.begin() + k, c->blocks.end());
  tail->ticks.assign(c->ticks.begin() + k, c->ticks.end());
  tail->children.swap(c->children);
  for (auto& kv : tail->children) kv.second->parent = tail.get();
  c->tokens.resize(k * PKV_BLOCK_TOKENS);
  c->blocks.resize(k);
  c->ticks.resize(k);
  const Key key = key_at(tail->tokens.data());
  c->children.emplace(key, std::move(tail));
}

void drop_subtree(pkv_prefix_cache* pc, Node* n) {
  for (auto& kv : n->children) drop_subtree(pc, kv.second.get());
  for (int32_t b : n->blocks) pkv_block_decref(pc->alloc, b);
  pc->n_blocks -= (int32_t)n->blocks.size();
}

// Evictable blocks: the last block of a leaf node whose only reference is
// the tree's. Ordered by (tick, block id): least recently reached first,
// ties (not expected: one operation reaches one path) by block id.
struct Candidate {
  uint64_t tick;
  int32_t block;
  Node* node;
  bool operator>(const Candidate& o) const {
    return tick != o.tick ? tick > o.tick : block > o.block;
  }
};

bool evictable(pkv_prefix_cache* pc, const Node* n) {
  return n != &pc->root && n->children.empty() && !n->blocks.empty() &&
         pkv_block_refcount(pc->alloc, n->blocks.back()) == 1;
}

void collect(pkv_prefix_cache* pc, Node* n, std::vector<Candidate>& out) {
  if (evictable(pc, n)) out.push_back({n->ticks.back(), n->blocks.back(), n});
  for (auto& kv : n->children) collect(pc, kv.second.get(), out);
}

}  // namespace

extern "C" int pkv_prefix_cache_create(pkv_allocator* alloc, pkv_prefix_cache** out) {
  if (!alloc || !out) return PKV_EINVAL;
  *out = new (std::nothrow) pkv_prefix_cache;
  if (!*out) return PKV_ENOMEM;
  (*out)->alloc = alloc;
  return PKV_OK;
}

extern "C" void pkv_prefix_cache_destroy(pkv_prefix_cache* pc) {
  if (!pc) return;
  drop_subtree(pc, &pc->root);
  delete pc;
}

extern "C" int32_t pkv_prefix_cached_blocks(const pkv_prefix_cache* pc) {
  return pc ? pc->n_blocks : PKV_EINVAL;
}

extern "C" int32_t pkv_prefix_match(pkv_prefix_cache* pc, const int32_t* tokens, int32_t n_tokens,
                                    int32_t* table, int32_t max_blocks) {
  if (!pc || n_tokens < 0 || max_blocks < 0 || (n_tokens > 0 && !tokens) ||
      (max_blocks > 0 && !table))
    return PKV_EINVAL;
  const int32_t want = n_tokens / PKV_BLOCK_TOKENS < max_blocks ? n_tokens / PKV_BLOCK_TOKENS
                                                                  : max_blocks;
  const uint64_t now = ++pc->tick;
  Node* n = &pc->root;
  int32_t m = 0;
  while (m < want) {
    auto it = n->children.find(key_at(tokens + (int64_t)m * PKV_BLOCK_TOKENS));
    if (it == n->children.end()) break;
    Node* c = it->second.get();
    size_t k = 0;
    while (k < c->blocks.size() && m < want &&
           block_equal(c->tokens.data() + k * PKV_BLOCK_TOKENS,
                       tokens + (int64_t)m * PKV_BLOCK_TOKENS)) {
      table[m] = c->blocks[k];
      pkv_block_incref(pc->alloc, c->blocks[k]);
      c->ticks[k] = now;
      ++k;
      ++m;
    }
    if (k < c->blocks.size()) break;
    n = c;
  }
  return m;
}

extern "C" int32_t pkv_prefix_insert(pkv_prefix_cache* pc, const int32_t* tokens,
                                     int32_t n_tokens, const int32_t* table, int32_t n_blocks) {
  if (!pc || n_tokens < 0 || n_blocks < 0 || (n_tokens > 0 && !tokens) || (n_blocks > 0 && !table))
    return PKV_EINVAL;
  const int32_t want = n_tokens / PKV_BLOCK_TOKENS < n_blocks ? n_tokens / PKV_BLOCK_TOKENS
                                                                : n_blocks;
  for (int32_t i = 0; i < want; ++i)
    if (pkv_block_refcount(pc->alloc, table[i]) < 1) return PKV_EINVAL;
  try {
    const uint64_t now = ++pc->tick;
    Node* n = &pc->root;
    int32_t m = 0;
    while (m < want) {
      const int32_t* tk = tokens + (int64_t)m * PKV_BLOCK_TOKENS;
      auto it = n->children.find(key_at(tk));
      if (it == n->children.end()) {
        // a new leaf for the rest: the tree takes a reference to each block
        std::unique_ptr<Node> leaf(new Node);
        leaf->parent = n;
        leaf->tokens.assign(tk, tokens + (int64_t)want * PKV_BLOCK_TOKENS);
        leaf->blocks.assign(table + m, table + want);
        leaf->ticks.assign((size_t)(want - m), now);
        for (int32_t b : leaf->blocks) pkv_block_incref(pc->alloc, b);
        const int32_t added = want - m;
        pc->n_blocks += added;
        n->children.emplace(key_at(tk), std::move(leaf));
        return added;
      }
      Node* c = it->second.get();
      size_t k = 0;
      while (k < c->blocks.size() && m < want &&
             block_equal(c->tokens.data() + k * PKV_BLOCK_TOKENS,
                         tokens + (int64_t)m * PKV_BLOCK_TOKENS)) {
        c->ticks[k] = now;   // already cached (possibly in other blocks): keep the tree's
        ++k;
        ++m;
      }
      if (k < c->blocks.size()) {
        if (m == want) return 0;
        split(c, k);   // the rest diverges inside c's run
      }
      n = c;
    }
    return 0;
  } catch (...) {
    return PKV_ENOMEM;
  }
}

extern "C" int32_t pkv_prefix_evict(pkv_prefix_cache* pc, int32_t n_blocks) {
  if (!pc || n_blocks < 0) return PKV_EINVAL;
  if (n_blocks == 0) return 0;
  try {
    // one walk of the tree, then a heap: each node is in it at most once
    // (a leaf is pushed again only after its entry was taken, a parent only
    // when its last child goes), and nothing else changes refcounts here
    std::vector<Candidate> heap;
    collect(pc, &pc->root, heap);
    std::greater<Candidate> later;
    std::make_heap(heap.begin(), heap.end(), later);
    int32_t freed = 0;
    while (freed < n_blocks && !heap.empty()) {
      std::pop_heap(heap.begin(), heap.end(), later);
      Node* victim = heap.back().node;
      heap.pop_back();
      pkv_block_decref(pc->alloc, victim->blocks.back());
      victim->blocks.pop_back();
      victim->ticks.pop_back();
      victim->tokens.resize(victim->blocks.size() * PKV_BLOCK_TOKENS);
      --pc->n_blocks;
      ++freed;
      Node* next = victim;
      if (victim->blocks.empty()) {
        Node* p = victim->parent;
        for (auto it = p->children.begin(); it != p->children.end(); ++it)
          if (it->second.get() == victim) {
            p->children.erase(it);
            break;
          }
        next = p;
      }
      if (evictable(pc, next)) {
        heap.push_back({next->ticks.back(), next->blocks.back(), next});
        std::push_heap(heap.begin(), heap.end(), later);
      }
    }
    return freed;
  } catch (...) {
    return PKV_ENOMEM;
  }
}
