// Continuous batching over the block allocator, host only.
//
// From the pages: "Designing an LLM serving system", "Continuous batching"
// (a step frees the blocks of sequences that are done, brings queued
// requests in while room remains, then decodes the batch that results),
// "Paged attention" (blocks
// allocated as a sequence grows; requests that begin with the same prompt
// point at the same prefix blocks; a shared block is copied on write) and
// "Scheduling: when prefill meets decode" (when memory runs out mid
// generation a sequence yields; its blocks are discarded and recomputed
// when it resumes); "Module 23: Serving", 23.3; "Scaling LLM serving",
// "Batching: static to continuous".
//
// One step, in order:
//   1. every request resident in the previous plan has produced one more
//      token; a request that has produced gen_len tokens is finished and its
//      blocks are released;
//   2. every remaining resident request grows by one token (a new block at
//      each 16-token boundary, copy on write of a shared last block); when
//      no block is free the most recently admitted resident request is
//      preempted: its blocks are released and it goes back to the front of
//      the queue, everything it has so far becoming its prompt, to be
//      recomputed when it is admitted again;
//   3. waiting requests are admitted first come first served while the
//      batch has room and the free blocks cover the request's prompt and
//      first token plus one block per resident request (the reserve for
//      next step's growth). A request that begins with the shared prefix
//      forks the prefix's blocks, and the prefix's partly filled last block
//      is copied on write before the request's own tokens go into it.
// The plan lists the resident requests (admission order), their tables and
// context lengths (each including this step's token), the copy-on-write
// pairs to run before any write, and the prompt tokens (row, position) the
// caller must write this step (the prefill's output, or the recomputed
// tokens of a preempted request).
#include <stdint.h>

#include <algorithm>
#include <deque>
#include <new>
#include <vector>

#include "pkv.h"

namespace {

struct Request {
  int64_t id;
  int32_t prompt_len;
  int32_t gen_len;
  int32_t generated;   // tokens produced so far (decode steps it took part in)
  bool shares_prefix;
  int32_t ctx;         // cached tokens including this step's one
  int32_t n_blocks;
  std::vector<int32_t> table;
  std::vector<int32_t> tokens;   // the prompt's token ids, for the prefix cache (may be empty)
};

int32_t blocks_for(int32_t tokens) { return (tokens + PKV_BLOCK_TOKENS - 1) / PKV_BLOCK_TOKENS; }

}  // namespace

struct pkv_batcher {
  pkv_allocator* alloc = nullptr;
  int32_t max_batch = 0, max_blocks = 0, prefix_tokens = 0, prefix_blocks = 0;
  std::vector<int32_t> prefix_table;
  std::deque<Request> waiting;
  std::vector<Request> running;   // admission order
  pkv_prefix_cache* cache = nullptr;   // optional: prompts matched against cached blocks
  std::vector<int32_t> match_table;
  int32_t cached_tokens = 0;           // this step's prompt tokens served from the cache
  // plan buffers, valid until the next step
  std::vector<int32_t> tables, ctx, cow_src, cow_dst, fill_rows, fill_pos;
  std::vector<int64_t> ids, finished, preempted;
};

namespace {

void release(pkv_batcher* b, Request& r) {
  pkv_seq_release(b->alloc, r.table.data(), r.n_blocks);
  std::fill(r.table.begin(), r.table.end(), -1);
  r.n_blocks = 0;
}

// Preempt the most recently admitted resident request (recompute later).
void preempt_last(pkv_batcher* b) {
  Request r = std::move(b->running.back());
  b->running.pop_back();
  release(b, r);
  r.prompt_len += r.generated;   // everything known so far is recomputed
  r.gen_len -= r.generated;
  r.generated = 0;
  r.ctx = 0;
  b->preempted.push_back(r.id);
  b->waiting.push_front(std::move(r));
}

void record_cow(pkv_batcher* b, int32_t src, int32_t dst) {
  if (src >= 0) {
    b->cow_src.push_back(src);
    b->cow_dst.push_back(dst);
  }
}

}  // namespace

extern "C" int pkv_batcher_create(int32_t num_blocks, int32_t max_batch, int32_t max_blocks_per_seq,
                                  int32_t prefix_tokens, pkv_batcher** out) {
  if (!out || num_blocks < 1 || max_batch < 1 || max_blocks_per_seq < 1 || prefix_tokens < 0 ||
      prefix_tokens > PKV_BLOCK_TOKENS * max_blocks_per_seq)
    return PKV_EINVAL;
  *out = nullptr;
  pkv_batcher* b = new (std::nothrow) pkv_batcher;
  if (!b) return PKV_ENOMEM;
  int rc = pkv_allocator_create(num_blocks, &b->alloc);
  if (rc != PKV_OK) {
    delete b;
    return rc;
  }
  b->max_batch = max_batch;
  b->max_blocks = max_blocks_per_seq;
  b->prefix_tokens = prefix_tokens;
  b->prefix_table.assign((size_t)max_blocks_per_seq, -1);
  if (prefix_tokens > 0) {
    int32_t n = 0, src = -1, dst = -1;
    rc = pkv_seq_grow(b->alloc, b->prefix_table.data(), &n, max_blocks_per_seq, prefix_tokens,
                      &src, &dst);
    if (rc != PKV_OK) {
      pkv_allocator_destroy(b->alloc);
      delete b;
      return rc;
    }
    b->prefix_blocks = n;
  }
  *out = b;
  return PKV_OK;
}

extern "C" void pkv_batcher_destroy(pkv_batcher* b) {
  if (!b) return;
  pkv_prefix_cache_destroy(b->cache);
  pkv_allocator_destroy(b->alloc);
  delete b;
}

extern "C" int pkv_batcher_enable_prefix_cache(pkv_batcher* b) {
  if (!b || b->cache) return PKV_EINVAL;
  try {
    b->match_table.assign((size_t)b->max_blocks, -1);
  } catch (...) {
    return PKV_ENOMEM;
  }
  return pkv_prefix_cache_create(b->alloc, &b->cache);
}

extern "C" int32_t pkv_batcher_cached_blocks(const pkv_batcher* b) {
  if (!b) return PKV_EINVAL;
  return b->cache ? pkv_prefix_cached_blocks(b->cache) : 0;
}

extern "C" int32_t pkv_batcher_prefix_table(const pkv_batcher* b, const int32_t** table) {
  if (!b) return PKV_EINVAL;
  if (table) *table = b->prefix_table.data();
  return b->prefix_blocks;
}

extern "C" int pkv_batcher_submit(pkv_batcher* b, int64_t request_id, int32_t prompt_len,
                                  int32_t gen_len, int32_t shares_prefix) {
  if (!b || prompt_len < 1 || gen_len < 1) return PKV_EINVAL;
  if (shares_prefix && (b->prefix_tokens == 0 || prompt_len < b->prefix_tokens)) return PKV_EINVAL;
  const int64_t total = (int64_t)prompt_len + gen_len;
  if (total > (int64_t)PKV_BLOCK_TOKENS * b->max_blocks) return PKV_EINVAL;
  // a request that could never fit, even alone beside the prefix
  if (blocks_for((int32_t)total) > pkv_num_blocks(b->alloc) - b->prefix_blocks) return PKV_ENOMEM;
  try {
    Request r;
    r.id = request_id;
    r.prompt_len = prompt_len;
    r.gen_len = gen_len;
    r.generated = 0;
    r.shares_prefix = shares_prefix != 0;
    r.ctx = 0;
    r.n_blocks = 0;
    r.table.assign((size_t)b->max_blocks, -1);
    b->waiting.push_back(std::move(r));
  } catch (...) {
    return PKV_ENOMEM;
  }
  return PKV_OK;
}

extern "C" int pkv_batcher_submit_tokens(pkv_batcher* b, int64_t request_id,
                                         const int32_t* tokens, int32_t prompt_len,
                                         int32_t gen_len) {
  if (!b || !tokens) return PKV_EINVAL;
  const int rc = pkv_batcher_submit(b, request_id, prompt_len, gen_len, 0);
  if (rc != PKV_OK) return rc;
  try {
    b->waiting.back().tokens.assign(tokens, tokens + prompt_len);
  } catch (...) {
    b->waiting.pop_back();
    return PKV_ENOMEM;
  }
  return PKV_OK;
}

extern "C" int pkv_batcher_step(pkv_batcher* b, pkv_step_plan* plan) {
  if (!b || !plan) return PKV_EINVAL;
  try {
    b->cow_src.clear();
    b->cow_dst.clear();
    b->fill_rows.clear();
    b->fill_pos.clear();
    b->finished.clear();
    b->preempted.clear();

    // 1. the previous step's token; release finished requests
    std::vector<Request> kept;
    kept.reserve(b->running.size());
    for (Request& r : b->running) {
      r.generated += 1;
      if (r.generated >= r.gen_len) {
        b->finished.push_back(r.id);
        release(b, r);
      } else {
        kept.push_back(std::move(r));
      }
    }
    b->running.swap(kept);

    // 2. grow the resident requests by this step's token
    for (size_t i = 0; i < b->running.size();) {
      Request& r = b->running[i];
      int32_t src = -1, dst = -1;
      const int rc = pkv_seq_grow(b->alloc, r.table.data(), &r.n_blocks, b->max_blocks, r.ctx + 1,
                                  &src, &dst);
      if (rc == PKV_OK) {
        r.ctx += 1;
        record_cow(b, src, dst);
        ++i;
        continue;
      }
      if (rc != PKV_ENOMEM) return rc;
      // no free block: a block only the prefix cache holds goes first, then
      // the newest resident request yields (possibly r itself)
      if (b->cache && pkv_prefix_evict(b->cache, 1) == 1) continue;
      preempt_last(b);
    }

    // 3. admit first come first served
    const int32_t prefix_full = b->prefix_tokens / PKV_BLOCK_TOKENS;
    b->cached_tokens = 0;
    while (!b->waiting.empty() && (int32_t)b->running.size() < b->max_batch) {
      Request& w = b->waiting.front();
      const int32_t ctx = w.prompt_len + 1;
      // prompt blocks already cached (all but the last prompt token, which
      // the request computes anyway)
      int32_t matched = 0;
      if (b->cache && !w.tokens.empty()) {
        const int32_t known = std::min((int32_t)w.tokens.size(), w.prompt_len - 1);
        matched = pkv_prefix_match(b->cache, w.tokens.data(), known, b->match_table.data(),
                                   b->max_blocks);
        if (matched < 0) return matched;
      }
      const int32_t own = blocks_for(ctx) - (w.shares_prefix ? prefix_full : 0) - matched;
      const int32_t short_by = own + (int32_t)b->running.size() - pkv_num_free(b->alloc);
      if (short_by > 0 && b->cache) pkv_prefix_evict(b->cache, short_by);
      if (own + (int32_t)b->running.size() > pkv_num_free(b->alloc)) {
        pkv_seq_release(b->alloc, b->match_table.data(), matched);
        break;
      }
      Request r = std::move(w);
      b->waiting.pop_front();
      int32_t start = 0;
      if (matched > 0) {
        for (int32_t k = 0; k < matched; ++k) r.table[k] = b->match_table[k];
        r.n_blocks = matched;
        start = matched * PKV_BLOCK_TOKENS;
        b->cached_tokens += start;
      }
      if (r.shares_prefix) {
        pkv_seq_fork(b->alloc, b->prefix_table.data(), b->prefix_blocks);
        for (int32_t k = 0; k < b->prefix_blocks; ++k) r.table[k] = b->prefix_table[k];
        r.n_blocks = b->prefix_blocks;
        start = b->prefix_tokens;
        if (b->prefix_tokens % PKV_BLOCK_TOKENS != 0) {
          // the request's first own token goes into the prefix's partly
          // filled last block: make that block private first
          int32_t src = -1, dst = -1;
          const int rc = pkv_seq_grow(b->alloc, r.table.data(), &r.n_blocks, b->max_blocks,
                                      b->prefix_tokens + 1, &src, &dst);
          if (rc != PKV_OK) return rc;   // covered by the admission check
          record_cow(b, src, dst);
        }
      }
      int32_t src = -1, dst = -1;
      const int rc = pkv_seq_grow(b->alloc, r.table.data(), &r.n_blocks, b->max_blocks, ctx, &src,
                                  &dst);
      if (rc != PKV_OK) return rc;       // covered by the admission check
      record_cow(b, src, dst);
      r.ctx = ctx;
      const int32_t row = (int32_t)b->running.size();
      for (int32_t p = start; p < r.prompt_len; ++p) {
        b->fill_rows.push_back(row);
        b->fill_pos.push_back(p);
      }
      // the prompt's full blocks join the cache now: in every layer this
      // step's writes come before any request's attention reads them
      if (b->cache && !r.tokens.empty()) {
        const int32_t n = std::min((int32_t)r.tokens.size(), r.prompt_len);
        const int32_t irc = pkv_prefix_insert(b->cache, r.tokens.data(), n, r.table.data(),
                                              r.n_blocks);
        if (irc < 0) return irc;
      }
      b->running.push_back(std::move(r));
    }

    // plan
    const size_t n = b->running.size();
    b->tables.assign(n * (size_t)b->max_blocks, -1);
    b->ctx.resize(n);
    b->ids.resize(n);
    for (size_t i = 0; i < n; ++i) {
      const Request& r = b->running[i];
      std::copy(r.table.begin(), r.table.end(), b->tables.begin() + i * b->max_blocks);
      b->ctx[i] = r.ctx;
      b->ids[i] = r.id;
    }
  } catch (...) {
    return PKV_ENOMEM;
  }
  plan->num_seqs = (int32_t)b->running.size();
  plan->max_blocks_per_seq = b->max_blocks;
  plan->block_tables = b->tables.data();
  plan->context_lens = b->ctx.data();
  plan->request_ids = b->ids.data();
  plan->n_cow = (int32_t)b->cow_src.size();
  plan->cow_src = b->cow_src.data();
  plan->cow_dst = b->cow_dst.data();
  plan->n_fill = (int32_t)b->fill_rows.size();
  plan->fill_rows = b->fill_rows.data();
  plan->fill_positions = b->fill_pos.data();
  plan->n_finished = (int32_t)b->finished.size();
  plan->finished_ids = b->finished.data();
  plan->n_preempted = (int32_t)b->preempted.size();
  plan->preempted_ids = b->preempted.data();
  plan->num_free_blocks = pkv_num_free(b->alloc);
  plan->num_waiting = (int32_t)b->waiting.size();
  plan->n_cached_tokens = b->cached_tokens;
  return PKV_OK;
}
