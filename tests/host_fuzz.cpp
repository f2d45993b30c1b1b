// Randomised driver of the host half of the library (block allocator,
// prefix cache, continuous-batching scheduler), built with AddressSanitizer
// and UndefinedBehaviorSanitizer by tests/test_host_sanitizers.py. Random
// valid and invalid calls; after each, checks that hold whatever the
// sequence of calls: block conservation, refcounts never negative, plans
// whose tables, fill lists and copy pairs stay inside the pool and the
// contexts, and an empty pool once everything is released or evicted. Any
// out-of-bounds access, leak, use after free or undefined arithmetic
// aborts the run. Test infrastructure only.
#include <cstdio>
#include <cstdlib>
#include <random>
#include <vector>
#include <set>
#include "pkv.h"

#define CHECK(c) do { if (!(c)) { fprintf(stderr, "CHECK failed %s:%d: %s\n", __FILE__, __LINE__, #c); abort(); } } while (0)

static void fuzz_alloc(std::mt19937& g) {
  int nb = 1 + g() % 64;
  pkv_allocator* a = nullptr;
  CHECK(pkv_allocator_create(nb, &a) == PKV_OK);
  std::vector<std::vector<int32_t>> seqs;
  const int MB = 8;
  for (int it = 0; it < 400; ++it) {
    int op = g() % 8;
    if (op == 0) { int32_t id; pkv_block_alloc(a, &id); }
    else if (op == 1) { pkv_block_incref(a, (int)(g() % (nb + 4)) - 2); }
    else if (op == 2) { pkv_block_decref(a, (int)(g() % (nb + 4)) - 2); }
    else if (op == 3) {
      std::vector<int32_t> t(MB, -1); int32_t n = 0, cs, cd;
      int ctx = (int)(g() % (16 * MB + 3)) - 1;
      int rc = pkv_seq_grow(a, t.data(), &n, MB, ctx, &cs, &cd);
      if (rc == PKV_OK || rc == PKV_ENOMEM) { t.resize(n); seqs.push_back(t); }
    } else if (op == 4 && !seqs.empty()) {
      auto& t = seqs[g() % seqs.size()];
      std::vector<int32_t> tt(MB, -1);
      for (size_t i = 0; i < t.size(); ++i) tt[i] = t[i];
      int32_t n = (int32_t)t.size(), cs, cd;
      int ctx = 1 + (int)(g() % (16 * MB));
      if (ctx > 16 * n - 15 || n == 0) {
        int rc = pkv_seq_grow(a, tt.data(), &n, MB, ctx, &cs, &cd);
        if (rc == PKV_OK || rc == PKV_ENOMEM) { tt.resize(n); t = tt; }
      }
    } else if (op == 5 && !seqs.empty()) {
      auto& t = seqs[g() % seqs.size()];
      if (pkv_seq_fork(a, t.data(), (int32_t)t.size()) == PKV_OK) seqs.push_back(t);
    } else if (op == 6 && !seqs.empty()) {
      size_t i = g() % seqs.size();
      pkv_seq_release(a, seqs[i].data(), (int32_t)seqs[i].size());
      seqs.erase(seqs.begin() + i);
    } else if (op == 7) {
      std::vector<int32_t> bad = {(int32_t)(g() % (nb + 3)) - 1, nb + 5};
      pkv_seq_release(a, bad.data(), 2);
      pkv_seq_fork(a, bad.data(), 2);
    }
    int32_t live = 0;
    for (int b = 0; b < nb; ++b) { CHECK(pkv_block_refcount(a, b) >= 0); live += pkv_block_refcount(a, b) > 0; }
    CHECK(live + pkv_num_free(a) == nb);
  }
  pkv_allocator_destroy(a);
}

static void fuzz_prefix(std::mt19937& g) {
  int nb = 8 + g() % 120;
  pkv_allocator* a = nullptr;
  CHECK(pkv_allocator_create(nb, &a) == PKV_OK);
  pkv_prefix_cache* pc = nullptr;
  CHECK(pkv_prefix_cache_create(a, &pc) == PKV_OK);
  const int MB = 16;
  std::vector<std::vector<int32_t>> hist;
  for (int it = 0; it < 300; ++it) {
    std::vector<int32_t> tok;
    if (!hist.empty() && g() % 2) tok = hist[g() % hist.size()];
    int extra = g() % 60;
    for (int i = 0; i < extra; ++i) tok.push_back(g() % 4);
    if ((int)tok.size() > 16 * MB) tok.resize(16 * MB);
    std::vector<int32_t> t(MB, -1);
    int n_match_tok = tok.empty() ? 0 : (int)tok.size() - 1;
    int m = pkv_prefix_match(pc, tok.data(), n_match_tok, t.data(), (int)(g() % (MB + 1)));
    CHECK(m >= 0);
    int32_t n = m, cs, cd;
    int need = ((int)tok.size() + 15) / 16 - m;
    if (need > pkv_num_free(a)) pkv_prefix_evict(pc, need - pkv_num_free(a));
    int rc = tok.empty() ? PKV_OK : pkv_seq_grow(a, t.data(), &n, MB, (int)tok.size(), &cs, &cd);
    if (rc == PKV_OK) {
      int ins = pkv_prefix_insert(pc, tok.data(), (int)tok.size(), t.data(), n);
      CHECK(ins >= 0);
      hist.push_back(tok);
    }
    pkv_seq_release(a, t.data(), n);
    if (g() % 7 == 0) pkv_prefix_evict(pc, g() % 5);
    // bad calls
    pkv_prefix_match(pc, nullptr, 16, t.data(), 4);
    pkv_prefix_insert(pc, tok.data(), (int)tok.size(), nullptr, 3);
    std::vector<int32_t> bad(MB, nb + 7);
    if (tok.size() >= 16) CHECK(pkv_prefix_insert(pc, tok.data(), (int)tok.size(), bad.data(), 1) == PKV_EINVAL);
    CHECK(pkv_prefix_cached_blocks(pc) + pkv_num_free(a) == nb);
  }
  CHECK(pkv_prefix_evict(pc, 1 << 20) >= 0);
  CHECK(pkv_num_free(a) == nb);
  pkv_prefix_cache_destroy(pc);
  pkv_allocator_destroy(a);
}

static long st_pre = 0, st_cached = 0, st_cow = 0, st_fin = 0, st_fill = 0;
static void fuzz_batcher(std::mt19937& g) {
  int nb = 4 + g() % 60, mbatch = 1 + g() % 8, mb = 2 + g() % 20;
  int prefix = (g() % 3 == 0) ? (int)(g() % (16 * 3)) : 0;
  pkv_batcher* b = nullptr;
  int rc = pkv_batcher_create(nb, mbatch, mb, prefix, &b);
  if (rc != PKV_OK) { CHECK(b == nullptr || true); return; }
  bool cache = g() % 2;
  if (cache) CHECK(pkv_batcher_enable_prefix_cache(b) == PKV_OK);
  std::vector<std::vector<int32_t>> hist;
  int64_t id = 0;
  for (int it = 0; it < 400; ++it) {
    if (g() % 3 == 0) {
      int plen = (int)(g() % (16 * mb + 4)) - 2, gen = (int)(g() % 40) - 1;
      if (cache && g() % 2) {
        std::vector<int32_t> tok;
        if (!hist.empty() && g() % 2) tok = hist[g() % hist.size()];
        while ((int)tok.size() < plen) tok.push_back(g() % 3);
        if (plen >= 0 && (int)tok.size() > plen) tok.resize(plen);
        if (pkv_batcher_submit_tokens(b, id++, tok.data(), plen, gen) == PKV_OK) hist.push_back(tok);
      } else {
        pkv_batcher_submit(b, id++, plen, gen, prefix > 0 && g() % 2);
      }
    }
    pkv_step_plan p;
    CHECK(pkv_batcher_step(b, &p) == PKV_OK);
    st_pre += p.n_preempted; st_cached += p.n_cached_tokens; st_cow += p.n_cow; st_fin += p.n_finished; st_fill += p.n_fill;
    std::set<int32_t> priv;
    for (int r = 0; r < p.num_seqs; ++r) {
      int ctx = p.context_lens[r];
      CHECK(ctx >= 1 && ctx <= 16 * mb);
      for (int k = 0; k < (ctx + 15) / 16; ++k) {
        int32_t blk = p.block_tables[r * p.max_blocks_per_seq + k];
        CHECK(blk >= 0 && blk < nb);
      }
      for (int k = (ctx + 15) / 16; k < p.max_blocks_per_seq; ++k)
        CHECK(p.block_tables[r * p.max_blocks_per_seq + k] == -1);
    }
    for (int i = 0; i < p.n_fill; ++i) {
      CHECK(p.fill_rows[i] >= 0 && p.fill_rows[i] < p.num_seqs);
      CHECK(p.fill_positions[i] >= 0 && p.fill_positions[i] < p.context_lens[p.fill_rows[i]]);
    }
    for (int i = 0; i < p.n_cow; ++i) CHECK(p.cow_src[i] >= 0 && p.cow_dst[i] >= 0 && p.cow_src[i] < nb && p.cow_dst[i] < nb);
    CHECK(p.num_free_blocks >= 0 && p.num_free_blocks <= nb);
    if (cache) CHECK(pkv_batcher_cached_blocks(b) >= 0);
  }
  pkv_batcher_destroy(b);
}

int main(int argc, char** argv) {
  int iters = argc > 1 ? atoi(argv[1]) : 200;
  for (int s = 0; s < iters; ++s) {
    std::mt19937 g(s);
    fuzz_alloc(g);
    fuzz_prefix(g);
    fuzz_batcher(g);
  }
  // null handles
  pkv_allocator_destroy(nullptr); pkv_prefix_cache_destroy(nullptr); pkv_batcher_destroy(nullptr);
  printf("ok %d: preempted %ld cached %ld cow %ld finished %ld fill %ld\n", iters, st_pre, st_cached, st_cow, st_fin, st_fill);
  return 0;
}
