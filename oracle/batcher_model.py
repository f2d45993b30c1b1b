"""Reference model of the continuous-batching scheduler -- TEST INFRASTRUCTURE ONLY.

Plain Python over AllocatorModel, written from the pages:
  * "Designing an LLM serving system", "Continuous batching": a step frees
    the blocks of sequences that are done, brings queued requests in while
    room remains, then decodes the batch that results; "Paged attention":
    blocks allocated as a sequence grows, a shared prefix's blocks pointed
    at by every request that begins with it, copy on write of a shared
    block; "Scheduling: when prefill meets decode": when memory runs out a
    sequence yields, its blocks discarded and recomputed when it resumes.
  * "Module 23: Serving", 23.3 (a finished request's slot is refilled from
    the queue in the same step).

The policy details the pages leave open are the library's documented ones
(include/pkv.h, pkv_batcher_step): growth of resident requests before
admission, preemption of the most recently admitted request, first come
first served admission with a reserve of one block per resident request.
With a prefix cache ("Scaling LLM serving", "Reuse shared prefixes"): a
request with token ids is matched at admission (all but its last prompt
token), cached blocks are evicted before an admission is refused or a
request preempted, and the prompt's full blocks are cached at admission.
The model is compared with the library plan by plan (tests/test_batcher.py)
and its invariants are checked separately.
"""
from collections import deque

from .allocator_model import AllocatorModel, OutOfBlocks
from .prefix_cache_model import PrefixCacheModel

BLOCK = 16


def _blocks(tokens):
    return -(-tokens // BLOCK)


class _Req:
    def __init__(self, rid, prompt_len, gen_len, shares, tokens=None):
        self.id = rid
        self.prompt_len = prompt_len
        self.gen_len = gen_len
        self.generated = 0
        self.shares = shares
        self.ctx = 0
        self.table = []
        self.tokens = list(tokens) if tokens is not None else []


class BatcherModel:
    def __init__(self, num_blocks, max_batch, max_blocks, prefix_tokens=0):
        self.alloc = AllocatorModel(num_blocks)
        self.max_batch = max_batch
        self.max_blocks = max_blocks
        self.prefix_tokens = prefix_tokens
        self.prefix_table = []
        if prefix_tokens:
            self.alloc.seq_grow(self.prefix_table, prefix_tokens, max_blocks)
        self.waiting = deque()
        self.running = []
        self.cache = None

    def enable_prefix_cache(self):
        self.cache = PrefixCacheModel(self.alloc)

    def submit_tokens(self, rid, tokens, gen_len):
        self.submit(rid, len(tokens), gen_len, False)
        self.waiting[-1].tokens = list(tokens)

    def submit(self, rid, prompt_len, gen_len, shares=False):
        if prompt_len < 1 or gen_len < 1:
            raise ValueError("bad request")
        if shares and (self.prefix_tokens == 0 or prompt_len < self.prefix_tokens):
            raise ValueError("a sharing request starts with the whole prefix")
        if prompt_len + gen_len > BLOCK * self.max_blocks:
            raise ValueError("longer than a table")
        if _blocks(prompt_len + gen_len) > self.alloc.num_blocks - len(self.prefix_table):
            raise OutOfBlocks()
        self.waiting.append(_Req(rid, prompt_len, gen_len, shares))

    def _preempt_last(self, preempted):
        r = self.running.pop()
        self.alloc.seq_release(r.table)
        r.table = []
        r.prompt_len += r.generated
        r.gen_len -= r.generated
        r.generated = 0
        r.ctx = 0
        preempted.append(r.id)
        self.waiting.appendleft(r)

    def step(self):
        cow, fill, finished, preempted = [], [], [], []
        kept = []
        for r in self.running:
            r.generated += 1
            if r.generated >= r.gen_len:
                finished.append(r.id)
                self.alloc.seq_release(r.table)
                r.table = []
            else:
                kept.append(r)
        self.running = kept

        i = 0
        while i < len(self.running):
            r = self.running[i]
            try:
                src, dst = self.alloc.seq_grow(r.table, r.ctx + 1, self.max_blocks)
            except OutOfBlocks:
                if self.cache is not None and self.cache.evict(1) == 1:
                    continue
                self._preempt_last(preempted)
                continue
            r.ctx += 1
            if src >= 0:
                cow.append((src, dst))
            i += 1

        prefix_full = self.prefix_tokens // BLOCK
        cached_tokens = 0
        while self.waiting and len(self.running) < self.max_batch:
            w = self.waiting[0]
            ctx = w.prompt_len + 1
            matched = []
            if self.cache is not None and w.tokens:
                known = min(len(w.tokens), w.prompt_len - 1)
                matched = self.cache.match(w.tokens[:known], self.max_blocks)
            own = _blocks(ctx) - (prefix_full if w.shares else 0) - len(matched)
            short_by = own + len(self.running) - self.alloc.num_free()
            if short_by > 0 and self.cache is not None:
                self.cache.evict(short_by)
            if own + len(self.running) > self.alloc.num_free():
                self.alloc.seq_release(list(matched))
                break
            r = self.waiting.popleft()
            start = 0
            if matched:
                r.table = list(matched)
                start = BLOCK * len(matched)
                cached_tokens += start
            if r.shares:
                self.alloc.seq_fork(self.prefix_table)
                r.table = list(self.prefix_table)
                start = self.prefix_tokens
                if self.prefix_tokens % BLOCK:
                    src, dst = self.alloc.seq_grow(r.table, self.prefix_tokens + 1, self.max_blocks)
                    if src >= 0:
                        cow.append((src, dst))
            src, dst = self.alloc.seq_grow(r.table, ctx, self.max_blocks)
            if src >= 0:
                cow.append((src, dst))
            r.ctx = ctx
            row = len(self.running)
            fill.extend((row, p) for p in range(start, r.prompt_len))
            if self.cache is not None and r.tokens:
                n = min(len(r.tokens), r.prompt_len)
                self.cache.insert(r.tokens[:n], r.table)
            self.running.append(r)

        return {
            "ids": [r.id for r in self.running],
            "ctx": [r.ctx for r in self.running],
            "tables": [list(r.table) for r in self.running],
            "cow": cow,
            "fill": fill,
            "finished": finished,
            "preempted": preempted,
            "num_free": self.alloc.num_free(),
            "num_waiting": len(self.waiting),
            "cached_tokens": cached_tokens,
        }
