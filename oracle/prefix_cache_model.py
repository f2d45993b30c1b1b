"""Reference model of the prefix cache -- TEST INFRASTRUCTURE ONLY.

Plain Python over AllocatorModel, written from "Scaling LLM serving",
"Reuse shared prefixes" (cached prefixes kept so that a request starting
the same way picks up their KV cache) and "Caching and shortcuts" (with
paged attention this is block sharing), and "Designing an LLM serving
system", "Paged attention".

The cache is a plain dictionary with no tree structure: the entry for
prefix tokens[:16 * (k + 1)] holds the block with positions 16k .. 16k+15
of every sequence that starts with those tokens, and the tick of the last
match or insert that reached it. The library's radix tree must behave as
this dictionary does, operation by operation:
  * match(tokens): the longest k with every prefix up to 16k cached; the
    caller gets those blocks, each with a reference of its own;
  * insert(tokens, table): each missing whole-block prefix gets the
    caller's block (the cache takes a reference); prefixes already cached
    keep their block;
  * evict(n): up to n times, drop the entry reached least recently (ties
    by block id) among those with no cached extension whose block only the
    cache references.
"""
BLOCK = 16


class PrefixCacheModel:
    def __init__(self, alloc):
        self.alloc = alloc
        self.entries = {}      # prefix tuple -> [block, tick]
        self.children = {}     # prefix tuple -> number of cached one-block extensions
        self.tick = 0

    def cached_blocks(self):
        return len(self.entries)

    def match(self, tokens, max_blocks):
        self.tick += 1
        want = min(len(tokens) // BLOCK, max_blocks)
        out = []
        for k in range(want):
            key = tuple(tokens[:BLOCK * (k + 1)])
            e = self.entries.get(key)
            if e is None:
                break
            self.alloc.incref(e[0])
            e[1] = self.tick
            out.append(e[0])
        return out

    def insert(self, tokens, table):
        self.tick += 1
        want = min(len(tokens) // BLOCK, len(table))
        added = 0
        for k in range(want):
            key = tuple(tokens[:BLOCK * (k + 1)])
            e = self.entries.get(key)
            if e is None:
                self.alloc.incref(table[k])
                self.entries[key] = [table[k], self.tick]
                self.children[key] = 0
                if k > 0:
                    self.children[tuple(tokens[:BLOCK * k])] += 1
                added += 1
            else:
                e[1] = self.tick
        return added

    def evict(self, n):
        freed = 0
        while freed < n:
            best = None
            for key, (blk, tick) in self.entries.items():
                if self.children[key] == 0 and self.alloc.refcount[blk] == 1:
                    if best is None or (tick, blk) < (self.entries[best][1], self.entries[best][0]):
                        best = key
            if best is None:
                break
            self.alloc.decref(self.entries[best][0])
            del self.entries[best]
            del self.children[best]
            if len(best) > BLOCK:
                self.children[best[:-BLOCK]] -= 1
            freed += 1
        return freed
