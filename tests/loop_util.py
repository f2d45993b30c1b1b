"""Shared pieces of the continuous-batching tests (CPU and GPU): a request
workload, the keys/values of every token as a fixed function of
(layer, request, position), the host mirror of a plan and attention
recomputed from contiguous caches. Test infrastructure only."""
import numpy as np

import workload as w

L, N_Q, N_KV = 2, 8, 2
PREFIX = 20          # shared prefix tokens: one full block and 4 tokens of the next
MAX_BLOCKS = 24
NUM_BLOCKS = 24      # tight: growth outruns the admission reserve, requests are preempted
MAX_BATCH = 6


def requests(seed, n=14, prefix=PREFIX):
    """{id: (arrival step, prompt_len, gen_len, shares_prefix)}."""
    rnd = np.random.default_rng(seed)
    reqs = {}
    for rid in range(n):
        shares = bool(rnd.random() < 0.5)
        prompt = int(rnd.integers(prefix if shares else 1, 70))
        reqs[rid] = (int(rnd.integers(0, 30)), prompt, int(rnd.integers(10, 120)), shares)
    return reqs


class History:
    """Keys/values (bf16 bits) of every (layer, request, position): a
    request's own tokens are drawn once per (layer, request); positions
    below the prefix length of a sharing request are the prefix's. So a
    request that is preempted and recomputed gets the same keys and values
    back."""

    def __init__(self, d, shares, prefix=PREFIX):
        self.d = d
        self.shares = shares
        self.prefix = prefix
        self.pk = [w.normal_bf16(w.rng(7000 + l, 6), (prefix, N_KV, d)) for l in range(L)]
        self.pv = [w.normal_bf16(w.rng(7100 + l, 6), (prefix, N_KV, d)) for l in range(L)]
        self.cache = {}

    def _own(self, l, rid):
        key = (l, rid)
        if key not in self.cache:
            g = w.rng(1000 * l + rid, 5)
            shape = (16 * MAX_BLOCKS, N_KV, self.d)
            self.cache[key] = (w.normal_bf16(g, shape), w.normal_bf16(g, shape))
        return self.cache[key]

    def kv(self, l, rid, positions):
        k, v = self._own(l, rid)
        pos = np.asarray(positions, dtype=np.int64)
        ks, vs = k[pos].copy(), v[pos].copy()
        if self.shares[rid]:
            pre = pos < self.prefix
            ks[pre] = self.pk[l][pos[pre]]
            vs[pre] = self.pv[l][pos[pre]]
        return ks, vs

    def fill(self, l, ids, plan):
        """Keys/values of the plan's fill tokens for layer l."""
        rows = np.asarray(plan.fill_rows)
        pos = np.asarray(plan.fill_positions)
        ks = np.empty((len(rows), N_KV, self.d), np.uint16)
        vs = np.empty_like(ks)
        for row in np.unique(rows):
            sel = rows == row
            ks[sel], vs[sel] = self.kv(l, ids[row], pos[sel])
        return ks, vs

    def new_token(self, l, ids, plan):
        """Keys/values of the token each row appends this step (at ctx-1)."""
        n = plan.num_seqs
        ks = np.empty((n, N_KV, self.d), np.uint16)
        vs = np.empty_like(ks)
        for r in range(n):
            k1, v1 = self.kv(l, ids[r], [int(plan.context_lens[r]) - 1])
            ks[r], vs[r] = k1[0], v1[0]
        return ks, vs



class TokenHistory(History):
    """Keys/values of requests given by token ids: those of position p are
    drawn from a seed that is a function of (layer, tokens[0..p]) only, as a
    model's are of the tokens it has seen. Two requests that start with the
    same tokens have the same keys and values there, so a block that one
    caches holds exactly what the other would write."""

    def __init__(self, d, tokens):
        self.d = d
        self.tokens = tokens            # {request id: prompt + generated tokens}
        self.cache = {}

    def _own(self, l, rid):
        key = (l, rid)
        if key not in self.cache:
            t = self.tokens[rid]
            ks = np.empty((len(t), N_KV, self.d), np.uint16)
            vs = np.empty_like(ks)
            for p in range(len(t)):
                g = np.random.default_rng([l] + [int(x) for x in t[:p + 1]])
                ks[p] = w.normal_bf16(g, (N_KV, self.d))
                vs[p] = w.normal_bf16(g, (N_KV, self.d))
            self.cache[key] = (ks, vs)
        return self.cache[key]

    def kv(self, l, rid, positions):
        k, v = self._own(l, rid)
        pos = np.asarray(positions, dtype=np.int64)
        return k[pos].copy(), v[pos].copy()


def mirror_step(orc, k_pool, v_pool, plan, fill, kn, vn, d):
    """The plan carried out on host pools with the oracle's operations, in
    the documented order: copies, prompt writes, append."""
    if len(plan.cow_src):
        assert orc.copy_blocks(k_pool, v_pool, plan.cow_src, plan.cow_dst, N_KV, d) == 0
    if len(plan.fill_rows):
        assert orc.kv_write(k_pool, v_pool, fill[0], fill[1], plan.block_tables, plan.fill_rows,
                            plan.fill_positions) == 0
    if plan.num_seqs:
        assert orc.kv_append(k_pool, v_pool, kn, vn, plan.block_tables, plan.context_lens) == 0


def contiguous_decode(orc, q, hist, l, ids, ctx, scale):
    """The oracle's attention over caches rebuilt contiguously (identity
    tables over a fresh pool) from each request's token history."""
    d = hist.d
    n = len(ids)
    nbs = [-(-int(c) // 16) for c in ctx]
    tables = np.full((n, max(nbs)), -1, np.int32)
    base = 0
    for r in range(n):
        tables[r, :nbs[r]] = np.arange(base, base + nbs[r])
        base += nbs[r]
    ck = np.full((base, N_KV, 16, d), w.BF16_NAN, np.uint16)
    cv = np.full((base, N_KV, d, 16), w.BF16_NAN, np.uint16)
    for r in range(n):
        tok = np.arange(int(ctx[r]))
        ks, vs = hist.kv(l, ids[r], tok)
        blk = tables[r, tok // 16]
        ck[blk, :, tok % 16, :] = ks
        cv[blk, :, :, tok % 16] = vs
    want, rc = orc.decode(q, ck, cv, tables, np.asarray(ctx, np.int32), N_KV, scale)
    assert rc == 0
    return want
