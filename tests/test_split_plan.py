"""The balanced split's index arithmetic, restated on the CPU (no GPU).

The decode kernel cuts all tiles of a call, in (KV head, query group,
sequence, tile) order, into W equal ranges, one per wavefront; a wavefront
leaves one partial per unit (head, group, sequence) its range touches, in
slot wave + unit, and the last of a unit's wavefronts to arrive merges them.
This model follows the same integer formulas and checks, for random mixes
of context lengths (invalid ones included), head counts and wave counts
(more waves than tiles included), that:
  * every tile is processed exactly once;
  * no two partials share a slot, and every slot is below W + units;
  * the merge of a unit reads exactly the slots of its wavefronts, whose
    tiles add up to the unit's, and reads no unwritten slot;
  * the arrival count of a unit equals the number of partials merged, and
    units written directly see no arrival.
"""
import random

def seq_tiles(ctx, max_ctx):
    return (ctx + 15) // 16 if 1 <= ctx <= max_ctx else 0

def run(ctxs, max_ctx, n_hq, W):
    B = len(ctxs)
    per_row = sum(seq_tiles(c, max_ctx) for c in ctxs)
    total = n_hq * per_row
    writes = {}   # slot -> (unit, kind, tiles)
    arrivals = {} # unit -> waves that arrive (fused merge)
    covered = [0] * total
    def locate(r):
        acc = 0
        for s in range(B):
            n = seq_tiles(ctxs[s], max_ctx)
            if acc + n > r:
                return s, acc
            acc += n
        raise AssertionError
    direct = set()
    for w in range(W):
        cur = total * w // W
        end = total * (w + 1) // W
        if cur >= end:
            if cur < total:
                hq = cur // per_row
                s, before = locate(cur - hq * per_row)
                if cur - hq * per_row == before:
                    continue          # at a unit's first tile: belongs to no unit
                u = hq * B + s
                slot = w + u
                assert slot not in writes, ("dup neutral", slot)
                writes[slot] = (u, "neutral", 0)
                arrivals[u] = arrivals.get(u, 0) + 1
            continue
        hq = cur // per_row
        s, before = locate(cur - hq * per_row)
        pos = cur - hq * per_row - before
        while True:
            nt = seq_tiles(ctxs[s], max_ctx)
            assert 0 <= pos < nt
            tb = min(nt, pos + (end - cur))
            u = hq * B + s
            base = hq * per_row + sum(seq_tiles(c, max_ctx) for c in ctxs[:s])
            for t in range(pos, tb):
                covered[base + t] += 1
            if pos == 0 and tb == nt:
                assert u not in direct
                direct.add(u)
            else:
                slot = w + u
                assert slot not in writes, ("dup", slot)
                writes[slot] = (u, "partial", tb - pos)
                arrivals[u] = arrivals.get(u, 0) + 1
            cur += tb - pos
            if cur >= end:
                break
            pos = 0
            while True:
                s += 1
                if s == B:
                    s = 0
                    hq += 1
                if seq_tiles(ctxs[s], max_ctx):
                    break
            assert hq < n_hq
    assert all(c == 1 for c in covered), "coverage"
    # merge side
    slots_used = set()
    for hq in range(n_hq):
        for s in range(B):
            nt = seq_tiles(ctxs[s], max_ctx)
            u = hq * B + s
            if nt == 0:
                continue
            before = sum(seq_tiles(c, max_ctx) for c in ctxs[:s])
            t0 = hq * per_row + before
            t1 = t0 + nt
            w0 = ((t0 + 1) * W - 1) // total
            w1 = (t1 * W - 1) // total
            n = w1 - w0 + 1
            if n <= 1:
                assert u in direct, ("not direct", u)
                assert u not in arrivals, ("arrival at a direct unit", u)
                continue
            assert u not in direct
            assert arrivals.get(u, 0) == n, ("arrivals", u, arrivals.get(u), n)
            got = 0
            for p in range(n):
                slot = w0 + u + p
                assert slot in writes and writes[slot][0] == u, ("merge reads unwritten/foreign slot", slot, u, writes.get(slot))
                got += writes[slot][2]
                slots_used.add(slot)
            assert got == nt, ("tiles", got, nt)
    assert max(writes, default=0) < W + n_hq * B, "slot bound"
    # every partial is read by exactly one merge
    for slot, (u, kind, _) in writes.items():
        if kind == "partial":
            assert slot in slots_used, ("partial never merged", slot)



def test_split_index_arithmetic():
    rnd = random.Random(0)
    n_cases = 0
    for _ in range(3000):
        B = rnd.randint(1, 70)
        max_ctx = rnd.choice([16, 17, 100, 512, 2000])
        ctxs = [rnd.choice([0, 1, rnd.randint(1, max_ctx), max_ctx, max_ctx + 1]) for _ in range(B)]
        n_hq = rnd.randint(1, 9)
        per_row = sum(seq_tiles(c, max_ctx) for c in ctxs)
        if per_row == 0:
            continue
        W = rnd.choice([1, 2, 3, 7, 64, 200, 1000, rnd.randint(1, 3 * n_hq * per_row + 5)])
        run(ctxs, max_ctx, n_hq, W)
        n_cases += 1
    assert n_cases > 2500


def test_many_more_waves_than_tiles():
    """Units of one tile each with a thousand waves: most waves are empty,
    many sit at a unit's first tile and must not join its merge."""
    run([1, 2, 3], 16384, 8, 1024)
    run([1] * 64, 100, 8, 8192)
