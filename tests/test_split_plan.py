"""The balanced split's index arithmetic, restated on the CPU (no GPU).

The decode kernel cuts all tiles of a call, in (KV head, query group,
sequence, tile) order, into W equal ranges, one per wavefront; a wavefront
leaves one partial per unit (head, group, sequence) its range touches, in
slot wave + unit, and the merge kernel combines a unit's partials. With a
shared prefix (run_prefix below) the prefix units, one per (KV head, 32
member rows) over the prefix's tiles, are split by their own class of
waves, and a member's own unit holds only its tiles after the prefix.
This model follows the same integer formulas and checks, for random mixes
of context lengths (invalid ones included), head counts and wave counts
(more waves than tiles included), that:
  * every tile is processed exactly once;
  * no two partials share a slot, and every slot is below W + units;
  * the merge of a unit reads exactly the slots of its wavefronts, whose
    tiles add up to the unit's, and reads no unwritten slot;
  * the number of partials written for a unit equals the number merged, and
    units written directly have none.
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


def run_prefix(ctxs, max_ctx, n_kv, group, W, pre_tiles, first, count, cost=(2, 3), q_len=1):
    """The split with prefix units: the decode's (pkv_decode_step_prefix,
    q_len 1) or the verification pass's (pkv_paged_attn_verify_prefix, q_len
    query tokens, causal): the same integer formulas as the kernel, checked
    like run(). A KV head's q_len * group rows form row groups of 16 (of 32
    when there are more than 16); a member whose query tokens all lie after
    the prefix reads it through prefix units of 32 rows. With a prefix and
    two or more waves the waves form two classes, the last Wp splitting the
    prefix units' tiles; with one wave a single order holds both."""
    B = len(ctxs)
    qrows = q_len * group
    group_rows = 32 if qrows > 16 else 16
    n_qgroups = (qrows + group_rows - 1) // group_rows
    n_hq = n_kv * n_qgroups

    def tiles(c):
        return (c + 15) // 16 if q_len <= c <= max_ctx else 0

    def skip(s):
        c = ctxs[s]
        return pre_tiles if (pre_tiles > 0 and first <= s < first + count and tiles(c) > 0 and
                             c - q_len >= 16 * pre_tiles) else 0

    unit_t = [tiles(ctxs[s]) - skip(s) if tiles(ctxs[s]) else 0 for s in range(B)]
    per_row = sum(unit_t)
    t_seq = n_hq * per_row
    qgroups = (count * qrows + 31) // 32 if pre_tiles > 0 and count > 0 else 0
    pre_units = n_kv * qgroups
    t_pre = pre_units * pre_tiles
    if t_seq + t_pre == 0:
        return
    w_pre = 0
    if t_pre > 0 and W >= 2:
        if t_seq == 0:
            w_pre = W
        else:
            num = W * cost[0] * t_pre
            den = t_seq * cost[1] + cost[0] * t_pre
            w_pre = max(1, min(W - 1, (num + den // 2) // den))
    # global tile index: the sequences' tiles, then the prefix units'
    covered = [0] * (t_seq + t_pre)
    seq_writes, pre_writes = {}, {}
    direct = set()

    def span(w):
        pre_class = w_pre > 0 and w >= W - w_pre
        total = t_seq + t_pre if w_pre == 0 else (t_pre if pre_class else t_seq)
        waves = W if w_pre == 0 else (w_pre if pre_class else W - w_pre)
        base = W - w_pre if pre_class else 0
        origin = 0 if pre_class else t_seq
        return total, waves, base, origin

    def locate(r):
        acc = 0
        for s in range(B):
            if acc + unit_t[s] > r:
                return s, acc
            acc += unit_t[s]
        raise AssertionError

    def prefix_walk(w, c, end, origin):
        pu = (c - origin) // pre_tiles
        pos = (c - origin) - pu * pre_tiles
        while c < end:
            assert pu < pre_units
            tb = min(pre_tiles, pos + (end - c))
            for t in range(pos, tb):
                covered[t_seq + pu * pre_tiles + t] += 1
            slot = w + pu
            assert slot not in pre_writes, ("dup prefix slot", slot)
            pre_writes[slot] = (pu, tb - pos)
            c += tb - pos
            pos = 0
            pu += 1

    for w in range(W):
        total, waves, base, origin = span(w)
        cur = total * (w - base) // waves
        end = total * (w - base + 1) // waves
        if cur >= end:
            if cur < origin:
                hq = cur // per_row
                s, before = locate(cur - hq * per_row)
                if cur - hq * per_row != before:
                    slot = w + hq * B + s
                    assert slot not in seq_writes
                    seq_writes[slot] = (hq * B + s, 0)
            elif cur < total:
                pu = (cur - origin) // pre_tiles
                if cur - origin != pu * pre_tiles:
                    slot = w + pu
                    assert slot not in pre_writes
                    pre_writes[slot] = (pu, 0)
            continue
        if cur >= origin:
            prefix_walk(w, cur, end, origin)
            continue
        hq = cur // per_row
        s, before = locate(cur - hq * per_row)
        pos = cur - hq * per_row - before
        while True:
            nt = unit_t[s]
            assert 0 <= pos < nt
            tb = min(nt, pos + (end - cur))
            u = hq * B + s
            base_t = hq * per_row + sum(unit_t[:s])
            for t in range(pos, tb):
                covered[base_t + t] += 1
            if pos == 0 and tb == nt and skip(s) == 0:
                direct.add(u)
            else:
                slot = w + u
                assert slot not in seq_writes, ("dup", slot)
                seq_writes[slot] = (u, tb - pos)
            cur += tb - pos
            if cur >= end:
                break
            pos = 0
            done = False
            while True:
                s += 1
                if s == B:
                    s = 0
                    hq += 1
                    if hq >= n_hq:
                        done = True
                        break
                if unit_t[s]:
                    break
            if done:
                assert w_pre == 0
                prefix_walk(w, cur, end, origin)
                break
    assert all(c == 1 for c in covered), "coverage"
    assert max(seq_writes, default=0) < W + n_hq * B
    assert max(pre_writes, default=0) < W + pre_units
    # merge side: the bookkeeping the kernel writes (first slot, count) per
    # unit, from the unit's span; the slots hold exactly the unit's tiles
    seq_span = span(0)
    pre_span = span(W - 1)
    for hq in range(n_hq):
        h, qg = divmod(hq, n_qgroups)
        for s in range(B):
            nt = unit_t[s]
            if nt == 0:
                continue
            u = hq * B + s
            total, waves, _, _ = seq_span
            t0 = hq * per_row + sum(unit_t[:s])
            w0 = ((t0 + 1) * waves - 1) // total
            w1 = ((t0 + nt) * waves - 1) // total
            n = w1 - w0 + 1
            if n <= 1 and skip(s) == 0:
                assert u in direct
                continue
            slots = [w0 + u + p for p in range(n)]
            assert all(seq_writes.get(sl, (None,))[0] == u for sl in slots), ("slots", u)
            assert sum(seq_writes[sl][1] for sl in slots) == nt
            if skip(s):
                total, waves, base, origin = pre_span if w_pre else seq_span
                for gr in range(qg * group_rows, min(qrows, (qg + 1) * group_rows)):
                    pr = (s - first) * qrows + gr
                    pu = h * qgroups + pr // 32
                    x0 = origin + pu * pre_tiles
                    p0 = ((x0 + 1) * waves - 1) // total
                    p1 = ((x0 + pre_tiles) * waves - 1) // total
                    pslots = [base + p0 + pu + p for p in range(p1 - p0 + 1)]
                    assert all(pre_writes.get(sl, (None,))[0] == pu for sl in pslots), ("pre slots", pu)
                    assert sum(pre_writes[sl][1] for sl in pslots) == pre_tiles


def test_split_with_prefix_units():
    rnd = random.Random(1)
    n_cases = 0
    for _ in range(1500):
        B = rnd.randint(1, 40)
        pre_tiles = rnd.choice([1, 2, 5, 16, 40])
        max_ctx = rnd.choice([16 * pre_tiles + 1, 16 * pre_tiles + 200, 3000])
        ctxs = [rnd.choice([0, 1, rnd.randint(1, max_ctx), max_ctx, 16 * pre_tiles,
                            16 * pre_tiles + 1]) for _ in range(B)]
        n_kv = rnd.randint(1, 8)
        group = rnd.choice([1, 4, 5, 8, 16])
        first = rnd.randint(0, B - 1)
        count = rnd.randint(0, B - first)
        W = rnd.choice([1, 2, 3, 64, 1000, rnd.randint(1, 2000)])
        cost = rnd.choice([(2, 3), (1, 2), (1, 1), (1, 5)])
        run_prefix(ctxs, max_ctx, n_kv, group, W, pre_tiles, first, count, cost)
        n_cases += 1
    assert n_cases == 1500


def test_verify_split_with_prefix_units():
    """The verification pass's split with prefix units: q_len query tokens
    per member, row groups of 32 when a KV head has more than 16 rows,
    members only if their query tokens all lie after the prefix."""
    rnd = random.Random(2)
    for _ in range(1000):
        B = rnd.randint(1, 30)
        q_len = rnd.choice([1, 2, 5, 12, 33, 64])
        pre_tiles = rnd.choice([1, 2, 5, 16, 40])
        max_ctx = rnd.choice([16 * pre_tiles + q_len, 16 * pre_tiles + 200, 3000])
        ctxs = [rnd.choice([0, q_len - 1, q_len, rnd.randint(1, max_ctx), max_ctx,
                            16 * pre_tiles + q_len - 1, 16 * pre_tiles + q_len])
                for _ in range(B)]
        n_kv = rnd.randint(1, 8)
        group = rnd.choice([1, 4, 5, 8, 16])
        first = rnd.randint(0, B - 1)
        count = rnd.randint(0, B - first)
        W = rnd.choice([1, 2, 3, 64, 1000, rnd.randint(1, 2000)])
        cost = rnd.choice([(2, 3), (1, 2), (1, 1)])
        run_prefix(ctxs, max_ctx, n_kv, group, W, pre_tiles, first, count, cost, q_len)
