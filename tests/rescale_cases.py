"""Inputs whose scores rise and fall by many log2 units along a sequence.

The kernels keep a running reference maximum per query row and rescale the
running sum and accumulator only when a tile's maximum exceeds it by more
than a slack of 8 log2 units; the merge weights each partial by
2^(m_p - max). With N(0, 1) queries and keys at scale 1/sqrt(d) the scores
stay within a few units, so neither the rescale of a live accumulator nor
a merge over far-apart maxima would ever run. These cases make them run.

Construction: every query's dimension 0 is set to 1.0 and b(s, t) / scale
is added to dimension 0 of the key at position t of sequence s (rounded to
bf16; both sides read the same bits). A row's score at t is then b(s, t)
plus a noise term from the other dimensions. Profiles, in
natural-log units of the score:

  late_jump   0 everywhere, then J tokens of the sequence's last tile at a
              level L chosen so that they carry about as much softmax mass
              as the rest of the context: a wrong rescale of the live
              accumulator changes the output by O(1).
  early_peak  J tokens of the first tile at such a level, 0 afterwards:
              every later partial's maximum lies ~13 log2 units below the
              first one's, with balanced mass.
  staircase   7 units higher every T tokens: a rescale at every step, and
              partial maxima hundreds of log2 units apart.
  scale_*     no offsets, a large softmax scale (1, 8/sqrt(d), 100): random
              rescales; at 100 the softmax is nearly an argmax.

The other query dimensions are scaled by 1/4 in the offset profiles, so
the score noise is small beside the levels (the premises below then hold
by a margin), and values get +1 on low tokens and -1 on raised ones (the
staircase: alternating signs per step), so the output is far from what it
would be if either part's weight were wrong.

For a shared prefix the offsets of prefix positions depend on the position
only (the blocks are shared); after the prefix they are per sequence.

Test infrastructure: host-side input shaping plus the float64 scores the
premise checks use. It holds no attention result and imports neither the
oracle nor the GPU library.
"""
import math

import numpy as np

import workload as w

LOG2E = 1.4426950408889634
SLACK = 8.0            # log2 units the kernels let a tile maximum exceed the reference
PROFILES = ("late_jump", "early_peak", "staircase", "scale_1", "scale_8", "scale_100")


def profile_scale(profile, d):
    """The softmax scale a profile runs at."""
    if profile == "scale_1":
        return 1.0
    if profile == "scale_8":
        return 8.0 / math.sqrt(d)
    if profile == "scale_100":
        return 100.0
    return 1.0 / math.sqrt(d)


def _level(n_low, n_high):
    """A level (natural units) at which n_high tokens weigh about as much as
    n_low tokens of scores near 0 (their noise has standard deviation 1/4),
    and at least 9.5, so that the raised tokens clear the slack above any
    tile of the low part by about 3 log2 units."""
    return max(9.5, math.log(max(n_low, 1) / n_high))


def offsets(profile, ctx, g, prefix_len=0, prefix_profile=None):
    """b(t) for t < ctx of one sequence (float64, natural units). With
    prefix_len > 0, positions below it take prefix_profile(t) instead."""
    b = np.zeros(ctx)
    last0 = 16 * ((ctx - 1) // 16)
    if profile == "late_jump":
        n_last = ctx - last0
        j = int(g.integers(1, min(3, n_last) + 1))
        pos = last0 + g.choice(n_last, size=j, replace=False)
        b[pos] = _level(ctx - j, j) + g.uniform(-0.3, 0.3)
    elif profile == "early_peak":
        j = int(g.integers(1, min(3, ctx) + 1))
        pos = g.choice(min(16, ctx), size=j, replace=False)
        b[pos] = _level(ctx - j, j) + g.uniform(-0.3, 0.3)
    elif profile == "staircase":
        step = int(g.choice([48, 64, 160]))
        b = 7.0 * (np.arange(ctx) // step)
    if prefix_len > 0 and prefix_profile is not None:
        n = min(prefix_len, ctx)
        b[:n] = prefix_profile[:n]
    return b


def apply_offsets(k_pool, k_new, tables, offs, scale, append):
    """Add offs[s][t] / scale to dimension 0 of every key of sequence s
    (through its table; position ctx - 1 goes to k_new when append is set).
    Shared blocks get the same value from every sharer, as offs is then a
    function of the position only there."""
    orig = k_pool.copy()
    inv = 1.0 / scale
    for s, ctx in enumerate(tables.context_lens):
        ctx = int(ctx)
        b = offs[s]
        n_pool = ctx - 1 if append else ctx
        for t in range(n_pool):
            if b[t] == 0.0:
                continue
            blk = tables.block_tables[s, t // w.BLOCK]
            base = w.bf16_to_f32(orig[blk, :, t % w.BLOCK, 0]).astype(np.float64)
            k_pool[blk, :, t % w.BLOCK, 0] = w.bf16_bits((base + b[t] * inv).astype(np.float32))
        if append and b[ctx - 1] != 0.0:
            base = w.bf16_to_f32(k_new[s, :, 0]).astype(np.float64)
            k_new[s, :, 0] = w.bf16_bits((base + b[ctx - 1] * inv).astype(np.float32))


def set_query_dim0(q):
    """Dimension 0 of every query row = 1.0 (bf16 0x3F80)."""
    q[..., 0] = 0x3F80


def keys_of(k_pool, k_new, tables, s, append):
    """Contiguous float64 keys [n_kv, ctx, d] of sequence s as the kernels
    see them (the appended token from k_new)."""
    ctx = int(tables.context_lens[s])
    nb = -(-ctx // w.BLOCK)
    ids = tables.block_tables[s, :nb]
    k = k_pool[ids]                                   # [nb, h, 16, d]
    k = np.transpose(k, (1, 0, 2, 3)).reshape(k.shape[1], nb * w.BLOCK, k.shape[3])[:, :ctx]
    k = w.bf16_to_f32(np.ascontiguousarray(k)).astype(np.float64)
    if append:
        k[:, ctx - 1, :] = w.bf16_to_f32(k_new[s]).astype(np.float64)
    return k


def scores_log2(q_rows, keys, scale):
    """Scores of query rows [R, d] against keys [ctx, d], in log2 units."""
    return (q_rows.astype(np.float64) @ keys.T) * (scale * LOG2E)


def tile_max(x, lim=None):
    """Per-tile maxima (log2 units) of one row's scores x [ctx]; positions
    past lim (inclusive bound) are excluded. -inf for a tile it cannot see."""
    ctx = x.shape[0]
    if lim is not None:
        x = np.where(np.arange(ctx) <= lim, x, -np.inf)
    nt = -(-ctx // w.BLOCK)
    pad = np.full(nt * w.BLOCK, -np.inf)
    pad[:ctx] = x
    return pad.reshape(nt, w.BLOCK).max(axis=1)


def live_rescales(tm):
    """Tiles (index >= 1) whose maximum exceeds the maximum of every earlier
    tile by more than the slack: whatever tile a segment starts at, its
    reference is then below the tile's maximum minus the slack, so a
    segment holding this tile and an earlier one rescales a non-zero
    accumulator there."""
    run = np.maximum.accumulate(tm)
    return [i for i in range(1, len(tm)) if tm[i] > run[i - 1] + SLACK + 0.25]


def partition_spans(tm, tiles_per_part):
    """Largest minus smallest partition maximum (log2 units) of one row for
    fixed partitions of tiles_per_part tiles (partitions it cannot see
    excluded)."""
    n = len(tm)
    maxima = [tm[i:i + tiles_per_part].max() for i in range(0, n, tiles_per_part)]
    maxima = [m for m in maxima if np.isfinite(m)]
    return max(maxima) - min(maxima) if len(maxima) > 1 else 0.0


def segments(nts, n_hq, n_waves):
    """The balanced split's segments: for every unit (row hq, sequence s) the
    runs of its tiles that one wave processes, as (hq, s, ta, tb). Wave of
    tile x of the (row, sequence, tile) order: floor(((x+1) W - 1) / T)."""
    per_row = int(sum(nts))
    total = n_hq * per_row
    out = []
    before = np.concatenate([[0], np.cumsum(nts)[:-1]]).astype(np.int64)
    for hq in range(n_hq):
        for s, nt in enumerate(nts):
            if nt == 0:
                continue
            x = hq * per_row + before[s] + np.arange(nt, dtype=np.int64)
            wv = ((x + 1) * n_waves - 1) // total
            cut = np.flatnonzero(np.diff(wv)) + 1
            edges = [0, *cut.tolist(), int(nt)]
            for a, b in zip(edges[:-1], edges[1:]):
                out.append((hq, s, a, b))
    return out


def top_gap(x):
    """Gap (natural units) between a row's largest and second largest score
    (x in log2 units)."""
    if x.shape[0] < 2:
        return math.inf
    top = np.partition(x, -2)[-2:]
    return float(top[1] - top[0]) / LOG2E


def value_offsets(profile, b):
    """Per-position value offset for an offset profile (0 for scale_*)."""
    if profile in ("late_jump", "early_peak"):
        return np.where(b > 0, -1.0, 1.0)
    if profile == "staircase":
        return np.where(np.rint(b / 7.0).astype(np.int64) % 2 == 0, 1.0, -1.0)
    return np.zeros_like(b)


def apply_value_offsets(v_pool, v_new, tables, voffs, append):
    """Add voffs[s][t] to every dimension of the value at position t of
    sequence s (dim-major V tiles; position ctx - 1 goes to v_new when
    append is set)."""
    orig = v_pool.copy()
    for s, ctx in enumerate(tables.context_lens):
        ctx = int(ctx)
        vo = voffs[s]
        n_pool = ctx - 1 if append else ctx
        for t in range(n_pool):
            if vo[t] == 0.0:
                continue
            blk = tables.block_tables[s, t // w.BLOCK]
            base = w.bf16_to_f32(orig[blk, :, :, t % w.BLOCK]).astype(np.float64)
            v_pool[blk, :, :, t % w.BLOCK] = w.bf16_bits((base + vo[t]).astype(np.float32))
        if append and vo[ctx - 1] != 0.0:
            base = w.bf16_to_f32(v_new[s]).astype(np.float64)
            v_new[s] = w.bf16_bits((base + vo[ctx - 1]).astype(np.float32))


def shrink_query_noise(q):
    """Query dimensions 1 .. d-1 times 1/4 (exact in bf16: an exponent step,
    away from the subnormal range for these draws)."""
    x = w.bf16_to_f32(q[..., 1:]) * np.float32(0.25)
    q[..., 1:] = w.bf16_bits(x)


class Case:
    """One input set: a workload.HostCase with the keys, values and queries
    shaped for a profile, the scale it runs at, and (verification pass,
    prefill) the multi-token queries."""

    def __init__(self, hc, profile, scale, offs, qv=None, append=True):
        self.hc, self.profile, self.scale, self.offs = hc, profile, scale, offs
        self.qv = qv
        self.append = append


def _shape(name, n_q, n_kv, d, prefix_tokens=0):
    return w.Shape(name, 1, n_q, n_kv, d, 1, 1, 1, prefix_tokens=prefix_tokens)


def build(profile, n_q, n_kv, d, ctxs, seed, append=True, q_len=0, prefix_blocks=0,
          max_blocks=None):
    """A case for the decode (q_len = 0: one query per sequence, appended
    token in k_new / v_new when append is set), or for the verification
    pass / chunked prefill (q_len query tokens per sequence, all cached)."""
    shape = _shape(f"{profile} {seed}", n_q, n_kv, d, 16 * prefix_blocks)
    mb = max_blocks or -(-max(ctxs) // w.BLOCK)
    hc = w.host_case(shape, 77000 + seed, context_lens=ctxs, share=True, max_blocks=mb)
    g = np.random.default_rng([77001, seed])
    scale = profile_scale(profile, d)
    shaped = not profile.startswith("scale_")
    pre_len = 16 * prefix_blocks
    pre_prof = None
    if pre_len:
        # offsets of the shared positions: a function of the position only
        pre_prof = offsets(profile, pre_len, g) if profile != "late_jump" else np.zeros(pre_len)
    offs = [offsets(profile, int(c), g, pre_len, pre_prof) if shaped else np.zeros(int(c))
            for c in ctxs]
    append = append and q_len == 0
    qv = None
    if q_len:
        qv = w.normal_bf16(g, (len(ctxs), q_len, n_q, d))
    if shaped:
        apply_offsets(hc.k_pool, hc.k_new, hc.tables, offs, scale, append)
        apply_value_offsets(hc.v_pool, hc.v_new, hc.tables,
                            [value_offsets(profile, b) for b in offs], append)
        shrink_query_noise(hc.q)
        set_query_dim0(hc.q)
        if qv is not None:
            shrink_query_noise(qv)
            set_query_dim0(qv)
    return Case(hc, profile, scale, offs, qv, append)


def row_scores(case, s, j, i=None):
    """Scores (log2 units) of query head j of sequence s (token i of a
    multi-token query) over the sequence's context, and the row's causal
    limit (None for the decode)."""
    hc = case.hc
    G = hc.shape.n_q // hc.shape.n_kv
    keys = keys_of(hc.k_pool, hc.k_new, hc.tables, s, case.append)[j // G]
    if case.qv is None:
        q = w.bf16_to_f32(hc.q[s, j]).astype(np.float64)
        lim = None
    else:
        q = w.bf16_to_f32(case.qv[s, i, j]).astype(np.float64)
        ctx = int(hc.tables.context_lens[s])
        lim = ctx - case.qv.shape[1] + i
    return scores_log2(q[None, :], keys, case.scale)[0], lim


def verify_geometry(q_len, n_q, n_kv):
    """Row groups per KV head of the verification pass: 32-row groups when
    a KV head has more than 16 query rows (q_len x group), else one."""
    qrows = q_len * (n_q // n_kv)
    group_rows = 32 if qrows > 16 else 16
    return -(-qrows // group_rows)


def split_waves_cap(units, max_ctx, min_tiles=16, max_waves=8192):
    """The balanced split's wave count when the GPU holds more resident
    waves than this: one wave per min_tiles tiles of the upper bound."""
    return max(1, min(max_waves, -(-units * (-(-max_ctx // 16)) // min_tiles)))


def blind_segments(ctxs, q_len, n_q, n_kv, max_ctx):
    """Segments of the verification pass's split that hold only a unit's
    last tile while that tile holds only position ctx - 1 (ctx = 1 mod 16):
    every query token but the last sees nothing in them, so their partials
    carry maximum -inf and sum 0."""
    nts = [-(-c // 16) for c in ctxs]
    n_hq = n_kv * verify_geometry(q_len, n_q, n_kv)
    W = split_waves_cap(n_hq * len(ctxs), max_ctx)
    out = []
    for hq, s, a, b in segments(nts, n_hq, W):
        if a == nts[s] - 1 and b == nts[s] and a >= 1 and ctxs[s] % 16 == 1:
            out.append((hq, s))
    return out, W


# ---------------------------------------------------------------------------
# the cases the tests run (each a tuple the GPU test and the premise test
# rebuild identically)

DECODE_PATHS = ("fused", "unfused", "halves", "fixed16", "fixed64")
DECODE_SHAPES = {
    "g4d128": (32, 8, 128, 5, 1500, 4200),    # n_q, n_kv, d, batch, ctx range
    "g5d64": (20, 4, 64, 6, 600, 2500),
    "g8d128long": (64, 8, 128, 2, 8000, 8000),
}


def decode_specs():
    """(profile, path, shape name, seed): every profile through every decode
    path, the two shapes alternating, and three long-context cases."""
    out = []
    i = 0
    for profile in PROFILES:
        for path in DECODE_PATHS:
            out.append((profile, path, "g4d128" if i % 2 == 0 else "g5d64", i))
            i += 1
    for profile in ("late_jump", "staircase", "scale_8"):
        out.append((profile, "fused", "g8d128long", i))
        i += 1
    return out


def decode_case(profile, shape_name, seed):
    n_q, n_kv, d, B, lo, hi = DECODE_SHAPES[shape_name]
    g = np.random.default_rng([77002, seed])
    ctxs = [int(c) for c in g.integers(lo, hi, size=B, endpoint=True)]
    return build(profile, n_q, n_kv, d, ctxs, seed)


def verify_specs():
    """(profile, q_len, d, seed) for the verification pass."""
    out = []
    i = 100
    for profile in PROFILES:
        for q_len, d in ((5, 128), (20, 64), (33, 128)):
            out.append((profile, q_len, d, i))
            i += 1
    return out


def verify_case(profile, q_len, d, seed):
    """Four sequences, contexts drawn until the split holds a segment that
    no query token but the last can see into (a -inf partial)."""
    n_q, n_kv = 8, 2
    g = np.random.default_rng([77003, seed])
    for _ in range(2000):
        ctxs = []
        for _ in range(4):
            c = int(g.integers(max(q_len + 1, 40), 1000))
            if g.random() < 0.6:
                c = 16 * (c // 16) + 1
            ctxs.append(max(c, q_len))
        blind, _ = blind_segments(ctxs, q_len, n_q, n_kv, max(ctxs))
        if blind:
            break
    else:
        raise AssertionError("no context mix with a blind segment")
    return build(profile, n_q, n_kv, d, ctxs, seed, q_len=q_len)


def prefill_specs():
    """(profile, chunk, d, seed) for chunked prefill."""
    out = []
    i = 200
    for profile in PROFILES:
        for chunk, d in ((64, 128), (96, 64)):
            out.append((profile, chunk, d, i))
            i += 1
    return out


def prefill_case(profile, chunk, d, seed):
    n_q, n_kv = (8, 2) if d == 128 else (10, 2)
    g = np.random.default_rng([77004, seed])
    ctxs = [chunk + int(g.integers(0, 1500)) for _ in range(2)]
    return build(profile, n_q, n_kv, d, ctxs, seed, q_len=chunk)


def prefix_specs():
    """(profile, d, seed) for the shared-prefix step."""
    return [(profile, d, 300 + 2 * i + (d == 64)) for i, profile in enumerate(PROFILES)
            for d in (128, 64)]


def prefix_case(profile, d, seed):
    """A 12-block prefix shared by every sequence longer than it (members
    0 .. 5), plus two sequences that end inside it."""
    n_q, n_kv = (32, 8) if d == 128 else (20, 4)
    g = np.random.default_rng([77005, seed])
    pre = 12
    ctxs = [16 * pre + int(g.integers(200, 1500)) for _ in range(6)]
    ctxs += [int(g.integers(1, 16 * pre + 1)) for _ in range(2)]
    return build(profile, n_q, n_kv, d, ctxs, seed, prefix_blocks=pre), pre, 0, 6


def conditioned_rows(case):
    """Boolean [num_seqs, (q_len,) n_q]: the rows compared element by
    element. At scale 100 the softmax is nearly an argmax, and where a
    row's two largest scores lie within 6 natural units the fp32 rounding
    of the scores (about 1e-3 units there) could move its output by more
    than the tolerance: those rows are left out (the tests count them)."""
    hc = case.hc
    B, n_q = hc.q.shape[0], hc.shape.n_q
    if case.qv is None:
        keep = np.ones((B, n_q), dtype=bool)
        if case.profile != "scale_100":
            return keep
        for s in range(B):
            for j in range(n_q):
                keep[s, j] = top_gap(row_scores(case, s, j)[0]) >= 6.0
        return keep
    q_len = case.qv.shape[1]
    keep = np.ones((B, q_len, n_q), dtype=bool)
    if case.profile != "scale_100":
        return keep
    for s in range(B):
        for i in range(q_len):
            for j in range(n_q):
                x, lim = row_scores(case, s, j, i)
                keep[s, i, j] = top_gap(x[:lim + 1]) >= 6.0
    return keep
