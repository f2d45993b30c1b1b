"""The rescale cases do what they are built for (CPU only, no GPU).

tests/test_gpu_rescale.py runs the decode, verification, prefill and
shared-prefix kernels on inputs from rescale_cases.py against the oracle.
That comparison only shows something about the online softmax's rescale
and the merge's weighting if those branches run. This file checks, from
the float64 scores of the same bytes and the split's own index formulas,
that they do:
  * a live rescale: a row's tile whose maximum exceeds every earlier tile
    of the same segment by more than the 8-log2-unit slack, so the kernel
    multiplies a non-zero accumulator and sum by 2^(m_old - m_new);
  * a far-apart merge: the partials of one row (the segments of its unit,
    or fixed partitions) whose maxima differ by many log2 units;
  * in the verification pass, a segment whose partial has maximum -inf
    for every query token but the last (weight 0 in the merge).
The split's wave count is the one the library launches when the GPU holds
more resident waves than the split's cap (true on an MI355X at these
sizes: at most 658 waves against 1,024 resident at head_dim 128, 2,048 at
64).
"""
import numpy as np
import pytest

import rescale_cases as rc
import workload as w


def _row_tms(case, s, tile_tokens=16):
    """Tile maxima [rows, tiles] of every query row of sequence s."""
    hc = case.hc
    n_q = hc.shape.n_q
    G = n_q // hc.shape.n_kv
    keys = rc.keys_of(hc.k_pool, hc.k_new, hc.tables, s, case.append)
    ctx = int(hc.tables.context_lens[s])
    nt = -(-ctx // tile_tokens)
    out = []
    q_len = 1 if case.qv is None else case.qv.shape[1]
    for i in range(q_len):
        q = (w.bf16_to_f32(hc.q[s]) if case.qv is None else w.bf16_to_f32(case.qv[s, i]))
        rows = []
        for j in range(n_q):
            xj = rc.scores_log2(q[j][None, :], keys[j // G], case.scale)[0]
            if case.qv is not None:
                xj = np.where(np.arange(ctx) <= ctx - q_len + i, xj, -np.inf)
            pad = np.full(nt * tile_tokens, -np.inf)
            pad[:ctx] = xj
            rows.append(pad.reshape(nt, tile_tokens).max(axis=1))
        out.append(np.stack(rows))
    return np.concatenate(out) if q_len > 1 else out[0]


def _live(tm, ta, tb):
    """Number of rows with a live rescale inside tiles [ta, tb)."""
    seg = tm[:, ta:tb]
    run = np.maximum.accumulate(seg, axis=1)
    fire = seg[:, 1:] > run[:, :-1] + rc.SLACK + 0.25
    return int(np.any(fire & np.isfinite(run[:, :-1]), axis=1).sum())


def _spans(tm, cuts):
    """Per row: largest minus smallest finite maximum over the segments
    [cuts[k], cuts[k+1])."""
    m = np.stack([tm[:, a:b].max(axis=1) for a, b in zip(cuts[:-1], cuts[1:])], axis=1)
    fin = np.where(np.isfinite(m), m, np.nan)
    return np.nanmax(fin, axis=1) - np.nanmin(fin, axis=1)


def _decode_segments(case, path):
    """Per sequence, the tile cuts of its unit's partials for one KV head
    (the first), or None when one wave covers the unit."""
    hc = case.hc
    ctxs = [int(c) for c in hc.tables.context_lens]
    nts = [-(-c // 16) for c in ctxs]
    if path.startswith("fixed"):
        per = int(path[5:]) // 16
        return {s: list(range(0, nts[s], per)) + [nts[s]] for s in range(len(ctxs))}
    n_hq = hc.shape.n_kv   # one 16-row group per KV head (group <= 16)
    W = rc.split_waves_cap(n_hq * len(ctxs), max(ctxs))
    cuts = {}
    for hq, s, a, b in rc.segments(nts, n_hq, W):
        if hq == 0:
            cuts.setdefault(s, [0]).append(b)
    return cuts


@pytest.mark.parametrize("profile,path,shape_name,seed", rc.decode_specs())
def test_decode_premise(profile, path, shape_name, seed):
    case = rc.decode_case(profile, shape_name, seed)
    G = case.hc.shape.n_q // case.hc.shape.n_kv
    cuts = _decode_segments(case, path)
    live = 0
    span = 0.0
    for s in range(len(case.hc.tables.context_lens)):
        tm = _row_tms(case, s)[:G]          # rows of KV head 0
        c = cuts[s]
        for a, b in zip(c[:-1], c[1:]):
            live += _live(tm, a, b)
        if len(c) > 2:
            span = max(span, float(np.nanmax(_spans(tm, c))))
    print(f"{profile} {path} {shape_name}: {live} live rescales, widest merge span {span:.1f}")
    if profile != "early_peak" and path != "fixed16":   # one tile per partial there
        assert live >= 1, "no row rescales a live accumulator"
    want_span = {"late_jump": 10.0, "early_peak": 10.0, "staircase": 30.0, "scale_100": 100.0}
    if profile in want_span:
        assert span >= want_span[profile], "partial maxima not far apart"


@pytest.mark.parametrize("profile,q_len,d,seed", rc.verify_specs())
def test_verify_premise(profile, q_len, d, seed):
    case = rc.verify_case(profile, q_len, d, seed)
    hc = case.hc
    ctxs = [int(c) for c in hc.tables.context_lens]
    blind, W = rc.blind_segments(ctxs, q_len, hc.shape.n_q, hc.shape.n_kv, max(ctxs))
    assert blind
    # those segments: the last tile, where only the last query token sees
    # anything
    for _, s in blind[:2]:
        tm = _row_tms(case, s)
        n_q = hc.shape.n_q
        assert np.all(np.isneginf(tm[:-n_q, -1])) and np.all(np.isfinite(tm[-n_q:, -1]))
    live = 0
    nts = [-(-c // 16) for c in ctxs]
    n_hq = hc.shape.n_kv * rc.verify_geometry(q_len, hc.shape.n_q, hc.shape.n_kv)
    cuts = {}
    for hq, s, a, b in rc.segments(nts, n_hq, W):
        if hq == 0:
            cuts.setdefault(s, [0]).append(b)
    for s in range(len(ctxs)):
        tm = _row_tms(case, s)
        c = cuts[s]
        for a, b in zip(c[:-1], c[1:]):
            live += _live(tm, a, b)
    print(f"{profile} q_len {q_len}: {len(blind)} blind segments, {live} live rescales")
    if profile in ("staircase", "scale_1", "scale_8", "scale_100"):
        assert live >= 1


@pytest.mark.parametrize("profile,chunk,d,seed", rc.prefill_specs())
def test_prefill_premise(profile, chunk, d, seed):
    """The prefill takes one running-max decision per 64-token tile."""
    case = rc.prefill_case(profile, chunk, d, seed)
    live = 0
    for s in range(len(case.hc.tables.context_lens)):
        tm = _row_tms(case, s, tile_tokens=64)
        live += _live(tm, 0, tm.shape[1])
    print(f"{profile} chunk {chunk}: {live} live rescales")
    if profile in ("late_jump", "staircase", "scale_1", "scale_8", "scale_100"):
        assert live >= 1


@pytest.mark.parametrize("profile,d,seed", rc.prefix_specs())
def test_prefix_premise(profile, d, seed):
    """Member rows: the prefix part (read by the prefix units) and the
    member's own tiles give partials whose maxima lie far apart, and the
    own tiles rescale a live accumulator."""
    case, pre, first, count = rc.prefix_case(profile, d, seed)
    G = case.hc.shape.n_q // case.hc.shape.n_kv
    span = 0.0
    live = 0
    for s in range(first, first + count):
        tm = _row_tms(case, s)[:G]
        span = max(span, float(np.nanmax(_spans(tm, [0, pre, tm.shape[1]]))))
        live += _live(tm, pre, tm.shape[1])
    print(f"{profile} d {d}: prefix/own span {span:.1f}, {live} live rescales in own tiles")
    if profile in ("late_jump", "early_peak", "staircase"):
        assert span >= 10.0
    if profile in ("late_jump", "staircase", "scale_1", "scale_8"):
        assert live >= 1
