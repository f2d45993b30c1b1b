"""Pins of the CPU oracle to things other than itself.

Each check takes an ``oracle.Oracle`` and raises AssertionError if the oracle
disagrees with what the pages or the mathematics fix:
  * values the pages print (tests/golden/kv_sizes.json, each with its source);
  * a hand-derived pool image and a hand-computed closed form
    (tests/golden/append_tiny.json);
  * special cases with closed forms (one cached token, constant values,
    equal keys, one dominant key);
  * a library routine: torch's scaled_dot_product_attention in float64 on
    contiguous K/V, with torch's own grouped-query head expansion;
  * invariants: the physical block permutation, shared prefix blocks against
    private copies, grouped heads against explicitly repeated heads.
tests/test_oracle_pins.py runs them on the real oracle; tests/
test_oracle_mutants.py runs them on deliberately broken copies and requires
every copy to fail at least one.
"""
import json
import math
import os

import numpy as np

import workload as w

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _small_shape(n_q, n_kv, d, prefix=0):
    return w.Shape(f"pin {n_q}/{n_kv} d{d}", 1, n_q, n_kv, d, 1, 1, 1, prefix_tokens=prefix)


# ---------------------------------------------------------------------------
# KV size closed form

def check_kv_sizes(orc):
    doc = _load("kv_sizes.json")
    for c in doc["cases"]:
        got = orc.kv_bytes(c["layers"], c["kv_heads"], c["d"], c["L"], c["B"], c["bytes"])
        if "exact_bytes" in c:
            assert got == c["exact_bytes"], (c["cite"], got)
        elif "rounds_to" in c:
            scale = 1e9 if c["unit"].endswith("GB") else 1e6
            assert round(got / scale, c["decimals"]) == c["rounds_to"], (c["cite"], got)
        else:
            scale = 2**30 if c["unit"] == "GiB" else 1.0
            assert abs(got / scale - c["approx"]) <= c["tol"], (c["cite"], got)


def check_kv_linearity(orc):
    """Doubling any one factor doubles the cache ("Module 23: Serving",
    23.1, the kv-cache-calculator figure's lesson)."""
    base = dict(n_layers=32, n_kv_heads=8, d_head=128, context_len=8192, batch=1, bytes_per_value=2)
    ref = orc.kv_bytes(**base)
    for k in base:
        b2 = dict(base)
        b2[k] *= 2
        assert orc.kv_bytes(**b2) == 2 * ref, k


# ---------------------------------------------------------------------------
# append / copy

def check_append_golden(orc):
    g = _load("append_tiny.json")
    n_kv, d, nb = g["n_kv"], g["d"], g["num_blocks"]
    k_pool = np.zeros(nb * n_kv * 16 * d, np.uint16)
    v_pool = np.zeros_like(k_pool)
    rc = orc.kv_append(k_pool, v_pool, np.array(g["k_new_bits"], np.uint16),
                       np.array(g["v_new_bits"], np.uint16),
                       np.array(g["block_tables"], np.int32), np.array(g["context_lens"], np.int32))
    assert rc == 0
    ek = np.zeros_like(k_pool)
    ev = np.zeros_like(v_pool)
    for i, val in g["expect_k_nonzero"].items():
        ek[int(i)] = val
    for i, val in g["expect_v_nonzero"].items():
        ev[int(i)] = val
    assert np.array_equal(k_pool, ek), np.nonzero(k_pool != ek)
    assert np.array_equal(v_pool, ev), np.nonzero(v_pool != ev)
    return k_pool, v_pool


def check_write_golden(orc):
    """A multi-token write against a pool image worked out by hand
    (tests/golden/write_tiny.json), invalid tokens included."""
    g = _load("write_tiny.json")
    n_kv, d, nb = g["n_kv"], g["d"], g["num_blocks"]
    k_pool = np.zeros(nb * n_kv * 16 * d, np.uint16)
    v_pool = np.zeros_like(k_pool)
    toks = np.array(g["tokens"], np.int32)
    rc = orc.kv_write(k_pool, v_pool, np.array(g["k_src_bits"], np.uint16),
                      np.array(g["v_src_bits"], np.uint16), np.array(g["block_tables"], np.int32),
                      toks[:, 0].copy(), toks[:, 1].copy())
    assert rc == g["expect_status"]
    ek = np.zeros_like(k_pool)
    ev = np.zeros_like(v_pool)
    for i, val in g["expect_k_nonzero"].items():
        ek[int(i)] = val
    for i, val in g["expect_v_nonzero"].items():
        ev[int(i)] = val
    assert np.array_equal(k_pool, ek), np.nonzero(k_pool != ek)
    assert np.array_equal(v_pool, ev), np.nonzero(v_pool != ev)


def check_write_equals_append(orc):
    """Writing each sequence's token at position ctx - 1 is the append."""
    hc = w.host_case(_small_shape(8, 2, 64), 7, context_lens=[1, 16, 17, 40, 300], nan_fill=False)
    k1, v1 = hc.k_pool.copy(), hc.v_pool.copy()
    k2, v2 = hc.k_pool.copy(), hc.v_pool.copy()
    cl = hc.tables.context_lens
    assert orc.kv_append(k1, v1, hc.k_new, hc.v_new, hc.tables.block_tables, cl) == 0
    assert orc.kv_write(k2, v2, hc.k_new, hc.v_new, hc.tables.block_tables,
                        np.arange(len(cl), dtype=np.int32), (cl - 1).astype(np.int32)) == 0
    assert np.array_equal(k1, k2) and np.array_equal(v1, v2)


def check_decode_golden(orc):
    """Closed form worked by hand for the pool image above."""
    g = _load("append_tiny.json")
    k_pool, v_pool = check_append_golden(orc)
    dc = g["decode_check"]
    s = dc["seq"]
    q = np.array([[dc["q_bits"], dc["q_bits"]]], np.uint16)           # 2 query heads, G = 1
    bt = np.array([g["block_tables"][s]], np.int32)
    cl = np.array([g["context_lens"][s]], np.int32)
    out, rc = orc.decode(q, k_pool, v_pool, bt, cl, g["n_kv"], 1.0)
    assert rc == 0
    e1, e3 = math.exp(-1.0), math.exp(-3.0)
    want = np.array([[[9 * e1 / (15 + e1), 10 * e1 / (15 + e1)],
                      [11 * e3 / (15 + e3), 12 * e3 / (15 + e3)]]])
    assert np.allclose(out, want, rtol=1e-14, atol=0), (out, want)


def check_append_touches_only_its_slots(orc):
    shape = _small_shape(4, 2, 64)
    case = w.host_case(shape, 11, context_lens=[1, 16, 17, 40, 33], nan_fill=False, spare_blocks=3)
    k0, v0 = case.k_pool.copy(), case.v_pool.copy()
    k, v = case.k_pool.copy(), case.v_pool.copy()
    assert orc.kv_append(k, v, case.k_new, case.v_new, case.tables.block_tables,
                         case.tables.context_lens) == 0
    changed_k = int((k != k0).sum())
    changed_v = int((v != v0).sum())
    n = case.k_new.size
    # every written element differs unless the random old value was equal
    assert changed_k <= n and changed_v <= n and changed_k >= n - 4 and changed_v >= n - 4
    # reading the token back through the layout gives k_new / v_new
    for s, ctx in enumerate(case.tables.context_lens):
        kc, vc = w.gather_contiguous(k, v, case.tables, s)
        assert np.array_equal(kc[:, ctx - 1, :], case.k_new[s])
        assert np.array_equal(vc[:, ctx - 1, :], case.v_new[s])


def check_copy_blocks(orc):
    shape = _small_shape(4, 2, 64)
    case = w.host_case(shape, 5, context_lens=[40, 50], nan_fill=False, spare_blocks=4)
    k, v = case.k_pool.copy(), case.v_pool.copy()
    free = np.nonzero(~case.tables.used)[0].astype(np.int32)
    src = case.tables.block_tables[:, 0].astype(np.int32)
    dst = free[:2]
    assert orc.copy_blocks(k, v, src, dst, 2, 64) == 0
    assert np.array_equal(k[dst], case.k_pool[src]) and np.array_equal(v[dst], case.v_pool[src])
    others = np.setdiff1d(np.arange(case.tables.num_blocks), dst)
    assert np.array_equal(k[others], case.k_pool[others])
    assert np.array_equal(v[others], case.v_pool[others])


# ---------------------------------------------------------------------------
# decode special cases

def _decode(orc, case, scale=None):
    sh = case.shape
    out, rc = orc.decode(case.q, case.k_pool, case.v_pool, case.tables.block_tables,
                         case.tables.context_lens, sh.n_kv, sh.scale if scale is None else scale)
    return out, rc


def check_single_token(orc):
    """ctx = 1: the softmax has one term, so out is that token's value."""
    case = w.host_case(_small_shape(8, 2, 128), 3, context_lens=[1, 1, 1])
    out, rc = _decode(orc, case)
    assert rc == 0
    for s in range(3):
        _, vc = w.gather_contiguous(case.k_pool, case.v_pool, case.tables, s)
        v0 = w.bf16_to_f32(vc[:, 0, :]).astype(np.float64)          # [n_kv, d]
        assert np.array_equal(out[s], np.repeat(v0, 4, axis=0))


def check_constant_values(orc):
    """All cached values equal c: the weights sum to one, so out = c."""
    case = w.host_case(_small_shape(5, 1, 64), 4, context_lens=[7, 16, 100, 257])
    c_bits = w.bf16_bits(np.array([1.71875], np.float32))[0]
    case.v_pool[case.tables.used] = c_bits
    out, rc = _decode(orc, case)
    assert rc == 0
    assert np.allclose(out, 1.71875, rtol=0, atol=1e-12)


def check_equal_keys(orc):
    """All keys of a sequence equal: every score is the same, the weights are
    uniform, and out is the plain mean of V over exactly [0, ctx)."""
    case = w.host_case(_small_shape(8, 2, 64), 6, context_lens=[15, 16, 17, 33, 130])
    for s, ctx in enumerate(case.tables.context_lens):
        kc, vc = w.gather_contiguous(case.k_pool, case.v_pool, case.tables, s)
        kc[:] = kc[:, :1, :]                                       # copy token 0's key everywhere
        w.scatter_contiguous(kc, vc, case.tables, s, case.k_pool, case.v_pool)
    out, rc = _decode(orc, case)
    assert rc == 0
    for s, ctx in enumerate(case.tables.context_lens):
        _, vc = w.gather_contiguous(case.k_pool, case.v_pool, case.tables, s)
        mean = w.bf16_to_f32(vc).astype(np.float64).mean(axis=1)     # [n_kv, d]
        assert np.allclose(out[s], np.repeat(mean, 4, axis=0), rtol=0, atol=1e-12), s


def _sdpa(case, scale):
    """torch's scaled_dot_product_attention in float64 on contiguous K/V."""
    import torch
    import torch.nn.functional as F
    sh = case.shape
    outs = []
    for s in range(len(case.tables.context_lens)):
        kc, vc = w.gather_contiguous(case.k_pool, case.v_pool, case.tables, s)
        q = torch.from_numpy(w.bf16_to_f32(case.q[s]).astype(np.float64))[None, :, None, :]
        k = torch.from_numpy(w.bf16_to_f32(kc).astype(np.float64))[None]
        v = torch.from_numpy(w.bf16_to_f32(vc).astype(np.float64))[None]
        o = F.scaled_dot_product_attention(q, k, v, scale=scale, enable_gqa=sh.n_q != sh.n_kv)
        outs.append(o[0, :, 0, :].numpy())
    return np.stack(outs)


SDPA_CASES = [  # (n_q, n_kv, d, context lengths, scale or None for 1/sqrt(d))
    (20, 4, 64, [17, 40, 77, 130], None),
    (4, 4, 128, [1, 15, 16, 31], None),
    (32, 8, 128, [300, 64, 1], 0.37),
    (8, 1, 64, [5, 48, 49], None),
    (64, 8, 128, [33], None),
]


def check_sdpa(orc):
    for i, (n_q, n_kv, d, ctx, scale) in enumerate(SDPA_CASES):
        case = w.host_case(_small_shape(n_q, n_kv, d), 100 + i, context_lens=ctx, spare_blocks=2)
        sc = 1 / math.sqrt(d) if scale is None else scale
        out, rc = _decode(orc, case, sc)
        assert rc == 0
        ref = _sdpa(case, sc)
        assert np.allclose(out, ref, rtol=1e-12, atol=1e-12), (i, np.abs(out - ref).max())


def check_large_logits(orc):
    """Scores in the thousands (scale 100): exp() of the raw scores would
    overflow even in double precision; the definition still gives the value
    row of the largest score whenever it wins by a wide margin."""
    case = w.host_case(_small_shape(4, 2, 64), 9, context_lens=[40, 90])
    out, rc = _decode(orc, case, 100.0)
    assert rc == 0 and np.isfinite(out).all()
    ref = _sdpa(case, 100.0)
    assert np.allclose(out, ref, rtol=1e-9, atol=1e-9)


# ---------------------------------------------------------------------------
# invariants

def check_block_permutation(orc):
    """Physical placement is invisible: identity tables and permuted tables
    over the same logical bytes give identical results ("Designing an LLM
    serving system", Paged attention: blocks need not be contiguous)."""
    sh = _small_shape(20, 4, 64)
    a = w.host_case(sh, 21, context_lens=[17, 40, 77, 130], permute=False)
    b = w.host_case(sh, 21, context_lens=[17, 40, 77, 130], permute=True)
    assert not np.array_equal(a.tables.block_tables, b.tables.block_tables)
    oa, _ = _decode(orc, a)
    ob, _ = _decode(orc, b)
    assert np.array_equal(oa, ob)


def check_shared_prefix(orc):
    """Sequences pointing at shared prefix blocks give the same results as
    sequences holding private copies of the same bytes."""
    sh = _small_shape(8, 2, 64, prefix=64)
    ctx = [20, 64, 65, 100, 48]
    a = w.host_case(sh, 31, context_lens=ctx, share=True)
    b = w.host_case(sh, 31, context_lens=ctx, share=False)
    assert a.tables.num_blocks < b.tables.num_blocks
    oa, _ = _decode(orc, a)
    ob, _ = _decode(orc, b)
    assert np.array_equal(oa, ob)


def check_group_equals_repeat(orc):
    """Grouped-query heads are multi-head attention with each KV head
    repeated for its G query heads (consecutive groups)."""
    sh = _small_shape(12, 3, 64)
    case = w.host_case(sh, 41, context_lens=[9, 70])
    out_g, _ = _decode(orc, case)
    G = 4
    k_rep = np.ascontiguousarray(np.repeat(case.k_pool, G, axis=1))
    v_rep = np.ascontiguousarray(np.repeat(case.v_pool, G, axis=1))
    out_m, _ = orc.decode(case.q, k_rep, v_rep, case.tables.block_tables,
                          case.tables.context_lens, 12, sh.scale)
    assert np.array_equal(out_g, out_m)


def check_invalid_inputs(orc):
    sh = _small_shape(4, 2, 64)
    case = w.host_case(sh, 51, context_lens=[20, 30])
    bt = case.tables.block_tables.copy()
    bt[1, 1] = case.tables.num_blocks            # out of range
    out, rc = orc.decode(case.q, case.k_pool, case.v_pool, bt, case.tables.context_lens, 2, sh.scale)
    assert rc == -1 and np.isnan(out[1]).all() and np.isfinite(out[0]).all()
    cl = case.tables.context_lens.copy()
    cl[0] = 0
    out, rc = orc.decode(case.q, case.k_pool, case.v_pool, case.tables.block_tables, cl, 2, sh.scale)
    assert rc == -1 and np.isnan(out[0]).all() and np.isfinite(out[1]).all()


# ---------------------------------------------------------------------------
# the decode's single-precision twin (the naive fp32 loop)

U32 = 2.0 ** -24   # unit roundoff of binary32


def _gamma(n):
    return n * U32 / (1 - n * U32)


def _f32_bound(case, scale):
    """A bound on |f32 - exact| per (sequence, head) from the operations the
    fp32 loop performs, in the standard model (each operation's result is the
    exact one times (1 + e), |e| <= u; a sum of n terms within gamma_n of the
    sum of magnitudes):
      score   |dz| <= |scale| gamma_d sum_i |q_i k_i| + u |z|
      z - top adds both errors and one rounding: D = 2 max|dz| + u max|z - top|
      expf    within 2 u of its argument's exponential (glibc's expf is
              correctly rounded in almost all cases, below 1 ulp otherwise)
      weights relative error E = exp(D) - 1 + 2u
      sums    gamma_ctx on the total, gamma_(ctx+1) on the weighted values
    out = A / T errs by at most (|dA| + |out| |dT|) / T + u |out|, with
    |dA| <= (E + gamma_(ctx+1)) sum w |v| and |dT| <= (E + gamma_ctx) T."""
    sh = case.shape
    G = sh.n_q // sh.n_kv
    B = len(case.tables.context_lens)
    bound = np.zeros((B, sh.n_q))
    for s in range(B):
        kc, vc = w.gather_contiguous(case.k_pool, case.v_pool, case.tables, s)
        k = w.bf16_to_f32(kc).astype(np.float64)
        v = w.bf16_to_f32(vc).astype(np.float64)
        ctx = k.shape[1]
        for j in range(sh.n_q):
            q = w.bf16_to_f32(case.q[s, j]).astype(np.float64)
            kh, vh = k[j // G], v[j // G]
            z = scale * (kh @ q)
            dz = abs(scale) * _gamma(sh.d) * (np.abs(kh) @ np.abs(q)) + U32 * np.abs(z)
            D = 2 * dz.max() + U32 * (z.max() - z.min())
            E = math.expm1(D) + 2 * U32
            wgt = np.exp(z - z.max())
            T = wgt.sum()
            out = (wgt @ vh) / T
            dA = (E + _gamma(ctx + 1)) * (wgt @ np.abs(vh))
            dT = (E + _gamma(ctx)) * T
            bound[s, j] = ((dA + np.abs(out) * dT) / T + U32 * np.abs(out)).max()
    return bound


F32_CASES = [  # (n_q, n_kv, d, context lengths, scale or None for 1/sqrt(d))
    (20, 4, 64, [17, 40, 77, 130, 1], None),
    (32, 8, 128, [300, 64, 1, 1000], None),
    (8, 1, 64, [5, 48, 49, 2000], 0.37),
    (64, 8, 128, [33, 700], None),
]


def check_f32_within_bound_of_twin(orc):
    """The fp32 loop against its float64 twin (itself pinned to torch's
    scaled_dot_product_attention in float64): every row within the rounding
    bound of the fp32 operations (_f32_bound; a worst case, 1e-5 to 1e-3 at
    these inputs, against an observed few 1e-7)."""
    for i, (n_q, n_kv, d, ctx, scale) in enumerate(F32_CASES):
        case = w.host_case(_small_shape(n_q, n_kv, d), 700 + i, context_lens=ctx, spare_blocks=2)
        sc = 1 / math.sqrt(d) if scale is None else scale
        o64, r64 = _decode(orc, case, sc)
        o32, r32 = orc.decode_f32(case.q, case.k_pool, case.v_pool, case.tables.block_tables,
                                  case.tables.context_lens, n_kv, sc)
        assert r64 == 0 and r32 == 0 and o32.dtype == np.float32
        err = np.abs(o32.astype(np.float64) - o64).max(axis=2)
        bound = _f32_bound(case, sc)
        assert (err <= bound).all(), (i, float(err.max()), float(bound.min()))


def check_f32_exact_cases(orc):
    """Cases the fp32 loop must get exactly: one cached token (its weight is
    expf(0) = 1, so out is that token's value), values all equal to a power
    of two c (scaling by c commutes with every rounding, so out = c), and
    the same bits for an identity and a permuted block table."""
    case = w.host_case(_small_shape(8, 2, 128), 3, context_lens=[1, 1, 1])
    out, rc = orc.decode_f32(case.q, case.k_pool, case.v_pool, case.tables.block_tables,
                             case.tables.context_lens, 2, case.shape.scale)
    assert rc == 0
    for s in range(3):
        _, vc = w.gather_contiguous(case.k_pool, case.v_pool, case.tables, s)
        assert np.array_equal(out[s], np.repeat(w.bf16_to_f32(vc[:, 0, :]), 4, axis=0))
    case = w.host_case(_small_shape(5, 1, 64), 4, context_lens=[7, 16, 100, 257])
    case.v_pool[case.tables.used] = w.bf16_bits(np.array([-0.5], np.float32))[0]
    out, rc = orc.decode_f32(case.q, case.k_pool, case.v_pool, case.tables.block_tables,
                             case.tables.context_lens, 1, case.shape.scale)
    assert rc == 0 and (out == np.float32(-0.5)).all()
    sh = _small_shape(20, 4, 64)
    a = w.host_case(sh, 21, context_lens=[17, 40, 77, 130], permute=False)
    b = w.host_case(sh, 21, context_lens=[17, 40, 77, 130], permute=True)
    oa, _ = orc.decode_f32(a.q, a.k_pool, a.v_pool, a.tables.block_tables, a.tables.context_lens,
                           4, sh.scale)
    ob, _ = orc.decode_f32(b.q, b.k_pool, b.v_pool, b.tables.block_tables, b.tables.context_lens,
                           4, sh.scale)
    assert np.array_equal(oa, ob)


def check_f32_large_logits(orc):
    """Scale 100: scores in the thousands, where expf of an unshifted score
    overflows. Rows whose largest score leads the next by more than 30
    natural units are, to within e^-30 of the weights, that token's value."""
    case = w.host_case(_small_shape(4, 2, 64), 9, context_lens=[40, 90])
    out, rc = orc.decode_f32(case.q, case.k_pool, case.v_pool, case.tables.block_tables,
                             case.tables.context_lens, 2, 100.0)
    assert rc == 0 and np.isfinite(out).all()
    checked = 0
    for s in range(2):
        kc, vc = w.gather_contiguous(case.k_pool, case.v_pool, case.tables, s)
        for j in range(4):
            q = w.bf16_to_f32(case.q[s, j]).astype(np.float64)
            z = 100.0 * (w.bf16_to_f32(kc[j // 2]).astype(np.float64) @ q)
            top2 = np.sort(z)[-2:]
            if top2[1] - top2[0] > 30:
                v_top = w.bf16_to_f32(vc[j // 2, int(np.argmax(z))])
                assert np.abs(out[s, j] - v_top).max() < 1e-6, (s, j)
                checked += 1
    assert checked >= 4, checked


def check_f32_invalid_inputs(orc):
    """As the float64 decode: NaN rows and status -1 for a bad block id or a
    context length below one; the other rows finite."""
    sh = _small_shape(4, 2, 64)
    case = w.host_case(sh, 51, context_lens=[20, 30])
    bt = case.tables.block_tables.copy()
    bt[1, 1] = case.tables.num_blocks
    out, rc = orc.decode_f32(case.q, case.k_pool, case.v_pool, bt, case.tables.context_lens, 2,
                             sh.scale)
    assert rc == -1 and np.isnan(out[1]).all() and np.isfinite(out[0]).all()
    cl = case.tables.context_lens.copy()
    cl[0] = 0
    out, rc = orc.decode_f32(case.q, case.k_pool, case.v_pool, case.tables.block_tables, cl, 2,
                             sh.scale)
    assert rc == -1 and np.isnan(out[0]).all() and np.isfinite(out[1]).all()


# ---------------------------------------------------------------------------
# verification attention (q_len query tokens per sequence, causal among them)

def _verify_case(seed, n_q, n_kv, d, ctx, q_len):
    case = w.host_case(_small_shape(n_q, n_kv, d), seed, context_lens=ctx)
    g = w.rng(seed, 11)
    qv = w.normal_bf16(g, (len(ctx), q_len, n_q, d))
    return case, qv


def _verify(orc, case, qv, scale=None):
    sh = case.shape
    sc = sh.scale if scale is None else scale
    return orc.verify(qv, case.k_pool, case.v_pool, case.tables.block_tables,
                      case.tables.context_lens, sh.n_kv, sc)


def check_verify_one_token_is_decode(orc):
    """q_len = 1 is the decode step itself."""
    case, qv = _verify_case(21, 8, 2, 64, [1, 16, 17, 90], 1)
    case.q[:] = qv[:, 0]
    got, rc = _verify(orc, case, qv)
    want, rc2 = _decode(orc, case)
    assert rc == 0 and rc2 == 0
    assert np.array_equal(got[:, 0], want)


VERIFY_SDPA_CASES = [  # (n_q, n_kv, d, context lengths, q_len)
    (8, 2, 64, [5, 16, 17, 40], 5),
    (20, 4, 64, [33, 64, 100], 3),
    (32, 8, 128, [16, 31, 200], 8),
    (4, 4, 128, [2, 9], 2),
]


def check_verify_sdpa(orc):
    """Against torch's scaled_dot_product_attention in float64 on the
    contiguous cache, with the causal mask aligned to the sequence's end:
    query i may see token t iff t <= ctx - q_len + i."""
    import torch
    import torch.nn.functional as F
    for k, (n_q, n_kv, d, ctx, q_len) in enumerate(VERIFY_SDPA_CASES):
        case, qv = _verify_case(30 + k, n_q, n_kv, d, ctx, q_len)
        got, rc = _verify(orc, case, qv)
        assert rc == 0
        for s, c in enumerate(ctx):
            kc, vc = w.gather_contiguous(case.k_pool, case.v_pool, case.tables, s)
            qt = torch.from_numpy(w.bf16_to_f32(qv[s]).astype(np.float64)).permute(1, 0, 2)[None]
            kt = torch.from_numpy(w.bf16_to_f32(kc).astype(np.float64))[None]
            vt = torch.from_numpy(w.bf16_to_f32(vc).astype(np.float64))[None]
            mask = torch.arange(c)[None, :] <= (c - q_len + torch.arange(q_len))[:, None]
            o = F.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask, scale=1.0 / math.sqrt(d),
                                               enable_gqa=n_q != n_kv)
            ref = o[0].permute(1, 0, 2).numpy()                      # [q_len, n_q, d]
            assert np.allclose(got[s], ref, rtol=0, atol=1e-12), (k, s)


def check_verify_causal(orc):
    """Keys and values after a query's own position never change its row;
    they do change the rows of the later queries that see them."""
    ctx, q_len = [40, 21], 6
    case, qv = _verify_case(41, 8, 2, 64, ctx, q_len)
    base, rc = _verify(orc, case, qv)
    assert rc == 0
    for s, c in enumerate(ctx):
        cut = c - q_len + 2            # query 2 sees tokens [0, cut]
        kc, vc = w.gather_contiguous(case.k_pool, case.v_pool, case.tables, s)
        kc2, vc2 = kc.copy(), vc.copy()
        kc2[:, cut + 1:] = w.bf16_bits(-w.bf16_to_f32(kc[:, cut + 1:]) * 3)
        vc2[:, cut + 1:] = w.bf16_bits(w.bf16_to_f32(vc[:, cut + 1:]) + 5)
        k_pool, v_pool = case.k_pool.copy(), case.v_pool.copy()
        w.scatter_contiguous(kc2, vc2, case.tables, s, k_pool, v_pool)
        got, rc = orc.verify(qv, k_pool, v_pool, case.tables.block_tables,
                             case.tables.context_lens, case.shape.n_kv, case.shape.scale)
        assert rc == 0
        assert np.array_equal(got[s, :3], base[s, :3]), s
        assert not np.allclose(got[s, 3:], base[s, 3:]), s
        other = 1 - s
        assert np.array_equal(got[other], base[other])


def check_verify_invalid(orc):
    """Fewer cached tokens than query tokens is invalid: NaN rows, status -1,
    the other sequences untouched."""
    case, qv = _verify_case(43, 4, 1, 64, [3, 30], 4)
    got, rc = _verify(orc, case, qv)
    assert rc == -1
    assert np.isnan(got[0]).all() and np.isfinite(got[1]).all()


ALL_CHECKS = [check_kv_sizes, check_kv_linearity, check_append_golden, check_write_golden,
              check_write_equals_append, check_decode_golden,
              check_append_touches_only_its_slots, check_copy_blocks, check_single_token,
              check_constant_values, check_equal_keys, check_sdpa, check_large_logits,
              check_block_permutation, check_shared_prefix, check_group_equals_repeat,
              check_invalid_inputs, check_verify_one_token_is_decode, check_verify_sdpa,
              check_verify_causal, check_verify_invalid, check_f32_within_bound_of_twin,
              check_f32_exact_cases, check_f32_large_logits, check_f32_invalid_inputs]
