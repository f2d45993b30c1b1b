"""Chunked prefill against the paged cache on the GPU, against the oracle.

A chunk of C tokens is each sequence's last C cached tokens: chunk token i
at position ctx - C + i sees positions [0, ctx - C + i], i.e. the oracle's
verification attention with q_len = C (oracle_verify), pinned against
torch's scaled_dot_product_attention with the causal mask aligned to the
sequence's end. Cases span several 64-row groups, ragged last groups, a
first chunk (ctx = C), d 64 and 128, MHA / GQA / MQA, NaN in every unused
slot and block. At the LLaMA-3-8B shape (8 sequences, 512-token chunks on
top of 1,024..6,144 cached tokens) sampled rows are recomputed one by one
(oracle_decode_row over the sequence cut at the row's position). The bar:
max-abs error <= 1e-3 on fp32 outputs; invalid contexts flagged, NaN rows.
"""
import numpy as np
import pytest

import workload as w
from gpu_util import TOL, max_abs, to_dev_bf16, to_dev_i32

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pkv():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import paged_kv_cache_468_amd as lib
    return lib


def _shape(n_q, n_kv, d):
    return w.Shape(f"{n_q}/{n_kv} d{d}", 1, n_q, n_kv, d, 1, 1, 1)


def _run(pkv, hc, qv, max_ctx=None):
    import torch
    sh = hc.shape
    max_ctx = int(hc.tables.context_lens.max()) if max_ctx is None else max_ctx
    out = torch.full(qv.shape, float("nan"), dtype=torch.float32, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    pkv.pkv_paged_prefill(out, to_dev_bf16(qv), to_dev_bf16(hc.k_pool), to_dev_bf16(hc.v_pool),
                          to_dev_i32(hc.tables.block_tables), to_dev_i32(hc.tables.context_lens),
                          sh.scale, max_ctx, err_flag=err)
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64), int(err.item())


CASES = [  # n_q, n_kv, d, contexts, chunk   (rows per KV head = chunk * G)
    (32, 8, 128, [64, 300, 1000], 64),        # 256 rows: four 64-row groups
    (32, 8, 128, [128, 200], 128),            # a first chunk (ctx = chunk)
    (20, 4, 64, [100, 513], 37),              # G = 5: 185 rows, ragged last group
    (8, 8, 128, [257, 300], 256),             # MHA
    (64, 8, 128, [600], 100),                 # G = 8: 800 rows
    (8, 1, 64, [90, 91, 400], 33),            # MQA: 264 rows
    (32, 8, 128, [17, 40], 5),                # short chunks: one group, partly filled
]


@pytest.mark.parametrize("case", range(len(CASES)))
def test_prefill_matches_oracle(pkv, orc, case):
    n_q, n_kv, d, ctx, C = CASES[case]
    hc = w.host_case(_shape(n_q, n_kv, d), 400 + case, context_lens=ctx)
    qv = w.normal_bf16(w.rng(400 + case, 15), (len(ctx), C, n_q, d))
    got, err = _run(pkv, hc, qv)
    want, rc = orc.verify(qv, hc.k_pool, hc.v_pool, hc.tables.block_tables, hc.tables.context_lens,
                          n_kv, hc.shape.scale)
    assert rc == 0 and err == 0
    assert np.isfinite(got).all()
    e = max_abs(got, want)
    print(f"case {case}: chunk {C}, {C * n_q // n_kv} rows per KV head: max-abs {e:.2e}")
    assert e <= TOL, e


def test_invalid_context_flagged(pkv, orc):
    import paged_kv_cache_468_amd as lib
    n_q, n_kv, d, C = 8, 2, 64, 20
    ctx = [50, 19, 70]
    hc = w.host_case(_shape(n_q, n_kv, d), 440, context_lens=ctx)
    qv = w.normal_bf16(w.rng(440, 15), (3, C, n_q, d))
    got, err = _run(pkv, hc, qv)
    assert err & lib.PKV_DEVERR_CONTEXT
    assert np.isnan(got[1]).all()
    want, rc = orc.verify(qv, hc.k_pool, hc.v_pool, hc.tables.block_tables, hc.tables.context_lens,
                          n_kv, hc.shape.scale)
    assert max_abs(got[[0, 2]], want[[0, 2]]) <= TOL


def test_llama3_shape_sampled(pkv, orc):
    """8 sequences of the LLaMA-3-8B shape prefill a 512-token chunk on top
    of 1,024..6,144 cached tokens (the benchmark's launch); 96 sampled
    (sequence, token, head) rows, the first and last token of every
    sequence included, recomputed one by one."""
    import torch
    shape = w.CONFIGS[4]
    C, B = 512, 8
    g = w.rng(45, 16)
    ctx = (g.integers(1024, 6145, B) + C).astype(np.int32)
    sh1 = w.Shape(shape.name, 1, shape.n_q, shape.n_kv, shape.d, B, 1, 1)
    t = w.build_tables(sh1, 45, context_lens=ctx)
    ks, vs = w.pool_shapes(t.num_blocks, shape.n_kv, shape.d)
    kp = w.device_normal_bf16_(torch.empty(ks, dtype=torch.bfloat16, device="cuda"), 46)
    vp = w.device_normal_bf16_(torch.empty(vs, dtype=torch.bfloat16, device="cuda"), 47)
    qv = w.normal_bf16(g, (B, C, shape.n_q, shape.d))
    out = torch.full(qv.shape, float("nan"), dtype=torch.float32, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    pkv.pkv_paged_prefill(out, to_dev_bf16(qv), kp, vp, to_dev_i32(t.block_tables),
                          to_dev_i32(ctx), shape.scale, int(ctx.max()), err_flag=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    got = out.cpu().numpy()
    assert np.isfinite(got).all()
    k_h = kp.view(torch.int16).cpu().numpy().view(np.uint16)
    v_h = vp.view(torch.int16).cpu().numpy().view(np.uint16)
    G = shape.n_q // shape.n_kv
    picks = [(s, 0, 0) for s in range(B)] + [(s, C - 1, shape.n_q - 1) for s in range(B)]
    for _ in range(80):
        picks.append((int(g.integers(B)), int(g.integers(C)), int(g.integers(shape.n_q))))
    e = 0.0
    for s, i, j in picks:
        want, rc = orc.decode_row(qv[s, i, j], k_h, v_h, t.block_tables[s],
                                  int(ctx[s]) - C + i + 1, shape.n_kv, j // G, shape.scale)
        assert rc == 0
        e = max(e, float(np.abs(got[s, i, j] - want).max()))
    print(f"llama3 shape, 8 x 512-token chunks, {len(picks)} sampled rows: max-abs {e:.2e}")
    assert e <= TOL


def test_largest_chunk_sampled(pkv, orc):
    """The largest chunk, 16,384 tokens, on top of 300 cached ones, at the
    LLaMA-3-8B heads (65,536 rows per KV head): sampled rows, the chunk's
    first and last token included, recomputed one by one."""
    import torch
    shape = w.CONFIGS[4]
    C = 16384
    ctx = np.array([C + 300], np.int32)
    sh1 = w.Shape(shape.name, 1, shape.n_q, shape.n_kv, shape.d, 1, 1, 1)
    t = w.build_tables(sh1, 47, context_lens=ctx)
    ks, vs = w.pool_shapes(t.num_blocks, shape.n_kv, shape.d)
    kp = w.device_normal_bf16_(torch.empty(ks, dtype=torch.bfloat16, device="cuda"), 471)
    vp = w.device_normal_bf16_(torch.empty(vs, dtype=torch.bfloat16, device="cuda"), 472)
    g = w.rng(47, 16)
    qv = w.normal_bf16(g, (1, C, shape.n_q, shape.d))
    out = torch.full(qv.shape, float("nan"), dtype=torch.float32, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    pkv.pkv_paged_prefill(out, to_dev_bf16(qv), kp, vp, to_dev_i32(t.block_tables),
                          to_dev_i32(ctx), shape.scale, int(ctx.max()), err_flag=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    got = out.cpu().numpy()
    assert np.isfinite(got).all()
    k_h = kp.view(torch.int16).cpu().numpy().view(np.uint16)
    v_h = vp.view(torch.int16).cpu().numpy().view(np.uint16)
    G = shape.n_q // shape.n_kv
    picks = [(0, 0), (C - 1, shape.n_q - 1)] + [(int(g.integers(C)), int(g.integers(shape.n_q)))
                                                for _ in range(30)]
    e = 0.0
    for i, j in picks:
        want, rc = orc.decode_row(qv[0, i, j], k_h, v_h, t.block_tables[0], int(ctx[0]) - C + i + 1,
                                  shape.n_kv, j // G, shape.scale)
        assert rc == 0
        e = max(e, float(np.abs(got[0, i, j] - want).max()))
    print(f"16,384-token chunk, {len(picks)} sampled rows: max-abs {e:.2e}")
    assert e <= TOL


ORDER_CASES = [  # n_q, n_kv, d, contexts, chunk
    # equal contexts: the ranking by work breaks ties by sequence index
    (8, 2, 64, [40, 40, 100, 17, 100, 40, 17, 17, 250, 40, 100, 17, 33, 33, 250, 40], 9),
    # more sequences than a workgroup has threads: index order
    (4, 2, 64, [int(5 + (i * 37) % 60) for i in range(600)], 3),
    # KV heads not a multiple of the XCD count, pairs dealt over several rounds
    (12, 3, 128, [300, 20, 150, 150, 700, 64, 65, 500, 21, 300, 90], 20),
    # a count that is not a multiple of 4 (the ranking reads its keys four
    # at a time), many ties
    (4, 2, 64, [int(5 + (i * 53) % 40) for i in range(301)], 2),
    # one (sequence, KV head) pair, fewer than the XCDs: its five row tiles
    # go round the XCDs
    (8, 1, 128, [700], 160),
    # 15 pairs, not a whole number of deals: row tiles round the XCDs
    (12, 3, 64, [130, 70, 400, 255, 90], 40),
]


@pytest.mark.parametrize("case", range(len(ORDER_CASES)))
def test_work_order_covers_every_row(pkv, orc, case):
    """The workgroups take the (sequence, KV head) pairs longest context
    first; every row of every sequence is still written once (the output
    starts as NaN) and matches the oracle."""
    n_q, n_kv, d, ctx, C = ORDER_CASES[case]
    hc = w.host_case(_shape(n_q, n_kv, d), 460 + case, context_lens=ctx)
    qv = w.normal_bf16(w.rng(460 + case, 15), (len(ctx), C, n_q, d))
    got, err = _run(pkv, hc, qv)
    want, rc = orc.verify(qv, hc.k_pool, hc.v_pool, hc.tables.block_tables, hc.tables.context_lens,
                          n_kv, hc.shape.scale)
    assert rc == 0 and err == 0
    assert np.isfinite(got).all()
    e = max_abs(got, want)
    print(f"order case {case}: {len(ctx)} sequences, chunk {C}: max-abs {e:.2e}")
    assert e <= TOL, e
