"""A seeded random sweep of the decode step (and its vector-ALU partition
kernel), the verification pass, chunked prefill and the shared-prefix step
against the oracle, beside the
hand-picked cases of the other tests. Each
case draws: KV heads (1, 2, 4, 8) and group size (1 .. 20, at most 64 query
heads), head size 64 or 128, 1 .. 24 sequences whose contexts mix tiny ones,
ones around a block boundary and long ones (up to 3,000 tokens), table
widths and max_context_len above the longest context, the fixed partition
size or the balanced split, and fused or separate append. Pools are
NaN-filled outside the contexts. Each case is printed before it runs. Bar:
max-abs <= 1e-3 on the outputs; the pools bit-exact after the append."""
import math

import numpy as np
import pytest

import workload as w
from gpu_util import (TOL, DevCase, gpu_step, max_abs, oracle_step, to_dev_bf16, to_dev_i32,
                      to_host_u16)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pkv():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import paged_kv_cache_468_amd as lib
    return lib


def _draw(seed, min_ctx=1):
    g = np.random.default_rng([9100, seed])
    while True:
        n_kv = int(g.choice([1, 2, 4, 8]))
        G = int(g.choice([1, 2, 3, 4, 5, 7, 8, 16, 20]))
        if n_kv * G <= 64:
            break
    d = int(g.choice([64, 128]))
    B = int(g.integers(1, 25))
    ctx = []
    for _ in range(B):
        r = g.random()
        if r < 0.2:
            c = int(g.integers(1, 17))
        elif r < 0.45:
            c = int(16 * g.integers(1, 60) + g.integers(-1, 2))    # around a block boundary
        else:
            c = int(g.integers(17, 3001))
        ctx.append(max(min_ctx, c))
    slack = int(g.choice([0, 0, 16, 700]))
    part = int(g.choice([0, 0, 0, 16, 64, 256]))
    fused = bool(g.integers(2))
    return n_kv * G, n_kv, d, ctx, slack, part, fused, g


def _host(n_q, n_kv, d, ctx, slack, seed):
    shape = w.Shape(f"sweep {seed}", 1, n_q, n_kv, d, 1, 1, 1)
    max_ctx = max(ctx) + slack
    return w.host_case(shape, 9100 + seed, context_lens=ctx,
                       max_blocks=math.ceil(max_ctx / w.BLOCK)), max_ctx


@pytest.mark.parametrize("seed", range(30))
def test_decode_sweep(pkv, orc, seed):
    n_q, n_kv, d, ctx, slack, part, fused, _ = _draw(seed)
    print(f"seed {seed}: {n_q}/{n_kv} heads, d {d}, {len(ctx)} sequences up to {max(ctx)}, "
          f"slack {slack}, partition {part}, fused {fused}", flush=True)
    hc, max_ctx = _host(n_q, n_kv, d, ctx, slack, seed)
    dc = DevCase(hc)
    got = gpu_step(pkv, dc, partition=part, max_ctx=max_ctx, fused=fused)
    want, rc, k_ref, v_ref = oracle_step(orc, hc)
    assert rc == 0 and int(dc.err.item()) == 0
    assert np.array_equal(to_host_u16(dc.k_pool), k_ref)
    assert np.array_equal(to_host_u16(dc.v_pool), v_ref)
    e = max_abs(got, want)
    print(f"  max-abs {e:.2e}")
    assert np.isfinite(got).all() and e <= TOL


@pytest.mark.parametrize("seed", range(500, 515))
def test_valu_sweep(pkv, orc, seed):
    """The vector-ALU partition kernel and the merge on the same kind of
    draws (group sizes up to 8, the balanced split)."""
    import torch
    g = np.random.default_rng([9500, seed])
    n_kv = int(g.choice([1, 2, 4, 8]))
    G = int(g.integers(1, 9))
    n_q, _, d, ctx, slack, _, _, _ = _draw(seed)
    n_q = n_kv * G
    print(f"seed {seed}: {n_q}/{n_kv} heads, d {d}, {len(ctx)} sequences up to {max(ctx)}, "
          f"slack {slack}", flush=True)
    hc, max_ctx = _host(n_q, n_kv, d, ctx, slack, seed)
    dc = DevCase(hc)
    ws = pkv.pkv_decode_step_partition_valu(dc.out, dc.q, dc.k_new, dc.v_new, dc.k_pool, dc.v_pool,
                                            dc.bt, dc.cl, hc.shape.scale, max_ctx, err_flag=dc.err)
    pkv.pkv_paged_attn_merge(dc.out, dc.q, dc.k_pool, dc.v_pool, dc.bt, dc.cl, hc.shape.scale,
                             max_ctx, workspace=ws, err_flag=dc.err)
    torch.cuda.synchronize()
    got = dc.out.cpu().numpy().astype(np.float64)
    want, rc, k_ref, v_ref = oracle_step(orc, hc)
    assert rc == 0 and int(dc.err.item()) == 0
    assert np.array_equal(to_host_u16(dc.k_pool), k_ref)
    assert np.array_equal(to_host_u16(dc.v_pool), v_ref)
    e = max_abs(got, want)
    print(f"  max-abs {e:.2e}")
    assert np.isfinite(got).all() and e <= TOL


@pytest.mark.parametrize("seed", range(100, 115))
def test_verify_sweep(pkv, orc, seed):
    import torch
    g0 = np.random.default_rng([9200, seed])
    q_len = int(g0.integers(1, 13))
    n_q, n_kv, d, ctx, slack, _, _, g = _draw(seed, min_ctx=q_len)
    print(f"seed {seed}: {n_q}/{n_kv} heads, d {d}, {len(ctx)} sequences up to {max(ctx)}, "
          f"slack {slack}, q_len {q_len}", flush=True)
    hc, max_ctx = _host(n_q, n_kv, d, ctx, slack, seed)
    qv = w.normal_bf16(g, (len(ctx), q_len, n_q, d))
    out = torch.full(qv.shape, float("nan"), dtype=torch.float32, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    pkv.pkv_paged_attn_verify(out, to_dev_bf16(qv), to_dev_bf16(hc.k_pool), to_dev_bf16(hc.v_pool),
                              to_dev_i32(hc.tables.block_tables), to_dev_i32(hc.tables.context_lens),
                              hc.shape.scale, max_ctx, err_flag=err)
    torch.cuda.synchronize()
    want, rc = orc.verify(qv, hc.k_pool, hc.v_pool, hc.tables.block_tables,
                          hc.tables.context_lens, n_kv, hc.shape.scale)
    assert rc == 0 and int(err.item()) == 0
    got = out.cpu().numpy().astype(np.float64)
    e = max_abs(got, want)
    print(f"  max-abs {e:.2e}")
    assert np.isfinite(got).all() and e <= TOL


@pytest.mark.parametrize("seed", range(200, 210))
def test_prefill_sweep(pkv, orc, seed):
    """Chunked prefill over random shapes: chunks of 1 .. 160 tokens (so
    256-row workgroups from nearly empty to several per KV head), 1 .. 4
    sequences with 0 .. 1,000 cached tokens before the chunk."""
    import torch
    g = np.random.default_rng([9300, seed])
    while True:
        n_kv = int(g.choice([1, 2, 4, 8]))
        G = int(g.choice([1, 2, 3, 4, 5, 8]))
        if n_kv * G <= 32:
            break
    n_q, d = n_kv * G, int(g.choice([64, 128]))
    C = int(g.integers(1, 161))
    B = int(g.integers(1, 5))
    ctx = [C + int(g.integers(0, 1001)) for _ in range(B)]
    slack = int(g.choice([0, 16, 300]))
    print(f"seed {seed}: {n_q}/{n_kv} heads, d {d}, chunk {C}, contexts {ctx}, slack {slack}",
          flush=True)
    hc, max_ctx = _host(n_q, n_kv, d, ctx, slack, seed)
    qv = w.normal_bf16(g, (B, C, n_q, d))
    out = torch.full(qv.shape, float("nan"), dtype=torch.float32, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    pkv.pkv_paged_prefill(out, to_dev_bf16(qv), to_dev_bf16(hc.k_pool), to_dev_bf16(hc.v_pool),
                          to_dev_i32(hc.tables.block_tables), to_dev_i32(hc.tables.context_lens),
                          hc.shape.scale, max_ctx, err_flag=err)
    torch.cuda.synchronize()
    want, rc = orc.verify(qv, hc.k_pool, hc.v_pool, hc.tables.block_tables,
                          hc.tables.context_lens, n_kv, hc.shape.scale)
    assert rc == 0 and int(err.item()) == 0
    got = out.cpu().numpy().astype(np.float64)
    e = max_abs(got, want)
    print(f"  max-abs {e:.2e}")
    assert np.isfinite(got).all() and e <= TOL


@pytest.mark.parametrize("seed", range(300, 315))
def test_prefix_sweep(pkv, orc, seed):
    """pkv_decode_step_prefix on random shapes: a prefix of 1 .. 40 blocks
    shared by every sequence longer than it (shorter ones hold a copy of
    the block they write), a random member range, contexts past the
    prefix by 1 .. 3,000 tokens; against the oracle, pools bit-exact."""
    g = np.random.default_rng([9300, seed])
    while True:
        n_kv = int(g.choice([1, 2, 4, 8]))
        G = int(g.choice([1, 2, 3, 4, 5, 7, 8, 16, 20]))
        if n_kv * G <= 64:
            break
    d = int(g.choice([64, 128]))
    B = int(g.integers(2, 25))
    pre = int(g.choice([1, 2, 7, 16, 40]))
    ctx = [int(16 * pre + g.integers(1, 3001)) if g.random() < 0.75 else int(g.integers(1, 16 * pre + 1))
           for _ in range(B)]
    first = int(g.integers(0, B))
    count = int(g.integers(0, B - first + 1))
    slack = int(g.choice([0, 16, 700]))
    print(f"seed {seed}: {n_kv * G}/{n_kv} heads, d {d}, {B} sequences up to {max(ctx)}, prefix "
          f"{pre} blocks, members {first}..{first + count - 1}, slack {slack}", flush=True)
    shape = w.Shape(f"prefix sweep {seed}", 1, n_kv * G, n_kv, d, 1, 1, 1, prefix_tokens=16 * pre)
    max_ctx = max(ctx) + slack
    hc = w.host_case(shape, 9300 + seed, context_lens=ctx, share=True,
                     max_blocks=math.ceil(max_ctx / w.BLOCK))
    dc = DevCase(hc)
    pkv.pkv_decode_step_prefix(dc.out, dc.q, dc.k_new, dc.v_new, dc.k_pool, dc.v_pool, dc.bt,
                               dc.cl, shape.scale, max_ctx, to_dev_i32(hc.tables.prefix_phys),
                               first, count, err_flag=dc.err)
    import torch
    torch.cuda.synchronize()
    got = dc.out.cpu().numpy().astype(np.float64)
    want, rc, k_ref, v_ref = oracle_step(orc, hc)
    assert rc == 0 and int(dc.err.item()) == 0
    assert np.array_equal(to_host_u16(dc.k_pool), k_ref)
    assert np.array_equal(to_host_u16(dc.v_pool), v_ref)
    e = max_abs(got, want)
    print(f"  max-abs {e:.2e}")
    assert np.isfinite(got).all() and e <= TOL
