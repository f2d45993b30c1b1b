"""The decode step for a batch that shares a prompt prefix
(pkv_decode_step_prefix): the partition kernel reads the prefix's tiles once
for every member sequence (prefix units of its split, 32 member rows per
tile) and each member's own tiles after the prefix, and the merge kernel
combines both.

The bar: outputs within 1e-3 of the oracle (which walks every sequence's own
table), within 2.5e-5 of pkv_decode_step on the same inputs (only the order
of the fp32 sums differs), and the pools bitwise equal to pkv_decode_step's
(the append is the same). Members whose context ends inside the prefix,
sequences outside the member range, head groups above 16 and both head
sizes are covered; an empty prefix is pkv_decode_step bit for bit; a member
whose table does not start with the prefix is caught on the device.
"""
import math

import numpy as np
import pytest

import workload as w
from gpu_util import (TOL, DevCase, gpu_step, max_abs, oracle_step, to_dev_bf16, to_dev_i32,
                      to_host_u16)

pytestmark = pytest.mark.gpu

# GPU against GPU in another summation order: each fp32 result lies within
# about 1e-5 of the exact value (up to 9.3e-6 against the float64 oracle in
# these cases), so the two differ by at most about twice that.
CROSS = 2.5e-5


@pytest.fixture(scope="module")
def pkv():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import paged_kv_cache_468_amd as lib
    return lib


def _shape(n_q, n_kv, d, prefix):
    return w.Shape(f"{n_q}/{n_kv} d{d}", 1, n_q, n_kv, d, 1, 1, 1, prefix_tokens=prefix)


def _prefix_step(pkv, dc, first=0, count=None, table=None):
    import torch
    hc = dc.hc
    B = hc.q.shape[0]
    count = B - first if count is None else count
    pt = to_dev_i32(hc.tables.prefix_phys if table is None else table)
    pkv.pkv_decode_step_prefix(dc.out, dc.q, dc.k_new, dc.v_new, dc.k_pool, dc.v_pool, dc.bt,
                               dc.cl, hc.shape.scale, dc.max_ctx, pt, first, count,
                               err_flag=dc.err)
    torch.cuda.synchronize()
    return dc.out.cpu().numpy().astype(np.float64)


CASES = [
    # n_q, n_kv, d, prefix tokens, context lengths (some end inside the prefix)
    (32, 8, 128, 256, [100, 256, 257, 300, 1000, 2048, 4000, 17, 272, 5000]),
    (20, 4, 64, 48, [17, 40, 49, 77, 130, 300, 64, 65]),
    (16, 16, 128, 64, [65, 80, 200, 1000, 64, 3]),
    (64, 8, 128, 128, [129, 500, 2000, 8000, 60]),
    (32, 1, 128, 32, [33, 40, 90, 33, 1200]),     # 32 query heads per KV head: two row groups
    (4, 4, 64, 1024, [1025, 2000, 3000, 4096]),   # a long prefix, few rows
]


@pytest.mark.parametrize("case", range(len(CASES)))
@pytest.mark.parametrize("members", ["all", "inner"])
def test_prefix_step_parity(pkv, orc, case, members):
    n_q, n_kv, d, prefix, ctx = CASES[case]
    sh = _shape(n_q, n_kv, d, prefix)
    hc = w.host_case(sh, 300 + case, context_lens=ctx, share=True)
    B = len(ctx)
    first, count = (0, B) if members == "all" else (1, B - 2)
    a, b = DevCase(hc), DevCase(hc)
    got = _prefix_step(pkv, a, first, count)
    ref = gpu_step(pkv, b, fused=True)
    assert int(a.err.item()) == 0
    assert np.isfinite(got).all()
    want, rc, k_ref, v_ref = oracle_step(orc, hc)
    assert rc == 0
    err_o = max_abs(got, want)
    err_d = max_abs(got, ref)
    print(f"case {CASES[case][:4]} members {members}: vs oracle {err_o:.2e}, "
          f"vs pkv_decode_step {err_d:.2e}")
    assert err_o <= TOL
    assert err_d <= CROSS
    assert np.array_equal(to_host_u16(a.k_pool), to_host_u16(b.k_pool))
    assert np.array_equal(to_host_u16(a.v_pool), to_host_u16(b.v_pool))
    assert np.array_equal(to_host_u16(a.k_pool), k_ref)
    assert np.array_equal(to_host_u16(a.v_pool), v_ref)


def test_member_table_mismatch_flagged(pkv, orc):
    """A member past the prefix whose table holds another block inside the
    prefix range (here a block of another sequence, other values): the
    device check catches it, its rows are NaN and PKV_DEVERR_PREFIX is set;
    every other row is unaffected (oracle on the same tables)."""
    n_q, n_kv, d, prefix, ctx = CASES[0]
    hc = w.host_case(_shape(n_q, n_kv, d, prefix), 313, context_lens=ctx, share=True)
    bt = hc.tables.block_tables
    s, t = 4, 6                      # contexts 1000 and 4000: both past the prefix
    bt[s, 2] = bt[t, 40]             # a block of sequence t's own tokens
    assert bt[s, 2] != hc.tables.prefix_phys[2]
    dc = DevCase(hc)
    got = _prefix_step(pkv, dc)
    assert int(dc.err.item()) == pkv.PKV_DEVERR_PREFIX
    assert np.isnan(got[s]).all()
    others = np.arange(len(ctx)) != s
    assert np.isfinite(got[others]).all()
    want, rc, _, _ = oracle_step(orc, hc)
    assert rc == 0
    print(f"mismatch: other rows vs oracle {max_abs(got[others], want[others]):.2e}")
    assert max_abs(got[others], want[others]) <= TOL
    ref = gpu_step(pkv, DevCase(hc), fused=True)
    assert max_abs(got[others], ref[others]) <= CROSS


def test_empty_prefix_is_decode_step(pkv):
    """No members, or no prefix blocks: the same kernels as pkv_decode_step,
    the same bits."""
    n_q, n_kv, d, prefix, ctx = CASES[0]
    hc = w.host_case(_shape(n_q, n_kv, d, prefix), 310, context_lens=ctx, share=True)
    ref = gpu_step(pkv, DevCase(hc), fused=True)
    got = _prefix_step(pkv, DevCase(hc), 0, 0)
    assert np.array_equal(got, ref)
    got = _prefix_step(pkv, DevCase(hc), 0, len(ctx), table=np.zeros(0, np.int32))
    assert np.array_equal(got, ref)


def test_prefix_host_errors(pkv):
    import torch
    n_q, n_kv, d, prefix, ctx = CASES[1]
    hc = w.host_case(_shape(n_q, n_kv, d, prefix), 311, context_lens=ctx, share=True)
    dc = DevCase(hc)
    B = len(ctx)
    pt = to_dev_i32(hc.tables.prefix_phys)
    for first, count in ((-1, 2), (0, B + 1), (B, 1), (2, -1)):
        with pytest.raises(pkv.PkvError) as e:
            pkv.pkv_decode_step_prefix(dc.out, dc.q, dc.k_new, dc.v_new, dc.k_pool, dc.v_pool,
                                       dc.bt, dc.cl, hc.shape.scale, dc.max_ctx, pt, first, count)
        assert e.value.status == pkv.PKV_EINVAL
    long_table = torch.zeros(dc.bt.shape[1] + 1, dtype=torch.int32, device="cuda")
    with pytest.raises(pkv.PkvError) as e:
        pkv.pkv_decode_step_prefix(dc.out, dc.q, dc.k_new, dc.v_new, dc.k_pool, dc.v_pool, dc.bt,
                                   dc.cl, hc.shape.scale, dc.max_ctx, long_table, 0, B)
    assert e.value.status == pkv.PKV_EINVAL
    need = pkv.pkv_decode_prefix_workspace_bytes(B, n_q, n_kv, d, dc.max_ctx, len(pt), B)
    small = torch.empty(need - 1, dtype=torch.uint8, device="cuda")
    with pytest.raises(pkv.PkvError) as e:
        pkv.pkv_decode_step_prefix(dc.out, dc.q, dc.k_new, dc.v_new, dc.k_pool, dc.v_pool, dc.bt,
                                   dc.cl, hc.shape.scale, dc.max_ctx, pt, 0, B, workspace=small)
    assert e.value.status == pkv.PKV_EWORKSPACE
    torch.cuda.synchronize()
    assert int(dc.err.item()) == 0


def test_prefix_bad_block_id(pkv):
    """An id outside the pool inside the prefix, in the prefix table and in
    the tables of the sequences holding that block: flagged, and the same
    rows are NaN as with pkv_decode_step on the same tables (the members
    through the prefix units, the short sequences through their own
    tables); the other rows agree; nothing is read out of bounds."""
    n_q, n_kv, d, prefix, ctx = CASES[0]
    hc = w.host_case(_shape(n_q, n_kv, d, prefix), 312, context_lens=ctx, share=True)
    bad = hc.tables.num_blocks + 5
    table = hc.tables.prefix_phys.copy()
    bt = hc.tables.block_tables
    holders = bt[:, 3] == table[3]
    assert holders.sum() >= 3
    bt[holders, 3] = bad
    table[3] = bad
    dr = DevCase(hc)
    ref = gpu_step(pkv, dr, fused=True)
    assert int(dr.err.item()) & pkv.PKV_DEVERR_BLOCK_ID
    dc = DevCase(hc)
    got = _prefix_step(pkv, dc, 0, len(ctx), table=table)
    assert int(dc.err.item()) & pkv.PKV_DEVERR_BLOCK_ID
    nan_rows = np.isnan(got).all(axis=(1, 2))
    assert np.array_equal(nan_rows, holders)
    assert np.array_equal(np.isnan(ref).all(axis=(1, 2)), holders)
    assert np.isfinite(got[~holders]).all()
    assert max_abs(got[~holders], ref[~holders]) <= CROSS


def test_prefix_llama3_shape(pkv, orc):
    """The LLaMA-3-8B layer at full size (64 sequences, contexts U[1024, 8192],
    2,048-token prefix): within CROSS of pkv_decode_step everywhere, pools
    equal, and sampled rows within 1e-3 of the oracle."""
    import torch
    cfg = w.CONFIGS[4]
    shape = w.Shape(cfg.name, 1, cfg.n_q, cfg.n_kv, cfg.d, cfg.batch, cfg.ctx_lo, cfg.ctx_hi,
                    prefix_tokens=cfg.prefix_tokens)
    seed = 77
    cl0 = w.context_lengths(shape, seed)
    max_ctx = int(cl0.max())
    t = w.build_tables(shape, seed, share=True, max_blocks=math.ceil(max_ctx / w.BLOCK))
    ks, vs = w.pool_shapes(t.num_blocks, shape.n_kv, shape.d)
    k_pool = w.device_normal_bf16_(torch.empty(ks, dtype=torch.bfloat16, device="cuda"), 771)
    v_pool = w.device_normal_bf16_(torch.empty(vs, dtype=torch.bfloat16, device="cuda"), 772)
    if len(t.copies):
        dst = torch.from_numpy(t.copies[:, 0].astype(np.int64)).cuda()
        src = torch.from_numpy(t.copies[:, 1].astype(np.int64)).cuda()
        k_pool[dst] = k_pool[src]
        v_pool[dst] = v_pool[src]
    B = len(t.context_lens)
    g = w.rng(seed, 3)
    q_h = w.normal_bf16(g, (B, shape.n_q, shape.d))
    kn_h = w.normal_bf16(g, (B, shape.n_kv, shape.d))
    vn_h = w.normal_bf16(g, (B, shape.n_kv, shape.d))
    dev = lambda a: torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    q, k_new, v_new = dev(q_h), dev(kn_h), dev(vn_h)
    bt = to_dev_i32(t.block_tables)
    cl = to_dev_i32(t.context_lens)
    pt = to_dev_i32(t.prefix_phys)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    k2, v2 = k_pool.clone(), v_pool.clone()
    out = torch.full((B, shape.n_q, shape.d), float("nan"), dtype=torch.float32, device="cuda")
    ref = torch.full_like(out, float("nan"))
    torch.cuda.synchronize()
    k_ref, v_ref = to_host_u16(k_pool), to_host_u16(v_pool)
    print(f"llama3 shape: {t.num_blocks} blocks, prefix {len(t.prefix_phys)} blocks", flush=True)

    pkv.pkv_decode_step_prefix(out, q, k_new, v_new, k_pool, v_pool, bt, cl, shape.scale, max_ctx,
                               pt, 0, B, err_flag=err)
    pkv.pkv_decode_step(ref, q, k_new, v_new, k2, v2, bt, cl, shape.scale, max_ctx, err_flag=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    got = out.cpu().numpy().astype(np.float64)
    assert np.isfinite(got).all()
    err_d = max_abs(got, ref.cpu().numpy().astype(np.float64))
    assert torch.equal(k_pool, k2) and torch.equal(v_pool, v2)
    assert orc.kv_append(k_ref, v_ref, kn_h, vn_h, t.block_tables, t.context_lens) == 0
    assert np.array_equal(to_host_u16(k_pool), k_ref)

    cl_h = t.context_lens
    pick = w.rng(seed, 9)
    seqs = [int(np.argmin(cl_h)), int(np.argmax(cl_h))] + [int(pick.integers(B)) for _ in range(14)]
    G = shape.n_q // shape.n_kv
    worst = 0.0
    for s in seqs:
        j = int(pick.integers(shape.n_q))
        want, rc = orc.decode_row(q_h[s, j], k_ref, v_ref, t.block_tables[s], int(cl_h[s]),
                                  shape.n_kv, j // G, shape.scale)
        assert rc == 0
        worst = max(worst, max_abs(got[s, j], want))
    print(f"llama3 shape: vs pkv_decode_step {err_d:.2e}, {len(seqs)} oracle rows {worst:.2e}")
    assert err_d <= CROSS
    assert worst <= TOL


def test_prefix_step_in_graph(pkv):
    """The call captured in a HIP graph and replayed with new inputs between
    replays: every replay equals an eager call on the same state, bit for
    bit."""
    import torch
    n_q, n_kv, d, prefix, ctx = CASES[0]
    hc = w.host_case(_shape(n_q, n_kv, d, prefix), 314, context_lens=ctx, share=True)
    dc = DevCase(hc)
    B = len(ctx)
    pt = to_dev_i32(hc.tables.prefix_phys)
    ws = torch.zeros(pkv.pkv_decode_prefix_workspace_bytes(B, n_q, n_kv, d, dc.max_ctx, len(pt), B),
                     dtype=torch.uint8, device="cuda")
    out_ref = torch.empty_like(dc.out)
    assert pkv.pkv_decode_split_waves(B, n_q, n_kv, d, dc.max_ctx) > 0
    # one eager call first (device queries behind the split are cached outside capture)
    pkv.pkv_decode_step_prefix(out_ref, dc.q, dc.k_new, dc.v_new, dc.k_pool, dc.v_pool, dc.bt,
                               dc.cl, hc.shape.scale, dc.max_ctx, pt, 0, B, workspace=ws,
                               err_flag=dc.err)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        pkv.prepare_decode_step_prefix(dc.out, dc.q, dc.k_new, dc.v_new, dc.k_pool, dc.v_pool,
                                       dc.bt, dc.cl, hc.shape.scale, dc.max_ctx, pt, 0, B,
                                       workspace=ws, err_flag=dc.err)()
    rng = w.rng(315, 0)
    for rep in range(4):
        dc.q.copy_(to_dev_bf16(w.normal_bf16(rng, tuple(dc.q.shape))))
        dc.k_new.copy_(to_dev_bf16(w.normal_bf16(rng, tuple(dc.k_new.shape))))
        dc.v_new.copy_(to_dev_bf16(w.normal_bf16(rng, tuple(dc.v_new.shape))))
        dc.out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = dc.out.cpu().numpy()
        pkv.pkv_decode_step_prefix(out_ref, dc.q, dc.k_new, dc.v_new, dc.k_pool, dc.v_pool, dc.bt,
                                   dc.cl, hc.shape.scale, dc.max_ctx, pt, 0, B, workspace=ws,
                                   err_flag=dc.err)
        torch.cuda.synchronize()
        assert int(dc.err.item()) == 0
        assert np.isfinite(got).all(), f"replay {rep}"
        assert np.array_equal(got, out_ref.cpu().numpy()), f"replay {rep} differs from eager"
