"""The decode's partition kernel with its scores and P.V on the vector ALUs
(pkv_decode_step_partition_valu), kept to measure what the matrix cores
buy. Its results are held to the same bar as the matrix path: every row
within 1e-3 of the oracle, the pools bit-exact after the append; bad block
ids and context lengths caught the same way. Shapes: 1 to 8 query heads per
KV head (3, 6 and 7 run on the next compiled row count, the extra rows
dropped), both head sizes, ragged and one-token contexts, more
waves than tiles, and the benchmark's LLaMA-3-8B and 80-layer layers at
full size (rows sampled). The shaped-score cases of the rescale tests
(late jumps, early peaks, staircases, large scales) drive its running
maximum and rescale as they do the matrix path's."""
import numpy as np
import pytest

import rescale_cases as rc
import workload as w
from gpu_util import TOL, DevCase, max_abs, oracle_step, to_dev_i32, to_host_u16

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pkv():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import paged_kv_cache_468_amd as lib
    return lib


def _shape(n_q, n_kv, d):
    return w.Shape(f"{n_q}/{n_kv} d{d}", 1, n_q, n_kv, d, 1, 1, 1)


def _valu_step(pkv, dc, max_ctx=None, scale=None):
    import torch
    max_ctx = dc.max_ctx if max_ctx is None else max_ctx
    sc = dc.hc.shape.scale if scale is None else scale
    ws = pkv.pkv_decode_step_partition_valu(dc.out, dc.q, dc.k_new, dc.v_new, dc.k_pool,
                                            dc.v_pool, dc.bt, dc.cl, sc, max_ctx, err_flag=dc.err)
    pkv.pkv_paged_attn_merge(dc.out, dc.q, dc.k_pool, dc.v_pool, dc.bt, dc.cl, sc, max_ctx,
                             workspace=ws, err_flag=dc.err)
    torch.cuda.synchronize()
    return dc.out.cpu().numpy().astype(np.float64)


CASES = [  # n_q, n_kv, d, contexts
    (20, 4, 64, [1, 16, 17, 300, 1000, 2048]),
    (32, 32, 128, [4096, 1, 15, 700]),          # G = 1
    (32, 8, 128, [1024, 8192, 3000, 17, 5]),    # G = 4
    (64, 8, 128, [8000, 8000, 100]),            # G = 8
    (8, 1, 128, [123, 456, 789]),               # MQA, G = 8
    (6, 3, 64, [2, 33, 64, 65, 129]),           # G = 2
    (12, 4, 128, [700, 31, 1]),                 # G = 3 (compiled as 4 rows)
    (24, 4, 64, [500, 17, 2000]),               # G = 6 (as 8)
    (14, 2, 128, [1500, 64, 9]),                # G = 7 (as 8)
]


@pytest.mark.parametrize("case", range(len(CASES)))
def test_valu_matches_oracle(pkv, orc, case):
    n_q, n_kv, d, ctx = CASES[case]
    print(f"case {CASES[case]}", flush=True)
    hc = w.host_case(_shape(n_q, n_kv, d), 2500 + case, context_lens=ctx, spare_blocks=3)
    dc = DevCase(hc)
    got = _valu_step(pkv, dc)
    want, rc, k_ref, v_ref = oracle_step(orc, hc)
    assert rc == 0 and int(dc.err.item()) == 0
    assert np.array_equal(to_host_u16(dc.k_pool), k_ref)
    assert np.array_equal(to_host_u16(dc.v_pool), v_ref)
    assert np.isfinite(got).all()
    e = max_abs(got, want)
    print(f"  max-abs {e:.2e}", flush=True)
    assert e <= TOL


RESCALE = [(p, shape, 9100 + i) for i, (p, shape) in enumerate(
    [(p, "g4d128") for p in rc.PROFILES] + [(p, "g5d64") for p in rc.PROFILES]
    + [(p, "g8d128long") for p in ("late_jump", "staircase", "scale_8")])]


@pytest.mark.parametrize("profile,shape_name,seed", RESCALE)
def test_valu_rescale(pkv, orc, profile, shape_name, seed):
    print(f"valu {profile} {shape_name} seed {seed}", flush=True)
    case = rc.decode_case(profile, shape_name, seed)
    dc = DevCase(case.hc)
    got = _valu_step(pkv, dc, scale=case.scale)
    want, rc_, k_ref, v_ref = oracle_step(orc, case.hc, scale=case.scale)
    assert rc_ == 0 and int(dc.err.item()) == 0
    assert np.array_equal(to_host_u16(dc.k_pool), k_ref)
    assert np.array_equal(to_host_u16(dc.v_pool), v_ref)
    keep = rc.conditioned_rows(case)
    assert int((~keep).sum()) <= 0.2 * keep.size
    assert np.isfinite(got).all()
    e = max_abs(got[keep], want[keep])
    print(f"  max-abs {e:.2e} over {int(keep.sum())} rows", flush=True)
    assert e <= TOL


def test_valu_more_waves_than_tiles(pkv, orc):
    hc = w.host_case(_shape(32, 8, 128), 2550, context_lens=[1, 17, 40, 300], max_blocks=1024)
    dc = DevCase(hc)
    got = _valu_step(pkv, dc, max_ctx=16 * 1024)
    want, rc, _, _ = oracle_step(orc, hc)
    assert rc == 0 and int(dc.err.item()) == 0
    assert max_abs(got, want) <= TOL


def test_valu_device_errors(pkv):
    """A bad block id and an invalid context length: flagged, NaN rows,
    the other rows finite."""
    hc = w.host_case(_shape(8, 2, 128), 2560, context_lens=[40, 90, 300, 77])
    bt = hc.tables.block_tables.copy()
    bt[1, 2] = hc.tables.num_blocks + 3
    cl = hc.tables.context_lens.copy()
    cl[2] = 0
    dc = DevCase(hc)
    dc.bt = to_dev_i32(bt)
    dc.cl = to_dev_i32(cl)
    got = _valu_step(pkv, dc)
    err = int(dc.err.item())
    assert err & pkv.PKV_DEVERR_BLOCK_ID and err & pkv.PKV_DEVERR_CONTEXT
    assert np.isnan(got[1]).all() and np.isnan(got[2]).all()
    assert np.isfinite(got[[0, 3]]).all()


def test_valu_refuses_large_groups(pkv):
    hc = w.host_case(_shape(32, 2, 128), 2570, context_lens=[40, 90])   # G = 16
    dc = DevCase(hc)
    with pytest.raises(pkv.PkvError) as info:
        _valu_step(pkv, dc)
    assert info.value.status == pkv.PKV_EUNSUPPORTED


@pytest.mark.parametrize("cfg", [4, 5])
def test_valu_full_size_layer(pkv, orc, cfg):
    """One layer of the LLaMA-3-8B (private copies) and 80-layer shapes at
    full size: the pools bit-exact after the append, 64 sampled rows
    recomputed by the oracle one by one."""
    import torch
    full = w.CONFIGS[cfg]
    shape = w.Shape(full.name, 1, full.n_q, full.n_kv, full.d, full.batch, full.ctx_lo,
                    full.ctx_hi)
    seed = 2580 + cfg
    t = w.build_tables(shape, seed, share=False)
    ks, vs = w.pool_shapes(t.num_blocks, shape.n_kv, shape.d)
    kp = w.device_normal_bf16_(torch.empty(ks, dtype=torch.bfloat16, device="cuda"), seed * 10 + 1)
    vp = w.device_normal_bf16_(torch.empty(vs, dtype=torch.bfloat16, device="cuda"), seed * 10 + 2)
    B, G, D = len(t.context_lens), shape.n_q // shape.n_kv, shape.d
    g = w.rng(seed, 3)
    q_h = w.normal_bf16(g, (B, shape.n_q, D))
    kn_h = w.normal_bf16(g, (B, shape.n_kv, D))
    vn_h = w.normal_bf16(g, (B, shape.n_kv, D))
    dev = lambda a: torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    out = torch.full((B, shape.n_q, D), float("nan"), dtype=torch.float32, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    bt, cl = to_dev_i32(t.block_tables), to_dev_i32(t.context_lens)
    max_ctx = int(t.context_lens.max())
    torch.cuda.synchronize()
    k_ref, v_ref = to_host_u16(kp), to_host_u16(vp)
    ws = pkv.pkv_decode_step_partition_valu(out, dev(q_h), dev(kn_h), dev(vn_h), kp, vp, bt, cl,
                                            shape.scale, max_ctx, err_flag=err)
    pkv.pkv_paged_attn_merge(out, dev(q_h), kp, vp, bt, cl, shape.scale, max_ctx, workspace=ws,
                             err_flag=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    assert orc.kv_append(k_ref, v_ref, kn_h, vn_h, t.block_tables, t.context_lens) == 0
    assert np.array_equal(to_host_u16(kp), k_ref) and np.array_equal(to_host_u16(vp), v_ref)
    got = out.cpu().numpy().astype(np.float64)
    assert np.isfinite(got).all()
    pick = w.rng(seed, 9)
    worst = 0.0
    for _ in range(64):
        s, j = int(pick.integers(B)), int(pick.integers(shape.n_q))
        want, rc = orc.decode_row(q_h[s, j], k_ref, v_ref, t.block_tables[s],
                                  int(t.context_lens[s]), shape.n_kv, j // G, shape.scale)
        assert rc == 0
        worst = max(worst, max_abs(got[s, j], want))
    print(f"config {cfg}: 64 sampled rows, max-abs {worst:.2e}", flush=True)
    assert worst <= TOL
