"""Parity of the HIP path (through the C ABI) with the CPU oracle.

Small cases span several 16-token tiles, several partitions and ragged
tails; values are N(0,1) bf16, unused slots and blocks hold NaN. The bar:
kv_append and copy_blocks bit-exact, decode max-abs error <= 1e-3 on fp32
outputs, and the invariants (block permutation, shared prefix vs private
copies) bitwise on the GPU.
"""
import numpy as np
import pytest

import workload as w
from gpu_util import TOL, DevCase, gpu_step, max_abs, oracle_step, to_dev_i32, to_host_u16

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pkv():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import paged_kv_cache_468_amd as lib
    return lib


def _shape(n_q, n_kv, d, prefix=0):
    return w.Shape(f"{n_q}/{n_kv} d{d}", 1, n_q, n_kv, d, 1, 1, 1, prefix_tokens=prefix)


def _check_case(pkv, orc, hc, partition=0, scale=None, fused=False):
    dc = DevCase(hc)
    got = gpu_step(pkv, dc, partition=partition, scale=scale, fused=fused)
    want, rc, k_ref, v_ref = oracle_step(orc, hc, scale=scale)
    assert rc == 0
    assert int(dc.err.item()) == 0
    assert np.array_equal(to_host_u16(dc.k_pool), k_ref), "kv_append K pool differs"
    assert np.array_equal(to_host_u16(dc.v_pool), v_ref), "kv_append V pool differs"
    assert np.isfinite(got).all()
    err = max_abs(got, want)
    assert err <= TOL, err
    return got, err


def test_tiny_config(pkv, orc):
    """The tiny single-layer shape: 20 q / 4 KV heads, d 64, contexts
    17/40/77/130 in a 64-block pool with randomly permuted ids."""
    hc = w.host_case(w.CONFIGS[1], 0)
    for part in (0, 16, 64, 1024):
        _, err = _check_case(pkv, orc, hc, partition=part)
        print(f"tiny config partition {part}: max-abs {err:.2e}")


CASES = [  # n_q, n_kv, d, contexts, partition
    (20, 4, 64, [1, 16, 17, 300, 1000], 0),
    (20, 4, 64, [513, 2048, 31, 1500], 128),
    (32, 32, 128, [4096, 1, 15, 700], 0),
    (32, 8, 128, [1024, 8192, 3000, 17], 512),
    (32, 8, 128, [2049, 33, 64, 65], 16),
    (64, 8, 128, [8000, 8000, 100], 256),
    (8, 1, 128, [123, 456, 789], 64),          # MQA
    (16, 1, 64, [50, 1023, 1024, 1025], 1024),  # G = 16: one full MFMA block of rows
    (40, 2, 128, [333, 77], 64),               # G = 20: two query groups
    (12, 4, 128, [1, 2, 3, 4, 5], 0),          # tiny contexts, G = 3
]


@pytest.mark.parametrize("fused", [False, True], ids=["append+decode", "decode_step"])
@pytest.mark.parametrize("case", range(len(CASES)))
def test_random_shapes(pkv, orc, case, fused):
    n_q, n_kv, d, ctx, part = CASES[case]
    hc = w.host_case(_shape(n_q, n_kv, d), 1000 + case, context_lens=ctx, spare_blocks=5)
    _, err = _check_case(pkv, orc, hc, partition=part, fused=fused)
    print(f"case {CASES[case]}: max-abs {err:.2e}")


@pytest.mark.parametrize("case", [0, 2, 3, 6])
def test_matches_fp32_oracle(pkv, orc, case):
    """The same cases against the naive fp32 loop (the oracle's
    single-precision twin) as well: within 1e-3 of it too, and the two
    oracles within 1e-5 of each other."""
    n_q, n_kv, d, ctx, part = CASES[case]
    hc = w.host_case(_shape(n_q, n_kv, d), 3000 + case, context_lens=ctx, spare_blocks=3)
    got, _ = _check_case(pkv, orc, hc, partition=part, fused=True)
    want64, _, k_ref, v_ref = oracle_step(orc, hc)
    want32, rc = orc.decode_f32(hc.q, k_ref, v_ref, hc.tables.block_tables,
                                hc.tables.context_lens, n_kv, hc.shape.scale)
    assert rc == 0
    want32 = want32.astype(np.float64)
    e32, twin = max_abs(got, want32), max_abs(want32, want64)
    print(f"case {case}: max-abs vs fp32 oracle {e32:.2e}, fp32 vs float64 oracle {twin:.2e}")
    assert e32 <= TOL and twin <= 1e-5


def test_partition_merge_agrees(pkv, orc):
    """Different partition sizes only change where the running softmax is
    split; the merged results agree to fp32 rounding."""
    hc = w.host_case(_shape(32, 8, 128), 77, context_lens=[1000, 777, 64, 1024])
    outs = []
    for part in (16, 64, 512, 1024, 0):
        dc = DevCase(hc)
        outs.append(gpu_step(pkv, dc, partition=part))
    for o in outs[1:]:
        assert max_abs(o, outs[0]) <= 1e-5


def test_block_permutation_bitwise(pkv):
    sh = _shape(20, 4, 64)
    a = DevCase(w.host_case(sh, 21, context_lens=[17, 40, 77, 130, 600], permute=False))
    b = DevCase(w.host_case(sh, 21, context_lens=[17, 40, 77, 130, 600], permute=True))
    oa = gpu_step(pkv, a, partition=64)
    ob = gpu_step(pkv, b, partition=64)
    assert np.array_equal(oa, ob)


def test_shared_prefix_bitwise(pkv, orc):
    """Shared prefix blocks give bitwise the same outputs as private copies
    of the same bytes (the LLaMA-3-8B sharing rule at a small size)."""
    sh = _shape(32, 8, 128, prefix=256)
    ctx = [100, 256, 257, 1000, 2048]
    a = DevCase(w.host_case(sh, 31, context_lens=ctx, share=True))
    b = DevCase(w.host_case(sh, 31, context_lens=ctx, share=False))
    assert a.hc.tables.num_blocks < b.hc.tables.num_blocks
    oa = gpu_step(pkv, a, partition=128)
    ob = gpu_step(pkv, b, partition=128)
    assert np.array_equal(oa, ob)
    want, _, _, _ = oracle_step(orc, a.hc)
    assert max_abs(oa, want) <= TOL


def test_single_token_is_value(pkv):
    """ctx = 1: the output is the appended token's value, exactly."""
    hc = w.host_case(_shape(8, 2, 128), 3, context_lens=[1, 1, 1])
    dc = DevCase(hc)
    got = gpu_step(pkv, dc)
    v = w.bf16_to_f32(hc.v_new).astype(np.float64)            # [B, n_kv, d]
    assert np.array_equal(got, np.repeat(v, 4, axis=1))


def test_constant_values(pkv):
    hc = w.host_case(_shape(32, 8, 128), 4, context_lens=[7, 16, 1000, 4097])
    c = w.bf16_bits(np.array([-2.375], np.float32))[0]
    hc.v_pool[hc.tables.used] = c
    hc.v_new[:] = c
    w.fill_unused_nan(hc.k_pool, hc.v_pool, hc.tables)
    got = gpu_step(pkv, DevCase(hc))
    assert np.abs(got + 2.375).max() <= 1e-4


def test_equal_keys_give_mean(pkv, orc):
    hc = w.host_case(_shape(8, 2, 64), 6, context_lens=[15, 16, 17, 33, 700])
    for s in range(len(hc.tables.context_lens)):
        kc, vc = w.gather_contiguous(hc.k_pool, hc.v_pool, hc.tables, s)
        kc[:] = hc.k_new[s][:, None, :]                        # every key = the new key
        w.scatter_contiguous(kc, vc, hc.tables, s, hc.k_pool, hc.v_pool)
    got = gpu_step(pkv, DevCase(hc), partition=64)
    for s, ctx in enumerate(hc.tables.context_lens):
        _, vc = w.gather_contiguous(hc.k_pool, hc.v_pool, hc.tables, s)
        vc[:, ctx - 1, :] = hc.v_new[s]
        mean = w.bf16_to_f32(vc).astype(np.float64).mean(axis=1)
        assert np.abs(got[s] - np.repeat(mean, 4, axis=0)).max() <= 1e-4


def test_copy_blocks_bitwise(pkv, orc):
    import torch
    hc = w.host_case(_shape(32, 8, 128), 8, context_lens=[100, 300], spare_blocks=6, nan_fill=False)
    dc = DevCase(hc)
    free = np.nonzero(~hc.tables.used)[0].astype(np.int32)
    src = hc.tables.block_tables[:, :3].reshape(-1)[:5].astype(np.int32)
    dst = free[:5]
    pkv.pkv_copy_blocks(dc.k_pool, dc.v_pool, to_dev_i32(src), to_dev_i32(dst), err_flag=dc.err)
    torch.cuda.synchronize()
    k, v = hc.k_pool.copy(), hc.v_pool.copy()
    assert orc.copy_blocks(k, v, src, dst, 8, 128) == 0
    assert np.array_equal(to_host_u16(dc.k_pool), k)
    assert np.array_equal(to_host_u16(dc.v_pool), v)
    assert int(dc.err.item()) == 0


def test_device_errors_flagged(pkv):
    """Bad block ids and bad context lengths are caught by the kernels'
    own checks: the error bit is set, the affected rows are NaN, nothing
    else changes, nothing is read out of bounds."""
    import torch
    sh = _shape(8, 2, 128)
    hc = w.host_case(sh, 9, context_lens=[40, 90, 300])
    ref = gpu_step(pkv, DevCase(hc), partition=64, append=False)
    for part in (64, 1024, 0):
        bt = hc.tables.block_tables.copy()
        bt[1, 2] = hc.tables.num_blocks + 7
        dc = DevCase(hc)
        dc.bt = to_dev_i32(bt)
        got = gpu_step(pkv, dc, partition=part, append=False)
        assert int(dc.err.item()) & pkv.PKV_DEVERR_BLOCK_ID
        assert np.isnan(got[1]).all()
        assert np.abs(got[[0, 2]] - ref[[0, 2]]).max() <= 1e-5
        cl = hc.tables.context_lens.copy()
        cl[2] = 0
        dc = DevCase(hc)
        dc.cl = to_dev_i32(cl)
        got = gpu_step(pkv, dc, partition=part, append=False)
        assert int(dc.err.item()) & pkv.PKV_DEVERR_CONTEXT
        assert np.isnan(got[2]).all() and np.isfinite(got[:2]).all()
    # append with a bad id leaves the pools untouched
    bt = hc.tables.block_tables.copy()
    bt[0, (40 - 1) // 16] = -3
    dc = DevCase(hc)
    dc.bt = to_dev_i32(bt)
    k0 = to_host_u16(dc.k_pool)
    pkv.pkv_kv_append(dc.k_pool, dc.v_pool, dc.k_new[:1].contiguous(), dc.v_new[:1].contiguous(),
                      dc.bt[:1].contiguous(), dc.cl[:1].contiguous(), err_flag=dc.err)
    torch.cuda.synchronize()
    assert int(dc.err.item()) & pkv.PKV_DEVERR_BLOCK_ID
    assert np.array_equal(to_host_u16(dc.k_pool), k0)


@pytest.mark.parametrize("part", [128, 0])
def test_decode_equals_partition_then_merge(pkv, part):
    import torch
    hc = w.host_case(_shape(32, 8, 128), 12, context_lens=[900, 40, 2000])
    a = DevCase(hc)
    b = DevCase(hc)
    oa = gpu_step(pkv, a, partition=part, append=False)
    ws = pkv.pkv_paged_attn_partition(b.out, b.q, b.k_pool, b.v_pool, b.bt, b.cl, 1 / 128 ** 0.5,
                                      b.max_ctx, partition_tokens=part)
    pkv.pkv_paged_attn_merge(b.out, b.q, b.k_pool, b.v_pool, b.bt, b.cl, 1 / 128 ** 0.5,
                             b.max_ctx, partition_tokens=part, workspace=ws)
    torch.cuda.synchronize()
    assert np.array_equal(oa, b.out.cpu().numpy().astype(np.float64))


@pytest.mark.parametrize("ctx", [[1, 2, 3], [1, 17, 40, 300], [5000, 1, 1, 1, 33]])
def test_balanced_split_more_waves_than_tiles(pkv, orc, ctx):
    """A max_context_len far above the actual contexts: the balanced split
    then has more waves than tiles, and waves with empty ranges inside a
    unit must leave neutral partials for the merge."""
    hc = w.host_case(_shape(32, 8, 128), 50 + len(ctx), context_lens=ctx, max_blocks=1024)
    dc = DevCase(hc)
    got = gpu_step(pkv, dc, partition=0, max_ctx=16 * 1024)
    want, rc, _, _ = oracle_step(orc, hc)
    assert rc == 0 and int(dc.err.item()) == 0
    assert max_abs(got, want) <= TOL


def test_balanced_split_uneven_mix(pkv, orc):
    """Many short sequences next to a few long ones: wave ranges cross many
    unit boundaries in both directions."""
    rnd = np.random.default_rng(5)
    ctx = list(rnd.integers(1, 40, size=45)) + [3000, 2500, 1, 16, 17, 4095]
    hc = w.host_case(_shape(20, 4, 64), 61, context_lens=ctx)
    got = gpu_step(pkv, DevCase(hc), partition=0)
    want, rc, _, _ = oracle_step(orc, hc)
    assert rc == 0
    assert max_abs(got, want) <= TOL


@pytest.mark.parametrize("part", [0, 128])
@pytest.mark.parametrize("shape", [(32, 8, 128), (40, 2, 128), (20, 4, 64), (8, 1, 128)])
def test_decode_step_equals_append_then_decode(pkv, shape, part):
    """pkv_decode_step (one kernel with the balanced split), and its two
    halves (pkv_decode_step_partition, pkv_paged_attn_merge), against
    pkv_kv_append + pkv_paged_attn_decode: pools and outputs bit for bit."""
    ctx = [1, 15, 16, 17, 300, 1000, 2049]
    hc = w.host_case(_shape(*shape), 90 + shape[0], context_lens=ctx, spare_blocks=3)
    a, b, c = DevCase(hc), DevCase(hc), DevCase(hc)
    oa = gpu_step(pkv, a, partition=part)
    ob = gpu_step(pkv, b, partition=part, fused=True)
    oc = gpu_step(pkv, c, partition=part, fused=True, halves=True)
    for x in (a, b, c):
        assert int(x.err.item()) == 0
    for x in (b, c):
        assert np.array_equal(to_host_u16(a.k_pool), to_host_u16(x.k_pool))
        assert np.array_equal(to_host_u16(a.v_pool), to_host_u16(x.v_pool))
    assert np.array_equal(oa, ob) and np.array_equal(oa, oc)


def test_workspace_needs_no_initialisation(pkv):
    """The workspace may hold anything before a call (here all bits set),
    and repeated calls on one workspace give the same bits."""
    import torch
    sh = _shape(32, 8, 128)
    ctx = [4000, 3000, 17, 1, 2500, 800]
    hc = w.host_case(sh, 95, context_lens=ctx)
    dc = DevCase(hc)
    B = len(ctx)
    for part in (0, 256):
        need = pkv.pkv_decode_workspace_bytes(B, 32, 8, 128, dc.max_ctx, part)
        ws = torch.full((need,), 255, dtype=torch.uint8, device="cuda")
        outs = []
        for _ in range(3):
            pkv.pkv_paged_attn_decode(dc.out, dc.q, dc.k_pool, dc.v_pool, dc.bt, dc.cl, sh.scale,
                                      dc.max_ctx, part, workspace=ws, err_flag=dc.err)
            torch.cuda.synchronize()
            outs.append(dc.out.cpu().numpy())
            ws.fill_(255)
        assert int(dc.err.item()) == 0
        assert np.isfinite(outs[0]).all()
        assert np.array_equal(outs[0], outs[1]) and np.array_equal(outs[0], outs[2])


def test_decode_step_device_errors(pkv):
    """Invalid context lengths and bad block ids through pkv_decode_step:
    flagged, NaN rows, other sequences unaffected, nothing appended for the
    bad sequences."""
    sh = _shape(8, 2, 128)
    hc = w.host_case(sh, 96, context_lens=[40, 90, 300, 77])
    ref = gpu_step(pkv, DevCase(hc), partition=0, fused=True)
    bt = hc.tables.block_tables.copy()
    bt[1, (90 - 1) // 16] = hc.tables.num_blocks + 3      # the block being written
    cl = hc.tables.context_lens.copy()
    cl[2] = 0
    dc = DevCase(hc)
    dc.bt = to_dev_i32(bt)
    dc.cl = to_dev_i32(cl)
    k0 = to_host_u16(dc.k_pool)
    got = gpu_step(pkv, dc, partition=0, fused=True)
    err = int(dc.err.item())
    assert err & pkv.PKV_DEVERR_BLOCK_ID and err & pkv.PKV_DEVERR_CONTEXT
    assert np.isnan(got[1]).all() and np.isnan(got[2]).all()
    # the split moves with the context lengths: the healthy rows agree to rounding
    assert np.abs(got[[0, 3]] - ref[[0, 3]]).max() <= 1e-5
    k1 = to_host_u16(dc.k_pool)
    # only sequences 0 and 3 were appended
    changed = np.nonzero((k0 != k1).any(axis=(1, 2, 3)))[0]
    expect = {int(hc.tables.block_tables[0, 39 // 16]), int(hc.tables.block_tables[3, 76 // 16])}
    assert set(int(b) for b in changed) <= expect


@pytest.mark.parametrize("B", [256, 257, 300])
def test_balanced_split_large_batches(pkv, orc, B):
    """Batches around and above 256 sequences, where the kernel switches from
    context lengths held in registers to chunked scans."""
    rnd = np.random.default_rng(B)
    ctx = list(rnd.integers(1, 200, size=B))
    hc = w.host_case(_shape(8, 2, 64), 300 + B, context_lens=ctx)
    for fused in (False, True):
        got = gpu_step(pkv, DevCase(hc), partition=0, fused=fused)
        want, rc, _, _ = oracle_step(orc, hc)
        assert rc == 0
        assert max_abs(got, want) <= TOL
