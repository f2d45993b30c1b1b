"""GPU parity where the online softmax rescales a live accumulator and the
merge combines partials whose maxima lie far apart.

"Scaling LLM serving", "Make attention itself cheaper": attention runs over
on-chip tiles without the score matrix ever being written, which is why the
kernels keep a running maximum, rescale the running sum and accumulator
when it rises, and merge partials over a sequence by their maxima. The
inputs (tests/rescale_cases.py) raise and lower the scores by tens to
thousands of log2 units along each sequence; tests/test_rescale_premises.py
shows, on the CPU and from the split's own formulas, that each case takes
the branches it is meant to take. Every path is compared with the oracle
element by element at 1e-3:
  * decode: pkv_decode_step (append fused), pkv_kv_append +
    pkv_paged_attn_decode, pkv_decode_step_partition + pkv_paged_attn_merge,
    fixed partitions of 16 and 64 tokens; pools bit-exact after the append;
  * pkv_decode_step_prefix (prefix units' partials merged with the
    members' own);
  * pkv_paged_attn_verify, with segments no query token but the last can
    see into (-inf partials);
  * pkv_paged_prefill.
At scale 100 rows whose two largest scores lie within 6 natural units are
left out of the element-wise comparison (their count is printed and
bounded): there the fp32 scores' rounding alone can move the output more
than the tolerance.
"""
import numpy as np
import pytest

import rescale_cases as rc
from gpu_util import (TOL, DevCase, gpu_step, max_abs, oracle_step, to_dev_bf16, to_dev_i32,
                      to_host_u16)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pkv():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import paged_kv_cache_468_amd as lib
    return lib


def _compare(case, got, want):
    keep = rc.conditioned_rows(case)
    left_out = int((~keep).sum())
    assert left_out <= 0.2 * keep.size, f"{left_out} of {keep.size} rows ill-conditioned"
    e = max_abs(got[keep], want[keep])
    print(f"  max-abs {e:.2e} over {int(keep.sum())} rows ({left_out} left out)", flush=True)
    assert np.isfinite(got).all()
    assert e <= TOL


@pytest.mark.parametrize("profile,path,shape_name,seed", rc.decode_specs())
def test_decode_rescale(pkv, orc, profile, path, shape_name, seed):
    print(f"decode {profile} {path} {shape_name} seed {seed}", flush=True)
    case = rc.decode_case(profile, shape_name, seed)
    dc = DevCase(case.hc)
    part = int(path[5:]) if path.startswith("fixed") else 0
    got = gpu_step(pkv, dc, partition=part, scale=case.scale,
                   fused=path in ("fused", "halves", "fixed64"), halves=path == "halves")
    want, rc_, k_ref, v_ref = oracle_step(orc, case.hc, scale=case.scale)
    assert rc_ == 0 and int(dc.err.item()) == 0
    assert np.array_equal(to_host_u16(dc.k_pool), k_ref)
    assert np.array_equal(to_host_u16(dc.v_pool), v_ref)
    _compare(case, got, want)


@pytest.mark.parametrize("profile,d,seed", rc.prefix_specs())
def test_prefix_rescale(pkv, orc, profile, d, seed):
    import torch
    print(f"prefix {profile} d {d} seed {seed}", flush=True)
    case, pre, first, count = rc.prefix_case(profile, d, seed)
    hc = case.hc
    dc = DevCase(hc)
    pkv.pkv_decode_step_prefix(dc.out, dc.q, dc.k_new, dc.v_new, dc.k_pool, dc.v_pool, dc.bt,
                               dc.cl, case.scale, dc.max_ctx, to_dev_i32(hc.tables.prefix_phys),
                               first, count, err_flag=dc.err)
    torch.cuda.synchronize()
    got = dc.out.cpu().numpy().astype(np.float64)
    want, rc_, k_ref, v_ref = oracle_step(orc, hc, scale=case.scale)
    assert rc_ == 0 and int(dc.err.item()) == 0
    assert np.array_equal(to_host_u16(dc.k_pool), k_ref)
    assert np.array_equal(to_host_u16(dc.v_pool), v_ref)
    _compare(case, got, want)


def _multi_token(pkv, orc, case, kernel):
    import torch
    hc = case.hc
    out = torch.full(case.qv.shape, float("nan"), dtype=torch.float32, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    args = (out, to_dev_bf16(case.qv), to_dev_bf16(hc.k_pool), to_dev_bf16(hc.v_pool),
            to_dev_i32(hc.tables.block_tables), to_dev_i32(hc.tables.context_lens), case.scale,
            int(hc.tables.context_lens.max()))
    if kernel == "verify":
        pkv.pkv_paged_attn_verify(*args, err_flag=err)
    else:
        pkv.pkv_paged_prefill(*args, err_flag=err)
    torch.cuda.synchronize()
    want, rc_ = orc.verify(case.qv, hc.k_pool, hc.v_pool, hc.tables.block_tables,
                           hc.tables.context_lens, hc.shape.n_kv, case.scale)
    assert rc_ == 0 and int(err.item()) == 0
    _compare(case, out.cpu().numpy().astype(np.float64), want)


@pytest.mark.parametrize("profile,q_len,d,seed", rc.verify_specs())
def test_verify_rescale(pkv, orc, profile, q_len, d, seed):
    print(f"verify {profile} q_len {q_len} d {d} seed {seed}", flush=True)
    _multi_token(pkv, orc, rc.verify_case(profile, q_len, d, seed), "verify")


@pytest.mark.parametrize("profile,chunk,d,seed", rc.prefill_specs())
def test_prefill_rescale(pkv, orc, profile, chunk, d, seed):
    print(f"prefill {profile} chunk {chunk} d {d} seed {seed}", flush=True)
    _multi_token(pkv, orc, rc.prefill_case(profile, chunk, d, seed), "prefill")
