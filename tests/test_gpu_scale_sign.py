"""The softmax scale at zero and below zero, on every attention path.

The kernels keep their running reference maximum on the scaled scores
(scale * log2 e * q.k), so the sign of the scale needs no special case; at
zero every score is 0 and each row is the plain mean of its visible values.
Both are checked against the oracle (which takes any finite scale) at the
usual bar: every row within 1e-3, the pools bit-exact after the append.
Paths: the fused decode step, append then decode (balanced split and fixed
64-token partitions), the vector-ALU partition kernel with the merge, the
verification pass and chunked prefill."""
import numpy as np
import pytest

import workload as w
from gpu_util import (TOL, DevCase, gpu_step, max_abs, oracle_step, to_dev_bf16, to_dev_i32,
                      to_host_u16)

pytestmark = pytest.mark.gpu

SCALES = [0.0, -0.125, -0.37]


@pytest.fixture(scope="module")
def pkv():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import paged_kv_cache_468_amd as lib
    return lib


def _shape(n_q, n_kv, d):
    return w.Shape(f"{n_q}/{n_kv} d{d}", 1, n_q, n_kv, d, 1, 1, 1)


@pytest.mark.parametrize("scale", SCALES)
@pytest.mark.parametrize("path", ["fused", "unfused", "fixed64", "valu"])
def test_decode_scale(pkv, orc, path, scale):
    import torch
    print(f"decode {path} scale {scale}", flush=True)
    shape = _shape(32, 8, 128) if path != "unfused" else _shape(20, 4, 64)
    hc = w.host_case(shape, 4100 + SCALES.index(scale), context_lens=[1, 17, 300, 2100, 64],
                     spare_blocks=2)
    dc = DevCase(hc)
    if path == "valu":
        ws = pkv.pkv_decode_step_partition_valu(dc.out, dc.q, dc.k_new, dc.v_new, dc.k_pool,
                                                dc.v_pool, dc.bt, dc.cl, scale, dc.max_ctx,
                                                err_flag=dc.err)
        pkv.pkv_paged_attn_merge(dc.out, dc.q, dc.k_pool, dc.v_pool, dc.bt, dc.cl, scale,
                                 dc.max_ctx, workspace=ws, err_flag=dc.err)
        torch.cuda.synchronize()
        got = dc.out.cpu().numpy().astype(np.float64)
    else:
        got = gpu_step(pkv, dc, partition=64 if path == "fixed64" else 0, scale=scale,
                       fused=path in ("fused", "fixed64"))
    want, rc, k_ref, v_ref = oracle_step(orc, hc, scale=scale)
    assert rc == 0 and int(dc.err.item()) == 0
    assert np.array_equal(to_host_u16(dc.k_pool), k_ref)
    assert np.array_equal(to_host_u16(dc.v_pool), v_ref)
    assert np.isfinite(got).all()
    e = max_abs(got, want)
    print(f"  max-abs {e:.2e}", flush=True)
    assert e <= TOL


@pytest.mark.parametrize("scale", SCALES)
@pytest.mark.parametrize("kernel,q_len", [("verify", 4), ("prefill", 40)])
def test_multi_token_scale(pkv, orc, kernel, q_len, scale):
    import torch
    print(f"{kernel} q_len {q_len} scale {scale}", flush=True)
    shape = _shape(32, 8, 128)
    hc = w.host_case(shape, 4200 + SCALES.index(scale), context_lens=[40, 77, 600, 1500],
                     spare_blocks=2)
    B = len(hc.tables.context_lens)
    qv = w.normal_bf16(w.rng(4200, 5), (B, q_len, shape.n_q, shape.d))
    out = torch.full(qv.shape, float("nan"), dtype=torch.float32, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    args = (out, to_dev_bf16(qv), to_dev_bf16(hc.k_pool), to_dev_bf16(hc.v_pool),
            to_dev_i32(hc.tables.block_tables), to_dev_i32(hc.tables.context_lens), scale,
            int(hc.tables.context_lens.max()))
    if kernel == "verify":
        pkv.pkv_paged_attn_verify(*args, err_flag=err)
    else:
        pkv.pkv_paged_prefill(*args, err_flag=err)
    torch.cuda.synchronize()
    want, rc = orc.verify(qv, hc.k_pool, hc.v_pool, hc.tables.block_tables,
                          hc.tables.context_lens, shape.n_kv, scale)
    assert rc == 0 and int(err.item()) == 0
    got = out.cpu().numpy().astype(np.float64)
    assert np.isfinite(got).all()
    e = max_abs(got, want)
    print(f"  max-abs {e:.2e}", flush=True)
    assert e <= TOL
