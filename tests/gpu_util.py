"""Helpers for the GPU tests: move seeded host cases to the device, run the
library, bring results back. Test infrastructure; the product path never
imports this."""
import numpy as np

import workload as w

TOL = 1e-3   # max-abs error allowed against the oracle on fp32 outputs


def torch_mod():
    import torch
    return torch


def to_dev_bf16(a):
    torch = torch_mod()
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()


def to_dev_i32(a):
    torch = torch_mod()
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()


def to_host_u16(t):
    torch = torch_mod()
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


class DevCase:
    """Device copy of a workload.HostCase (one layer)."""

    def __init__(self, hc: w.HostCase):
        torch = torch_mod()
        self.hc = hc
        self.k_pool = to_dev_bf16(hc.k_pool)
        self.v_pool = to_dev_bf16(hc.v_pool)
        self.q = to_dev_bf16(hc.q)
        self.k_new = to_dev_bf16(hc.k_new)
        self.v_new = to_dev_bf16(hc.v_new)
        self.bt = to_dev_i32(hc.tables.block_tables)
        self.cl = to_dev_i32(hc.tables.context_lens)
        self.err = torch.zeros(1, dtype=torch.int32, device="cuda")
        B, n_q, d = hc.q.shape
        self.out = torch.full((B, n_q, d), float("nan"), dtype=torch.float32, device="cuda")
        self.max_ctx = int(hc.tables.context_lens.max())


def gpu_step(pkv, dc: DevCase, partition=0, append=True, scale=None, max_ctx=None, fused=False,
             halves=False):
    """append (unless append=False) and decode; fused=True runs both as
    pkv_decode_step, or with halves=True as its two calls
    (pkv_decode_step_partition, then pkv_paged_attn_merge)."""
    torch = torch_mod()
    sh = dc.hc.shape
    scale = sh.scale if scale is None else scale
    max_ctx = dc.max_ctx if max_ctx is None else max_ctx
    if fused and halves:
        assert append
        ws = pkv.pkv_decode_step_partition(dc.out, dc.q, dc.k_new, dc.v_new, dc.k_pool, dc.v_pool,
                                           dc.bt, dc.cl, scale, max_ctx,
                                           partition_tokens=partition, err_flag=dc.err)
        pkv.pkv_paged_attn_merge(dc.out, dc.q, dc.k_pool, dc.v_pool, dc.bt, dc.cl, scale, max_ctx,
                                 partition_tokens=partition, workspace=ws, err_flag=dc.err)
    elif fused:
        assert append
        pkv.pkv_decode_step(dc.out, dc.q, dc.k_new, dc.v_new, dc.k_pool, dc.v_pool, dc.bt, dc.cl,
                            scale, max_ctx, partition_tokens=partition, err_flag=dc.err)
    else:
        if append:
            pkv.pkv_kv_append(dc.k_pool, dc.v_pool, dc.k_new, dc.v_new, dc.bt, dc.cl,
                              err_flag=dc.err)
        pkv.pkv_paged_attn_decode(dc.out, dc.q, dc.k_pool, dc.v_pool, dc.bt, dc.cl, scale, max_ctx,
                                  partition_tokens=partition, err_flag=dc.err)
    torch.cuda.synchronize()
    return dc.out.cpu().numpy().astype(np.float64)


def oracle_step(orc, hc: w.HostCase, append=True, scale=None):
    k = hc.k_pool.copy()
    v = hc.v_pool.copy()
    if append:
        assert orc.kv_append(k, v, hc.k_new, hc.v_new, hc.tables.block_tables,
                             hc.tables.context_lens) == 0
    out, rc = orc.decode(hc.q, k, v, hc.tables.block_tables, hc.tables.context_lens,
                         hc.shape.n_kv, hc.shape.scale if scale is None else scale)
    return out, rc, k, v


def max_abs(a, b):
    return float(np.max(np.abs(a - b))) if a.size else 0.0
