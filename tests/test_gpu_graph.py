"""The library's launches captured in a HIP graph and replayed.

A graph of kv_append + partition + merge is captured once, then replayed
several times with eager work between the replays: new query and new-token
values and new context lengths are copied into the device buffers the graph
reads, and the stream is synchronised. After every replay the graph's output
must equal, bit for bit, an eager decode of the same state, and the pools
must hold the appended tokens. Nothing in the graph clears memory, and
nothing is allocated during capture. The same for chunked prefill, whose
work order follows the context lengths the graph reads at each replay.
"""
import numpy as np
import pytest

import workload as w
from gpu_util import DevCase, to_dev_bf16, to_dev_i32, to_host_u16

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pkv():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import paged_kv_cache_468_amd as lib
    return lib


def _shape(n_q, n_kv, d):
    return w.Shape(f"{n_q}/{n_kv} d{d}", 1, n_q, n_kv, d, 1, 1, 1)


@pytest.mark.parametrize("part", [0, 64])
def test_graph_replays_match_eager(pkv, part):
    import torch
    sh = _shape(32, 8, 128)
    ctx0 = np.array([700, 1, 33, 2048, 517, 16], np.int32)
    hc = w.host_case(sh, 71, context_lens=ctx0, max_blocks=160, spare_blocks=8)
    dc = DevCase(hc)
    max_ctx = 16 * 160
    ws_bytes = pkv.pkv_decode_workspace_bytes(len(ctx0), 32, 8, 128, max_ctx, part)
    ws = torch.zeros(max(ws_bytes, 1), dtype=torch.uint8, device="cuda")
    out_ref = torch.empty_like(dc.out)
    # the device query behind the balanced split is cached outside capture
    assert pkv.pkv_decode_split_waves(len(ctx0), 32, 8, 128, max_ctx) > 0
    torch.cuda.synchronize()

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        calls = [
            pkv.prepare_kv_append(dc.k_pool, dc.v_pool, dc.k_new, dc.v_new, dc.bt, dc.cl,
                                  err_flag=dc.err),
            pkv.prepare_paged_attn_decode(dc.out, dc.q, dc.k_pool, dc.v_pool, dc.bt, dc.cl,
                                          sh.scale, max_ctx, part, workspace=ws, err_flag=dc.err),
        ]
        for c in calls:
            c()

    rng = w.rng(72, 0)
    for rep in range(4):
        # eager work between replays: new inputs into the buffers the graph reads
        ctx = ctx0 - rng.integers(0, 2, size=len(ctx0)).astype(np.int32) * (ctx0 > 1)
        dc.cl.copy_(to_dev_i32(ctx))
        dc.q.copy_(to_dev_bf16(w.normal_bf16(rng, tuple(dc.q.shape))))
        dc.k_new.copy_(to_dev_bf16(w.normal_bf16(rng, tuple(dc.k_new.shape))))
        dc.v_new.copy_(to_dev_bf16(w.normal_bf16(rng, tuple(dc.v_new.shape))))
        dc.out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = dc.out.cpu().numpy()
        # eager decode of the same state into another buffer
        pkv.pkv_paged_attn_decode(out_ref, dc.q, dc.k_pool, dc.v_pool, dc.bt, dc.cl, sh.scale,
                                  max_ctx, part, workspace=ws, err_flag=dc.err)
        torch.cuda.synchronize()
        assert int(dc.err.item()) == 0
        assert np.isfinite(got).all(), f"replay {rep}"
        assert np.array_equal(got, out_ref.cpu().numpy()), f"replay {rep} differs from eager"
        # the appended token of sequence 0 is where the table says
        k_host = to_host_u16(dc.k_pool)
        p = int(ctx[0]) - 1
        blk = hc.tables.block_tables[0, p // 16]
        assert np.array_equal(k_host[blk, :, p % 16, :], to_host_u16(dc.k_new)[0])


def test_prefill_graph_replays_match_eager(pkv):
    """pkv_paged_prefill captured once and replayed with new queries and new
    context lengths between replays: the workgroups rank the sequences by
    context length on the device, so a replay must follow the new lengths;
    every replay equals an eager launch of the same state bit for bit."""
    import torch
    sh = _shape(32, 8, 128)
    C = 64
    ctx0 = np.array([900, 300, 1500, 64, 700], np.int32)
    hc = w.host_case(sh, 73, context_lens=ctx0, max_blocks=100)
    kp, vp = to_dev_bf16(hc.k_pool), to_dev_bf16(hc.v_pool)
    bt, cl = to_dev_i32(hc.tables.block_tables), to_dev_i32(ctx0)
    q = torch.empty((len(ctx0), C, sh.n_q, sh.d), dtype=torch.bfloat16, device="cuda")
    out = torch.empty(q.shape, dtype=torch.float32, device="cuda")
    out_ref = torch.empty_like(out)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    max_ctx = int(ctx0.max())
    rng = w.rng(74, 0)
    q.copy_(to_dev_bf16(w.normal_bf16(rng, tuple(q.shape))))
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        pkv.pkv_paged_prefill(out, q, kp, vp, bt, cl, sh.scale, max_ctx, err_flag=err)
    for rep in range(4):
        # shorter contexts (never below the chunk) reorder the sequences' ranks
        ctx = np.maximum(ctx0 - rng.integers(0, 700, size=len(ctx0)).astype(np.int32), C)
        cl.copy_(to_dev_i32(ctx))
        q.copy_(to_dev_bf16(w.normal_bf16(rng, tuple(q.shape))))
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = out.cpu().numpy()
        pkv.pkv_paged_prefill(out_ref, q, kp, vp, bt, cl, sh.scale, max_ctx, err_flag=err)
        torch.cuda.synchronize()
        assert int(err.item()) == 0
        assert np.isfinite(got).all(), f"replay {rep}"
        assert np.array_equal(got, out_ref.cpu().numpy()), f"replay {rep} differs from eager"
