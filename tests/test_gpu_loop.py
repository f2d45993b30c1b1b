"""Continuous batching on the GPU, step by step against the oracle.

Requests arrive over time, some beginning with a shared prefix whose last
block is partly filled, in a pool small enough that requests are preempted
and recomputed. Every step runs the native batcher, then per layer the
copy-on-write copies, the prompt writes (pkv_kv_write) and pkv_decode_step.
Checked at every step:
  * the pools, bit for bit, against a host mirror that applies the same
    plan with the oracle's copy, write and append;
  * every resident request's output, within 1e-3, against the oracle run on
    a cache rebuilt contiguously from that request's token history (its
    keys and values are a fixed function of (layer, request, position), the
    shared prefix's where it shares), i.e. attention recomputed from a
    contiguous cache;
  * every request finishes after exactly gen_len decode steps.
"""
import numpy as np
import pytest

import workload as w
import loop_util as lu
from gpu_util import TOL, max_abs, to_dev_bf16, to_host_u16

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pkv():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import paged_kv_cache_468_amd as lib
    return lib


@pytest.mark.parametrize("d,n_kv,n_tok", [(64, 2, 1), (128, 8, 300), (64, 1, 4099)])
def test_kv_write_bit_exact(pkv, orc, d, n_kv, n_tok):
    """Prompt tokens written at (row, position) through the tables, against
    the oracle's write: bit for bit, with invalid rows, positions and table
    entries skipped and flagged on both sides."""
    import torch
    num_blocks, num_seqs, max_blocks = 700, 9, 40
    g = w.rng(31 + n_tok, 8)
    tables = g.permutation(num_blocks)[:num_seqs * max_blocks].astype(np.int32)
    tables = tables.reshape(num_seqs, max_blocks)
    tables[3, 5:] = -1                            # a short table
    # distinct (row, position) pairs, a few invalid
    flat = g.choice(num_seqs * 16 * max_blocks, size=n_tok, replace=False)
    rows = (flat // (16 * max_blocks)).astype(np.int32)
    pos = (flat % (16 * max_blocks)).astype(np.int32)
    if n_tok > 10:
        rows[1], pos[2], pos[3] = num_seqs, 16 * max_blocks, -1
    ks = w.normal_bf16(g, (n_tok, n_kv, d))
    vs = w.normal_bf16(g, (n_tok, n_kv, d))
    sk, sv = w.pool_shapes(num_blocks, n_kv, d)
    hk = w.normal_bf16(g, sk)
    hv = w.normal_bf16(g, sv)
    dk, dv = to_dev_bf16(hk), to_dev_bf16(hv)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    pkv.pkv_kv_write(dk, dv, to_dev_bf16(ks), to_dev_bf16(vs), torch.from_numpy(tables).cuda(),
                     torch.from_numpy(rows).cuda(), torch.from_numpy(pos).cuda(), err_flag=err)
    torch.cuda.synchronize()
    rc = orc.kv_write(hk, hv, ks, vs, tables, rows, pos)
    skipped = bool((rows >= num_seqs).any() or (pos < 0).any() or (pos >= 16 * max_blocks).any()
                   or (tables[np.clip(rows, 0, num_seqs - 1),
                              np.clip(pos, 0, 16 * max_blocks - 1) // 16] < 0).any())
    assert (rc == -1) == skipped
    assert (int(err.item()) != 0) == skipped
    assert np.array_equal(to_host_u16(dk), hk)
    assert np.array_equal(to_host_u16(dv), hv)

@pytest.mark.parametrize("d,n_kv", [(128, 8), (64, 4)])
def test_kv_write_prompt_order_bit_exact(pkv, orc, d, n_kv):
    """Prompts written in order, as after a prefill: per sequence a run of
    consecutive positions starting anywhere in a block (so runs of 16 input
    tokens straddle blocks and sequences), lengths 1 .. 200, one invalid
    table entry. Bit for bit against the oracle's write."""
    import torch
    num_blocks, max_blocks = 400, 20
    g = w.rng(77 + d, 8)
    starts = [0, 5, 16, 31, 7, 100, 3]
    lens = [200, 1, 16, 45, 90, 17, 60]
    num_seqs = len(starts)
    tables = g.permutation(num_blocks)[:num_seqs * max_blocks].astype(np.int32)
    tables = tables.reshape(num_seqs, max_blocks)
    tables[5, (100 + 10) // 16] = num_blocks + 3          # one bad entry: those tokens skipped
    rows = np.concatenate([np.full(n, r, np.int32) for r, n in enumerate(lens)])
    pos = np.concatenate([np.arange(s0, s0 + n, dtype=np.int32) for s0, n in zip(starts, lens)])
    n_tok = len(rows)
    ks = w.normal_bf16(g, (n_tok, n_kv, d))
    vs = w.normal_bf16(g, (n_tok, n_kv, d))
    sk, sv = w.pool_shapes(num_blocks, n_kv, d)
    hk = np.full(sk, w.BF16_NAN, np.uint16)
    hv = np.full(sv, w.BF16_NAN, np.uint16)
    dk, dv = to_dev_bf16(hk), to_dev_bf16(hv)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    pkv.pkv_kv_write(dk, dv, to_dev_bf16(ks), to_dev_bf16(vs), torch.from_numpy(tables).cuda(),
                     torch.from_numpy(rows).cuda(), torch.from_numpy(pos).cuda(), err_flag=err)
    torch.cuda.synchronize()
    assert orc.kv_write(hk, hv, ks, vs, tables, rows, pos) == -1
    assert int(err.item()) == pkv.PKV_DEVERR_BLOCK_ID
    assert np.array_equal(to_host_u16(dk), hk)
    assert np.array_equal(to_host_u16(dv), hv)


# prefix lengths: one whole block and 4 tokens of a second, which sharers
# copy on write; two whole blocks, every one of them shared
@pytest.mark.parametrize("prefix", [lu.PREFIX, 32])
@pytest.mark.parametrize("d", [64, 128])
def test_continuous_batching_matches_contiguous_recompute(pkv, orc, d, prefix):
    import torch
    from paged_kv_cache_468_amd.loop import ServingLoop
    L = lu.L
    scale = 1.0 / np.sqrt(d)
    reqs = lu.requests(d, prefix=prefix)
    hist = lu.History(d, {rid: r[3] for rid, r in reqs.items()}, prefix=prefix)
    b = pkv.Batcher(lu.NUM_BLOCKS, lu.MAX_BATCH, lu.MAX_BLOCKS, prefix)
    sk, sv = w.pool_shapes(lu.NUM_BLOCKS, lu.N_KV, d)
    host_k = [np.full(sk, w.BF16_NAN, np.uint16) for _ in range(L)]
    host_v = [np.full(sv, w.BF16_NAN, np.uint16) for _ in range(L)]
    kp = [to_dev_bf16(x) for x in host_k]
    vp = [to_dev_bf16(x) for x in host_v]
    loop = ServingLoop(b, kp, vp, lu.N_Q, scale, lu.MAX_BATCH)

    # the shared prefix, written once through its own table
    ptable, _ = b.prefix_table()
    loop.write_prefix([to_dev_bf16(hist.pk[l]) for l in range(L)],
                      [to_dev_bf16(hist.pv[l]) for l in range(L)])
    for l in range(L):
        assert orc.kv_write(host_k[l], host_v[l], hist.pk[l], hist.pv[l], ptable.reshape(1, -1),
                            np.zeros(prefix, np.int32),
                            np.arange(prefix, dtype=np.int32)) == 0

    steps_seen, finished, preempted, prefix_calls = {}, [], 0, 0
    for step in range(2000):
        for rid, (arr, prompt, gen, shares) in reqs.items():
            if arr == step:
                b.submit(rid, prompt, gen, shares)
        p = loop.schedule()
        n = p.num_seqs
        prefix_calls += loop.members[1] > 0
        ids = [int(x) for x in p.request_ids]
        finished += [int(x) for x in p.finished_ids]
        preempted += len(p.preempted_ids)
        if n == 0 and p.num_waiting == 0 and step > 30:
            break
        fill = [hist.fill(l, ids, p) for l in range(L)]
        new = [hist.new_token(l, ids, p) for l in range(L)]
        g = w.rng(50000 + step, 7)
        q_h = [w.normal_bf16(g, (n, lu.N_Q, d)) for _ in range(L)]
        if step % 25 == 0:
            print(f"d={d} step {step}: {n} rows, {len(p.fill_rows)} fill, {len(p.cow_src)} cow",
                  flush=True)
        out = loop.run(lambda l: (to_dev_bf16(fill[l][0]), to_dev_bf16(fill[l][1])),
                       [to_dev_bf16(x) for x in q_h], [to_dev_bf16(x[0]) for x in new],
                       [to_dev_bf16(x[1]) for x in new])
        torch.cuda.synchronize()
        assert int(loop.err.item()) == 0, f"step {step}"
        got = out.cpu().numpy().astype(np.float64)
        for l in range(L):
            lu.mirror_step(orc, host_k[l], host_v[l], p, fill[l], new[l][0], new[l][1], d)
            assert np.array_equal(to_host_u16(kp[l]), host_k[l]), f"K pool differs at step {step}"
            assert np.array_equal(to_host_u16(vp[l]), host_v[l]), f"V pool differs at step {step}"
            if n:
                want = lu.contiguous_decode(orc, q_h[l], hist, l, ids, p.context_lens, scale)
                err = max_abs(got[l], want)
                assert err <= TOL, f"step {step} layer {l}: {err}"
        for rid in ids:
            steps_seen[rid] = steps_seen.get(rid, 0) + 1

    assert sorted(finished) == sorted(reqs)
    assert all(steps_seen[rid] == reqs[rid][2] for rid in reqs)
    assert preempted > 0, "the pool was meant to force preemption"
    # the prefix's whole block went through pkv_decode_step_prefix
    assert prefix_calls > 0


@pytest.mark.parametrize("d", [64, 128])
def test_continuous_batching_with_prefix_cache(pkv, orc, d):
    """The batcher with a prefix cache: requests carry token ids (system
    prompts, chats that extend an earlier request, unrelated prompts),
    admissions take cached blocks and write only the positions after them,
    the tight pool evicts cached blocks and preempts. Keys and values of a
    position are a function of the tokens up to it, so a cached block read by
    a later request must hold exactly its prefix. Every step: the pools bit
    for bit against the host mirror, every row's output within 1e-3 against
    attention over caches rebuilt contiguously from the request's tokens."""
    import random
    import torch
    from paged_kv_cache_468_amd.loop import ServingLoop
    from test_batcher import _chat_requests
    L = lu.L
    scale = 1.0 / np.sqrt(d)
    rnd = random.Random(21)
    reqs = {rid: (prompt, gen, gt) for rid, prompt, gen, gt in _chat_requests(rnd, 30, max_gen=60)}
    hist = lu.TokenHistory(d, {rid: r[0] + r[2] for rid, r in reqs.items()})
    nb, mb = 32, 32
    b = pkv.Batcher(nb, lu.MAX_BATCH, mb, 0)
    b.enable_prefix_cache()
    sk, sv = w.pool_shapes(nb, lu.N_KV, d)
    host_k = [np.full(sk, w.BF16_NAN, np.uint16) for _ in range(L)]
    host_v = [np.full(sv, w.BF16_NAN, np.uint16) for _ in range(L)]
    kp = [to_dev_bf16(x) for x in host_k]
    vp = [to_dev_bf16(x) for x in host_v]
    loop = ServingLoop(b, kp, vp, lu.N_Q, scale, lu.MAX_BATCH)

    pending = sorted(reqs)
    cached = preempted = 0
    finished, steps_seen = [], {}
    for step in range(3000):
        if pending and rnd.random() < 0.5:
            rid = pending.pop(0)
            b.submit_tokens(rid, reqs[rid][0], reqs[rid][1])
        p = loop.schedule()
        n = p.num_seqs
        ids = [int(x) for x in p.request_ids]
        cached += p.n_cached_tokens
        preempted += len(p.preempted_ids)
        finished += [int(x) for x in p.finished_ids]
        if not pending and n == 0 and p.num_waiting == 0:
            break
        fill = [hist.fill(l, ids, p) for l in range(L)]
        new = [hist.new_token(l, ids, p) for l in range(L)]
        g = w.rng(60000 + step, 7)
        q_h = [w.normal_bf16(g, (n, lu.N_Q, d)) for _ in range(L)]
        if step % 25 == 0:
            print(f"d={d} step {step}: {n} rows, {len(p.fill_rows)} fill, "
                  f"{cached} cached tokens so far", flush=True)
        out = loop.run(lambda l: (to_dev_bf16(fill[l][0]), to_dev_bf16(fill[l][1])),
                       [to_dev_bf16(x) for x in q_h], [to_dev_bf16(x[0]) for x in new],
                       [to_dev_bf16(x[1]) for x in new])
        torch.cuda.synchronize()
        assert int(loop.err.item()) == 0, f"step {step}"
        got = out.cpu().numpy().astype(np.float64)
        for l in range(L):
            lu.mirror_step(orc, host_k[l], host_v[l], p, fill[l], new[l][0], new[l][1], d)
            assert np.array_equal(to_host_u16(kp[l]), host_k[l]), f"K pool differs at step {step}"
            assert np.array_equal(to_host_u16(vp[l]), host_v[l]), f"V pool differs at step {step}"
            if n:
                want = lu.contiguous_decode(orc, q_h[l], hist, l, ids, p.context_lens, scale)
                err = max_abs(got[l], want)
                assert err <= TOL, f"step {step} layer {l}: {err}"
        for rid in ids:
            steps_seen[rid] = steps_seen.get(rid, 0) + 1
    assert sorted(finished) == sorted(reqs)
    assert all(steps_seen[rid] == reqs[rid][1] for rid in reqs)
    assert cached > 1000 and preempted > 0, (cached, preempted)
    print(f"d={d}: {cached} prompt tokens from the cache, {preempted} preemptions")


def test_graph_replay_matches_eager_loop(pkv):
    """The serving loop with its decode launches replayed from cached HIP
    graphs, against the same loop issuing them eagerly. Two batchers fed the
    same requests make the same plans; each step's queries and new keys and
    values go into each loop's own input buffers. Every step's outputs, and
    the pools at the end, are bit for bit the same; graphs are captured once
    per row count and replayed from the cache otherwise (admissions,
    preemptions and finishes change the row count between replays)."""
    import torch
    from paged_kv_cache_468_amd.loop import ServingLoop
    d, L = 128, lu.L
    reqs = lu.requests(d)
    hist = lu.History(d, {rid: r[3] for rid, r in reqs.items()})
    sk, sv = w.pool_shapes(lu.NUM_BLOCKS, lu.N_KV, d)
    loops = []
    for graphs in (False, True):
        b = pkv.Batcher(lu.NUM_BLOCKS, lu.MAX_BATCH, lu.MAX_BLOCKS, lu.PREFIX)
        kp = [to_dev_bf16(np.full(sk, w.BF16_NAN, np.uint16)) for _ in range(L)]
        vp = [to_dev_bf16(np.full(sv, w.BF16_NAN, np.uint16)) for _ in range(L)]
        loop = ServingLoop(b, kp, vp, lu.N_Q, 1.0 / np.sqrt(d), lu.MAX_BATCH, graphs=graphs)
        loop.write_prefix([to_dev_bf16(hist.pk[l]) for l in range(L)],
                          [to_dev_bf16(hist.pv[l]) for l in range(L)])
        loops.append((b, loop, kp, vp))
    steps = 0
    for step in range(2000):
        plans = []
        for b, loop, _, _ in loops:
            for rid, (arr, prompt, gen, shares) in reqs.items():
                if arr == step:
                    b.submit(rid, prompt, gen, shares)
            plans.append(loop.schedule())
        p = plans[0]
        assert p.request_ids.tolist() == plans[1].request_ids.tolist()
        assert p.context_lens.tolist() == plans[1].context_lens.tolist()
        n = p.num_seqs
        if n == 0 and p.num_waiting == 0 and step > 30:
            break
        ids = [int(x) for x in p.request_ids]
        fill = [hist.fill(l, ids, p) for l in range(L)]
        new = [hist.new_token(l, ids, p) for l in range(L)]
        g = w.rng(70000 + step, 7)
        q_h = [w.normal_bf16(g, (n, lu.N_Q, d)) for _ in range(L)]
        outs = []
        for b, loop, _, _ in loops:
            qb, kb, vb = loop.inputs()
            for l in range(L):
                if n:
                    qb[l, :n].copy_(to_dev_bf16(q_h[l]))
                    kb[l, :n].copy_(to_dev_bf16(new[l][0]))
                    vb[l, :n].copy_(to_dev_bf16(new[l][1]))
            out = loop.run(lambda l: (to_dev_bf16(fill[l][0]), to_dev_bf16(fill[l][1])),
                           None, None, None)
            torch.cuda.synchronize()
            assert int(loop.err.item()) == 0, f"step {step}"
            outs.append(out.cpu().numpy())
        assert np.array_equal(outs[0], outs[1]), f"step {step}: graph replay differs"
        steps += 1
    for l in range(L):
        assert np.array_equal(to_host_u16(loops[0][2][l]), to_host_u16(loops[1][2][l]))
        assert np.array_equal(to_host_u16(loops[0][3][l]), to_host_u16(loops[1][3][l]))
    gl = loops[1][1]
    print(f"{steps} steps: {gl.graph_captures} captures, {gl.graph_hits} replays from the cache")
    assert gl.graph_hits > gl.graph_captures > 0
