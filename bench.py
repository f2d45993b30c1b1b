#!/usr/bin/env python3
"""Decode-step benchmark of paged attention on one MI355X.

One step is one decode iteration of the whole batch over every layer:
  host    every sequence grows by one token through the block allocator
          (pkv_seq_grow: a fresh block at each 16-token boundary), and the
          tables and context lengths go to the device (async, pinned);
  device  per layer: kv_append (the new token's K/V into its slot),
          the partition kernel (scores, online softmax, P.V per context
          partition) and the merge kernel (log-sum-exp merge of partitions).
The default workload is the LLaMA-3-8B grouped-query shape (32 layers,
32 query / 8 KV heads, head size 128, bf16 KV in 16-token blocks, 64
sequences with contexts uniform in [1024, 8192], a 2,048-token prefix shared
through refcounted blocks), and the same shape with private copies of the
prefix (no sharing). Inputs are seeded synthetic N(0,1) values drawn on the
device; the pool is fragmented (block ids handed out in a random order).

Printed: one JSON line with the KV GB/s of the step (value), steps/s,
the partition kernel's roofline (HIP events on the stream it runs on), the
CPU oracle timed on a bounded sample of the same bytes, and the parity of
that sample against the GPU output.

  python bench.py [--steps K] [--warmup W] [--config 4] [--no-share-run/--skip-no-share]
"""
import argparse
import hashlib
import re
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import workload as w  # noqa: E402

HBM_PEAK_GBS = 8000.0   # MI355X HBM3E, published
VOCAB = 128256          # LLaMA-3 vocabulary: the acceptance rule's draw runs over it
MFMA_BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 matrix peak, published
BLOCK = 16
# counter summaries: profiles/pmc_<kernel>_<workload>.txt, ending in a JSON record
PMC_FILE = os.path.join(ROOT, "profiles", "pmc_{kernel}_{workload}.txt")
KERNEL_SOURCE = os.path.join(ROOT, "paged_kv_cache_468_amd", "csrc", "attention.hip")

WORKLOAD_NAMES = {
    1: "tiny-1layer-20q4kv-d64",
    2: "0.5B-24layer-20q4kv-d64-B128",
    3: "llama2-7b-mha-32layer-32q32kv-d128-B32-ctx4096",
    4: "llama3-8b-gqa-32layer-32q8kv-d128-B64-ctx1024..8192-prefix2048",
    5: "80layer-gqa-64q8kv-d128-B60-ctx8000",
}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash(path=KERNEL_SOURCE):
    """Hash of the kernel source's code: comments and whitespace removed, so
    that a counter record stays valid across edits that change no code."""
    with open(path) as f:
        src = f.read()
    src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
    src = re.sub(r"//[^\n]*", " ", src)
    src = " ".join(src.split())
    return hashlib.sha256(src.encode()).hexdigest()[:16]


# ---------------------------------------------------------------------------
# workload state built through the library's own allocator

class State:
    pass


def members_first(cl, prefix_tokens):
    """The batch order: sequences longer than the prefix first, each group
    in its drawn order. With sharing those hold all of the prefix's blocks
    (a shorter one copies the block it writes), so they are
    pkv_decode_step_prefix's member range [0, count)."""
    if not prefix_tokens:
        return cl
    return cl[np.argsort(cl <= prefix_tokens, kind="stable")]


def build_state(pkv, torch, shape, seed, share, extra_tokens, partition_tokens, fused=True,
                prefix_kernel=False, valu=False):
    """Block tables from the refcounted allocator, pools filled on the
    device, every layer's buffers, and pre-marshalled library calls."""
    cl = members_first(w.context_lengths(shape, seed).astype(np.int32), shape.prefix_tokens)
    B = len(cl)
    L, n_q, n_kv, d = shape.n_layers, shape.n_q, shape.n_kv, shape.d
    final_ctx = cl + extra_tokens
    max_blocks = int(math.ceil(int(final_ctx.max()) / BLOCK))
    n_prefix = shape.prefix_tokens // BLOCK if share else 0
    # blocks held at the end of the run: the prefix owner's, plus each
    # sequence's own (the ones not shared)
    own = [int(math.ceil(int(c) / BLOCK)) - min(n_prefix, int(math.ceil(int(c0) / BLOCK)))
           + (1 if n_prefix and int(c0) <= shape.prefix_tokens else 0)
           for c, c0 in zip(final_ctx, cl)]
    num_blocks = n_prefix + sum(own)

    alloc = pkv.Allocator(num_blocks)
    # fragmented pool: take every block, give them back in a seeded random
    # order; the LIFO free list then hands them out in that order
    for _ in range(num_blocks):
        alloc.pkv_block_alloc()
    for b in w.rng(seed, 1).permutation(num_blocks):
        alloc.pkv_block_decref(int(b))

    tables = np.full((B, max_blocks), -1, np.int32)
    nblk = np.zeros(B, np.int32)
    cow = []
    if n_prefix:
        prefix = np.full(max_blocks, -1, np.int32)
        st, n, _, _ = alloc.pkv_seq_grow(prefix, 0, shape.prefix_tokens)
        assert st == pkv.PKV_OK and n == n_prefix
        for s in range(B):
            k = min(n_prefix, int(math.ceil(int(cl[s]) / BLOCK)))
            alloc.pkv_seq_fork(prefix, k)
            tables[s, :k] = prefix[:k]
            nblk[s] = k
    for s in range(B):
        st, nblk[s], src, dst = alloc.pkv_seq_grow(tables[s], int(nblk[s]), int(cl[s]))
        assert st == pkv.PKV_OK
        if src >= 0:
            cow.append((src, dst))

    S = State()
    S.shape, S.share, S.B, S.alloc = shape, share, B, alloc
    # prefix blocks each sequence's table holds (read from the one copy);
    # the blocks it writes or copied are its own
    S.shared_blocks = (np.array([int((tables[s, :n_prefix] == prefix[:n_prefix]).sum())
                                 for s in range(B)], np.int64) if n_prefix else np.zeros(B, np.int64))
    S.prefix_shared_tokens = BLOCK * n_prefix if n_prefix and S.shared_blocks.any() else 0
    # the prefix's block ids, and the sequences past it (placed first)
    S.prefix_ids = prefix[:n_prefix].copy() if n_prefix else np.zeros(0, np.int32)
    S.past_prefix = int((cl > shape.prefix_tokens).sum()) if n_prefix else 0
    S.ctx = cl.copy()
    S.tables, S.nblk, S.num_blocks, S.max_blocks = tables, nblk, num_blocks, max_blocks
    S.max_ctx = int(final_ctx.max())
    S.n_cow = len(cow)
    dev = torch.device("cuda")
    S.k_pool = torch.empty((L, num_blocks, n_kv, BLOCK, d), dtype=torch.bfloat16, device=dev)
    S.v_pool = torch.empty((L, num_blocks, n_kv, d, BLOCK), dtype=torch.bfloat16, device=dev)
    base = seed * 1000 + (0 if share else 500)
    w.device_normal_bf16_(S.k_pool, base + 1)
    w.device_normal_bf16_(S.v_pool, base + 2)
    S.q = w.device_normal_bf16_(torch.empty((L, B, n_q, d), dtype=torch.bfloat16, device=dev), base + 3)
    S.k_new = w.device_normal_bf16_(torch.empty((L, B, n_kv, d), dtype=torch.bfloat16, device=dev), base + 4)
    S.v_new = w.device_normal_bf16_(torch.empty((L, B, n_kv, d), dtype=torch.bfloat16, device=dev), base + 5)
    S.out = torch.zeros((L, B, n_q, d), dtype=torch.float32, device=dev)
    S.bt = torch.from_numpy(tables).to(dev)
    S.cl = torch.from_numpy(S.ctx).to(dev)
    S.err = torch.zeros(1, dtype=torch.int32, device=dev)
    # staging for the per-step table upload: two pinned buffers, reused
    # only after the copy that last read them has finished
    S.pin_bt = [torch.empty((B, max_blocks), dtype=torch.int32, pin_memory=True) for _ in range(2)]
    S.pin_cl = [torch.empty((B,), dtype=torch.int32, pin_memory=True) for _ in range(2)]
    S.pin_done = [None, None]

    if cow:   # copy-on-write of the prefix blocks the short sequences write into
        src = torch.tensor([c[0] for c in cow], dtype=torch.int32, device=dev)
        dst = torch.tensor([c[1] for c in cow], dtype=torch.int32, device=dev)
        for l in range(L):
            pkv.pkv_copy_blocks(S.k_pool[l], S.v_pool[l], src, dst, err_flag=S.err)

    S.partition = partition_tokens
    S.split_waves = pkv.pkv_decode_split_waves(B, n_q, n_kv, d, S.max_ctx) if partition_tokens == 0 else 0
    ws_bytes = pkv.pkv_decode_workspace_bytes(B, n_q, n_kv, d, S.max_ctx, S.partition)
    # the shared prefix read once for all sequences (pkv_decode_step_prefix)
    S.prefix_blocks = n_prefix if (prefix_kernel and fused and partition_tokens == 0) else 0
    S.prefix_table = None
    S.prefix_members = int((cl > shape.prefix_tokens).sum()) if S.prefix_blocks else 0
    if S.prefix_blocks:
        S.prefix_table = torch.from_numpy(prefix[:n_prefix].copy()).to(dev)
        ws_bytes = max(ws_bytes, pkv.pkv_decode_prefix_workspace_bytes(B, n_q, n_kv, d, S.max_ctx,
                                                                       n_prefix, S.prefix_members))
    S.ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    S.fused = fused
    # the partition kernel on the vector ALUs (comparison with the matrix path)
    S.valu = valu and fused and partition_tokens == 0 and not S.prefix_blocks
    S.calls = layer_calls(pkv, S)
    torch.cuda.synchronize()
    assert int(S.err.item()) == 0
    return S


def layer_calls(pkv, S):
    """Per layer, the (name, call) pairs of one decode step, marshalled on
    torch's current stream: pkv_decode_step as its two launches (the
    partition kernel with the append inside, then the merge kernel), or
    kv_append + partition + merge."""
    sh, calls = S.shape, []
    for l in range(sh.n_layers):
        if S.prefix_blocks:
            # the shared prefix read once for all sequences: prefix,
            # partition and merge kernels in one call
            calls.append([
                ("decode_step_prefix", pkv.prepare_decode_step_prefix(
                    S.out[l], S.q[l], S.k_new[l], S.v_new[l], S.k_pool[l], S.v_pool[l], S.bt,
                    S.cl, sh.scale, S.max_ctx, S.prefix_table, 0, S.prefix_members, workspace=S.ws,
                    err_flag=S.err))])
        elif S.valu:
            calls.append([
                ("decode_step_partition_valu", pkv.prepare_decode_step_partition_valu(
                    S.out[l], S.q[l], S.k_new[l], S.v_new[l], S.k_pool[l], S.v_pool[l], S.bt,
                    S.cl, sh.scale, S.max_ctx, workspace=S.ws, err_flag=S.err)),
                ("paged_attn_merge", pkv.prepare_paged_attn_merge(
                    S.out[l], S.q[l], S.k_pool[l], S.v_pool[l], S.bt, S.cl, sh.scale, S.max_ctx,
                    S.partition, workspace=S.ws, err_flag=S.err))])
        elif S.fused:
            # pkv_decode_step as its two launches, so that events can time each
            calls.append([
                ("decode_step_partition", pkv.prepare_decode_step_partition(
                    S.out[l], S.q[l], S.k_new[l], S.v_new[l], S.k_pool[l], S.v_pool[l], S.bt,
                    S.cl, sh.scale, S.max_ctx, S.partition, workspace=S.ws, err_flag=S.err)),
                ("paged_attn_merge", pkv.prepare_paged_attn_merge(
                    S.out[l], S.q[l], S.k_pool[l], S.v_pool[l], S.bt, S.cl, sh.scale, S.max_ctx,
                    S.partition, workspace=S.ws, err_flag=S.err))])
        else:
            calls.append([
                ("kv_append", pkv.prepare_kv_append(S.k_pool[l], S.v_pool[l], S.k_new[l], S.v_new[l],
                                                    S.bt, S.cl, err_flag=S.err)),
                ("paged_attn_partition", pkv.prepare_paged_attn_partition(
                    S.out[l], S.q[l], S.k_pool[l], S.v_pool[l], S.bt, S.cl, sh.scale, S.max_ctx,
                    S.partition, workspace=S.ws, err_flag=S.err)),
                ("paged_attn_merge", pkv.prepare_paged_attn_merge(
                    S.out[l], S.q[l], S.k_pool[l], S.v_pool[l], S.bt, S.cl, sh.scale, S.max_ctx,
                    S.partition, workspace=S.ws, err_flag=S.err))])
    return calls


def host_grow(pkv, S):
    """The allocator's per-step work: every sequence takes one more token."""
    S.ctx += 1
    for s in range(S.B):
        st, nb, src, dst = S.alloc.pkv_seq_grow(S.tables[s], int(S.nblk[s]), int(S.ctx[s]))
        if st != pkv.PKV_OK or src >= 0:
            raise RuntimeError(f"sequence {s}: grow returned {st}, copy-on-write ({src}, {dst})")
        S.nblk[s] = nb


def upload_tables(torch, S, i):
    b = i & 1
    if S.pin_done[b] is not None:
        S.pin_done[b].synchronize()
    S.pin_bt[b].numpy()[...] = S.tables
    S.pin_cl[b].numpy()[...] = S.ctx
    S.bt.copy_(S.pin_bt[b], non_blocking=True)
    S.cl.copy_(S.pin_cl[b], non_blocking=True)
    ev = torch.cuda.Event()
    ev.record()
    S.pin_done[b] = ev


def kv_bytes(S, ctx):
    """Algorithmic KV bytes of one layer: K and V of every cached token,
    each 2 bytes per element over n_kv * head_dim elements."""
    return 2 * S.shape.n_kv * S.shape.d * 2 * int(ctx.astype(np.int64).sum())


def unique_kv_bytes(S, ctx):
    """KV bytes of one layer that HBM must deliver when every physical block
    is read once: the shared prefix's blocks once, every sequence's own
    blocks (its tokens outside the shared blocks) once. Equal to kv_bytes
    without sharing."""
    per_tok = 2 * S.shape.n_kv * S.shape.d * 2
    own = ctx.astype(np.int64) - BLOCK * S.shared_blocks
    return per_tok * (S.prefix_shared_tokens + int(own.sum()))


def attn_alg_bytes(S, ctx):
    """Algorithmic bytes of one layer's attention: the KV it must consume,
    plus q (bf16), the fp32 output rows, the block-table entries and the
    context lengths."""
    sh = S.shape
    B = len(ctx)
    tbl = 4 * int(np.ceil(ctx / BLOCK).astype(np.int64).sum())
    return kv_bytes(S, ctx) + B * sh.n_q * sh.d * (2 + 4) + tbl + 4 * B


def prefix_call_alg_bytes(S, ctx):
    """Algorithmic bytes of one pkv_decode_step_prefix call: the bytes it
    must move when the prefix is read once. K and V of the prefix once, of
    every member's tokens after the prefix and of every other sequence's
    whole context (a member whose context ends inside the prefix reads its
    own blocks), q, the fp32 outputs, the
    table entries, the context lengths and the appended rows."""
    sh = S.shape
    B = len(ctx)
    per_tok = 2 * sh.n_kv * sh.d * 2
    pre = S.prefix_blocks * BLOCK
    reads = ((ctx - 1) // BLOCK >= S.prefix_blocks) & (np.arange(B) < S.prefix_members)
    own = int(np.where(reads, ctx - pre, ctx).astype(np.int64).sum())
    tiles = int(np.where(reads, np.ceil(ctx / BLOCK) - S.prefix_blocks,
                         np.ceil(ctx / BLOCK)).astype(np.int64).sum())
    return (per_tok * (own + pre) + B * sh.n_q * sh.d * (2 + 4) + 4 * (tiles + S.prefix_blocks)
            + 4 * B + append_alg_bytes(S, B))


def append_alg_bytes(S, B):
    """kv_append of one layer: the new K and V rows read and written."""
    return 2 * 2 * B * S.shape.n_kv * S.shape.d * 2


def _eager_step(calls):
    for layer in calls:
        for _, call in layer:
            call()


def capture_step(pkv, torch, S):
    """One step's launches (every layer) captured into a HIP graph. The
    calls are marshalled inside the capture so that they name the capture
    stream. Tables and context lengths are read from the same device
    buffers the eager upload fills before each replay."""
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        _eager_step(layer_calls(pkv, S))
    return g


def run(pkv, torch, S, steps, warmup, graph=True):
    """Warm-up, then K timed steps with HIP events around every launch (the
    kernels' durations), then, with graph=True, K timed steps that replay the
    captured step (the step time). Each step first grows every sequence by
    one token through the allocator and uploads the tables."""
    L = S.shape.n_layers
    names = [n for n, _ in S.calls[0]]
    step_no = 0
    for _ in range(warmup):
        host_grow(pkv, S)
        upload_tables(torch, S, step_no)
        step_no += 1
        _eager_step(S.calls)
    torch.cuda.synchronize()

    # timed steps, eager, with events around each launch
    ev = [[[torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)] for _ in range(L)]
          for _ in range(steps)]
    eager_ctx = []
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t0.record()
    ev_step = []
    for i in range(steps):
        host_grow(pkv, S)
        eager_ctx.append(S.ctx.copy())
        upload_tables(torch, S, step_no)
        step_no += 1
        for l, layer in enumerate(S.calls):
            e = ev[i][l]
            for k, (_, call) in enumerate(layer):
                e[k].record()
                call()
            e[len(layer)].record()
        ev_step.append(torch.cuda.Event(enable_timing=True))
        ev_step[-1].record()
    t1.record()
    torch.cuda.synchronize()
    eager_wall = time.perf_counter() - wall0
    eager_ms = max(t0.elapsed_time(t1), eager_wall * 1e3) / steps
    if int(S.err.item()):
        raise RuntimeError(f"device error flag {int(S.err.item())}")
    kern_us = {n: float(np.mean([[ev[i][l][k].elapsed_time(ev[i][l][k + 1]) for l in range(L)]
                                 for i in range(steps)]) * 1e3)
               for k, n in enumerate(names)}

    # per-step times: from one step's end event to the next (the first
    # from the start event), so they add up to the pass's time
    per_step = [t0.elapsed_time(ev_step[0])] + [ev_step[i].elapsed_time(ev_step[i + 1])
                                                for i in range(steps - 1)]
    step_ctx, ms_per_step, mode = eager_ctx, eager_ms, "eager"
    if graph:
        g = capture_step(pkv, torch, S)
        host_grow(pkv, S)                     # one warm-up replay
        upload_tables(torch, S, step_no)
        step_no += 1
        g.replay()
        torch.cuda.synchronize()
        graph_ctx = []
        ev_g = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
        wall0 = time.perf_counter()
        t0.record()
        for i in range(steps):
            host_grow(pkv, S)
            graph_ctx.append(S.ctx.copy())
            upload_tables(torch, S, step_no)
            step_no += 1
            g.replay()
            ev_g[i].record()
        t1.record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - wall0
        per_step = [t0.elapsed_time(ev_g[0])] + [ev_g[i].elapsed_time(ev_g[i + 1])
                                                 for i in range(steps - 1)]
        if int(S.err.item()):
            raise RuntimeError(f"device error flag {int(S.err.item())}")
        step_ctx, ms_per_step, mode = graph_ctx, max(t0.elapsed_time(t1), wall * 1e3) / steps, "hip-graph"

    # the roofline kernel: the partition kernel, which reads the KV cache
    # (with the append inside when fused); the merge reads only partials
    if S.prefix_blocks:
        # the prefix call as a whole: its three kernels against the bytes
        # it must move (the prefix counted once)
        dom = "decode_step_prefix"
        alg = lambda c: prefix_call_alg_bytes(S, c)
    else:
        dom = ("decode_step_partition_valu" if S.valu else
               "decode_step_partition" if S.fused else "paged_attn_partition")
        alg = lambda c: attn_alg_bytes(S, c) + (append_alg_bytes(S, S.B) if S.fused else 0)
    dom_bytes = sum(alg(c) for c in eager_ctx) / steps
    # Its launch duration without the per-launch event overhead: its
    # launches alone, one per layer, back to back from a graph, replayed
    # between two events. The kernel only reads the cache and rewrites its
    # own partials (fused: and stores this step's token again at the same
    # slot), so every replay sees the same state.
    b2b_us, b2b_bytes, b2b_launches = None, None, 0
    if graph:
        gk = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gk):
            for layer in layer_calls(pkv, S):
                for n, call in layer:
                    if n == dom:
                        call()
        gk.replay()
        torch.cuda.synchronize()
        reps = max(3, steps // 2)
        t0.record()
        for _ in range(reps):
            gk.replay()
        t1.record()
        torch.cuda.synchronize()
        if int(S.err.item()):
            raise RuntimeError(f"device error flag {int(S.err.item())}")
        b2b_launches = reps * L
        b2b_us = t0.elapsed_time(t1) * 1e3 / b2b_launches
        b2b_bytes = alg(S.ctx)
    kvb = sum(kv_bytes(S, c) * L for c in step_ctx)           # all layers, all timed steps
    kvu = sum(unique_kv_bytes(S, c) * L for c in step_ctx)
    return {
        "ms_per_step": ms_per_step,
        "ms_per_step_median": float(np.median(per_step)),
        "ms_per_step_min": float(np.min(per_step)),
        "ms_per_step_max": float(np.max(per_step)),
        "kv_gbs_unique": kvu / (ms_per_step * steps * 1e-3) / 1e9,
        "kv_bytes_unique_per_step": kvu / steps,
        "step_mode": mode,
        "eager_ms_per_step": eager_ms,
        "steps_per_s": 1e3 / ms_per_step,
        "kv_gbs": kvb / (ms_per_step * steps * 1e-3) / 1e9,
        "seq_tokens_per_s": sum(int(c.astype(np.int64).sum()) for c in step_ctx) / (ms_per_step * steps * 1e-3),
        "tokens_per_s": S.B / (ms_per_step * 1e-3),
        "kv_bytes_per_step": kvb / steps,
        "kernels_us": kern_us,
        "dominant": dom,
        "dominant_us": b2b_us if b2b_us else kern_us[dom],
        "dominant_alg_bytes": b2b_bytes if b2b_us else dom_bytes,
        "dominant_gbs": (b2b_bytes / (b2b_us * 1e-6) if b2b_us else dom_bytes / (kern_us[dom] * 1e-6)) / 1e9,
        "dominant_timing": (f"HIP events around {b2b_launches} back-to-back launches of the kernel "
                            "(one per layer, replayed from a graph)" if b2b_us else
                            "HIP events around each launch in the eager timed steps"),
        "dominant_us_per_launch_events": kern_us[dom],
        "partition_tokens": S.partition,
        "split_waves": S.split_waves,
        "num_blocks_per_layer": S.num_blocks,
        "cow_copies": S.n_cow,
    }


# ---------------------------------------------------------------------------
# CPU oracle on a bounded sample of the same bytes (layer 0)

def cpu_baseline(torch, S, budget_s, threads_budget_s):
    """The oracle on a bounded sample of the final state: layers 0, 1, ...
    in turn (each copied back from the device), sequences in a seeded random
    order, until budget_s seconds of oracle time on one core. Then the same
    function on the host's threads (at most 16) over whole layers until
    threads_budget_s seconds. Returns the threaded run (with the one-core
    run inside; the one-core run alone when threads_budget_s is 0), the
    largest difference from the GPU output over the one-core sample, the
    sample's size, and the largest difference over the whole layers."""
    import oracle
    orc = oracle.default()
    sh = S.shape
    u16 = lambda t: t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    done, tokens, kvb, t_used, worst, layers = 0, 0, 0, 0.0, 0.0, 0
    order = w.rng(12345, 7).permutation(S.B)
    pairs = []   # (layer, sequence, float64 rows) in the order computed
    for l in range(sh.n_layers):
        k_l, v_l, q_l = u16(S.k_pool[l]), u16(S.v_pool[l]), u16(S.q[l])
        got = S.out[l].cpu().numpy().astype(np.float64)
        layers += 1
        for s in order:
            t0 = time.perf_counter()
            want, rc = orc.decode(q_l[s:s + 1], k_l, v_l, S.tables[s:s + 1], S.ctx[s:s + 1], sh.n_kv,
                                  sh.scale)
            t_used += time.perf_counter() - t0
            assert rc == 0
            pairs.append((l, int(s), want[0]))
            worst = max(worst, float(np.abs(want[0] - got[s]).max()))
            kvb += 2 * sh.n_kv * sh.d * 2 * int(S.ctx[s])
            tokens += int(S.ctx[s])
            done += 1
            if t_used >= budget_s:
                break
        del k_l, v_l
        if t_used >= budget_s:
            break
    gbs = kvb / t_used / 1e9
    single = {
        "value": gbs, "unit": "GB/s", "cores": 1, "kind": "oracle",
        "sample": (f"{done} (sequence, layer) pairs from layers 0..{layers - 1} of the final state, "
                   f"sequences in seeded random order, all {sh.n_q} query heads each "
                   f"({tokens} context tokens); single-threaded C oracle in float64, "
                   f"{t_used:.1f} s"),
        "seconds": t_used,
        "steps_per_s_equiv": gbs * 1e9 / (kv_bytes(S, S.ctx) * sh.n_layers),
    }
    # The oracle's single-precision twin (the naive fp32 loop) over the first
    # pairs of the same order, for a third of the budget: its rate on one
    # core, its difference from the float64 oracle (its own rounding error)
    # and from the GPU.
    t_f, kvb_f, done_f, err_twin, err_gpu, cur_l = 0.0, 0, 0, 0.0, 0.0, -1
    for l, s, want in pairs:
        if l != cur_l:
            k_l, v_l, q_l = u16(S.k_pool[l]), u16(S.v_pool[l]), u16(S.q[l])
            got = S.out[l].cpu().numpy().astype(np.float64)
            cur_l = l
        t0 = time.perf_counter()
        want32, rc = orc.decode_f32(q_l[s:s + 1], k_l, v_l, S.tables[s:s + 1], S.ctx[s:s + 1],
                                    sh.n_kv, sh.scale)
        t_f += time.perf_counter() - t0
        assert rc == 0
        w32 = want32[0].astype(np.float64)
        err_twin = max(err_twin, float(np.abs(w32 - want).max()))
        err_gpu = max(err_gpu, float(np.abs(w32 - got[s]).max()))
        kvb_f += 2 * sh.n_kv * sh.d * 2 * int(S.ctx[s])
        done_f += 1
        if t_f >= budget_s / 3:
            break
    if cur_l >= 0:
        del k_l, v_l
    single["fp32_twin"] = {
        "value": kvb_f / t_f / 1e9 if t_f > 0 else None, "unit": "GB/s", "cores": 1,
        "sample": f"the first {done_f} of the same pairs; single-threaded C loop in float32, "
                  f"{t_f:.1f} s",
        "max_abs_vs_float64_oracle": err_twin, "max_abs_vs_gpu": err_gpu,
    }
    del pairs
    if threads_budget_s <= 0:
        return single, worst, done, None
    # The same function on P host threads, each over its own shard of the
    # sequences, over whole layers (layer 0 first) until the budget: the
    # oracle on the machine's host cores, and every row of those layers
    # compared with the GPU output.
    P = oracle.host_threads()
    t_p, kvb_p, layers_p, worst_p = 0.0, 0, 0, 0.0
    for l in range(sh.n_layers):
        k_l, v_l, q_l = u16(S.k_pool[l]), u16(S.v_pool[l]), u16(S.q[l])
        got = S.out[l].cpu().numpy().astype(np.float64)
        t0 = time.perf_counter()
        want, rc = orc.decode_sharded(q_l, k_l, v_l, S.tables, S.ctx, sh.n_kv, sh.scale, P)
        t_p += time.perf_counter() - t0
        assert rc == 0
        worst_p = max(worst_p, float(np.abs(want - got).max()))
        kvb_p += kv_bytes(S, S.ctx)
        layers_p += 1
        del k_l, v_l
        if t_p >= threads_budget_s:
            break
    gbs_p = kvb_p / t_p / 1e9
    multi = {
        "value": gbs_p, "unit": "GB/s", "cores": P, "kind": "oracle",
        "sample": (f"layers 0..{layers_p - 1} of the final state whole (all {S.B} sequences x "
                   f"{sh.n_q} query heads each), the sequences split over {P} host threads, each "
                   f"running the single-threaded C oracle in float64 on its shard; {t_p:.1f} s"),
        "seconds": t_p,
        "steps_per_s_equiv": gbs_p * 1e9 / (kv_bytes(S, S.ctx) * sh.n_layers),
        "single_core": single,
        "full_layers_checked": layers_p,
        "full_layers_max_abs": worst_p,
    }
    return multi, worst, done, worst_p


def measured_gbs(traffic, us):
    """HBM bytes per launch from the counter records over the launch's
    duration: the rate HBM actually delivered (None without a record)."""
    return None if traffic is None or not us else traffic / (us * 1e-6) / 1e9


def counter_workload(config, shard, share):
    """Name of the decode workload in the counter summaries' file names."""
    base = {1: "tiny", 2: "0.5b", 3: "llama2-7b", 4: "llama3-8b", 5: "80layer"}[config]
    if shard > 1:
        base += f"-shard{shard}"
    if config == 4:
        base += "-shared" if share else "-no-share"
    return base


def stored_traffic(workload, kernel, kernel_file="paged_attn_balanced"):
    """HBM bytes per launch of the roofline kernel (entry `kernel`) from the
    committed counter summary of this workload (profiles/pmc_*), if it was
    taken on the current kernel source."""
    path = PMC_FILE.format(kernel=kernel_file, workload=workload)
    if not os.path.exists(path):
        return None, "no counter summary"
    rec = None
    with open(path) as f:
        for line in f:
            if line.startswith("{"):
                rec = json.loads(line)
    if rec is None:
        return None, "no record in counter summary"
    if rec.get("kernel_source_sha256_16") != kernel_source_hash():
        return None, "kernel changed since the counters were taken"
    per = rec.get("hbm_bytes_per_dispatch", {})
    if kernel not in per:
        return None, f"no counters for {kernel}"
    return per[kernel], None


def verify_bench(pkv, torch, S, q_len, steps, warmup, graph=True, prefix_kernel=True,
                 cpu_seconds=0.0):
    """The verification pass of speculative decoding on the decode bench's
    state: per layer, pkv_kv_write of the q_len new tokens of every sequence
    (at positions ctx - q_len .. ctx - 1) and the verification attention;
    then once, pkv_spec_accept over a 128,256-token vocabulary. With a
    shared prefix (and prefix_kernel) the attention is
    pkv_paged_attn_verify_prefix over the sequences past the prefix (placed
    first), else pkv_paged_attn_verify. The contexts stay fixed between
    steps (the tokens are rewritten in place); the KV bytes per step are
    those of the decode at the same contexts."""
    sh, L, B = S.shape, S.shape.n_layers, S.B
    dev = torch.device("cuda")
    base = 7000
    q = w.device_normal_bf16_(torch.empty((L, B, q_len, sh.n_q, sh.d), dtype=torch.bfloat16,
                                          device=dev), base + 1)
    k_src = w.device_normal_bf16_(torch.empty((L, B * q_len, sh.n_kv, sh.d), dtype=torch.bfloat16,
                                              device=dev), base + 2)
    v_src = w.device_normal_bf16_(torch.empty_like(k_src), base + 3)
    out = torch.empty((L, B, q_len, sh.n_q, sh.d), dtype=torch.float32, device=dev)
    rows = torch.arange(B, dtype=torch.int32, device=dev).repeat_interleave(q_len)
    ctx = torch.from_numpy(S.ctx.copy()).to(dev)
    pos = (ctx.repeat_interleave(q_len) - q_len +
           torch.arange(q_len, dtype=torch.int32, device=dev).repeat(B)).to(torch.int32)
    S.cl.copy_(ctx)
    use_prefix = prefix_kernel and S.share and len(S.prefix_ids) > 0 and S.past_prefix > 0
    # (measured slower than the plain pass at the LLaMA-3-8B shape: off by default)
    if use_prefix:
        pre_ids = torch.from_numpy(S.prefix_ids).to(dev)
        ws_bytes = pkv.pkv_verify_prefix_workspace_bytes(B, q_len, sh.n_q, sh.n_kv, sh.d, S.max_ctx,
                                                         len(S.prefix_ids), S.past_prefix)
    else:
        ws_bytes = pkv.pkv_verify_workspace_bytes(B, q_len, sh.n_q, sh.n_kv, sh.d, S.max_ctx)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)

    # the acceptance rule once per step over a LLaMA-3 sized vocabulary:
    # target probabilities for the q_len positions, draft probabilities for
    # the q_len - 1 drafts (softmax of seeded N(0,1) logits), seeded drafts
    # and uniforms
    gamma = q_len - 1
    gen = torch.Generator(device=dev)
    gen.manual_seed(base + 4)
    p_t = torch.softmax(torch.randn((B, q_len, VOCAB), device=dev, generator=gen), dim=-1)
    q_d = torch.softmax(torch.randn((B, max(gamma, 1), VOCAB), device=dev, generator=gen),
                        dim=-1)[:, :gamma].contiguous()
    drafts = torch.randint(0, VOCAB, (B, gamma), device=dev, generator=gen, dtype=torch.int32)
    unif = torch.rand((B, q_len), device=dev, generator=gen)
    n_acc = torch.empty(B, dtype=torch.int32, device=dev)
    nxt = torch.empty(B, dtype=torch.int32, device=dev)
    acc_ws = torch.empty(max(pkv.pkv_spec_accept_workspace_bytes(B, VOCAB), 1), dtype=torch.uint8,
                         device=dev)

    def accept():
        pkv.pkv_spec_accept(p_t, q_d, drafts, unif, n_acc, nxt, workspace=acc_ws, err_flag=S.err)

    def write(l):
        pkv.pkv_kv_write(S.k_pool[l], S.v_pool[l], k_src[l], v_src[l], S.bt, rows, pos,
                         err_flag=S.err)

    def verify(l):
        if use_prefix:
            pkv.pkv_paged_attn_verify_prefix(out[l], q[l], S.k_pool[l], S.v_pool[l], S.bt, S.cl,
                                             sh.scale, S.max_ctx, pre_ids, 0, S.past_prefix,
                                             workspace=ws, err_flag=S.err)
        else:
            pkv.pkv_paged_attn_verify(out[l], q[l], S.k_pool[l], S.v_pool[l], S.bt, S.cl, sh.scale,
                                      S.max_ctx, workspace=ws, err_flag=S.err)

    for _ in range(warmup):
        for l in range(L):
            write(l)
            verify(l)
        accept()
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(L * steps)]
    eva = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
    t0 = time.perf_counter()
    for i in range(steps):
        for l in range(L):
            e = ev[i * L + l]
            e[0].record()
            write(l)
            e[1].record()
            verify(l)
            e[2].record()
        eva[i][0].record()
        accept()
        eva[i][1].record()
    torch.cuda.synchronize()
    eager_ms = (time.perf_counter() - t0) * 1e3 / steps
    if int(S.err.item()):
        raise RuntimeError(f"device error flag {int(S.err.item())}")
    write_us = float(np.mean([e[0].elapsed_time(e[1]) for e in ev])) * 1e3
    verify_us = float(np.mean([e[1].elapsed_time(e[2]) for e in ev])) * 1e3
    accept_us = float(np.mean([e[0].elapsed_time(e[1]) for e in eva])) * 1e3
    ms, mode = eager_ms, "eager"
    if graph:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for l in range(L):
                write(l)
                verify(l)
            accept()
        g.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            g.replay()
        torch.cuda.synchronize()
        ms, mode = (time.perf_counter() - t0) * 1e3 / steps, "hip-graph"
        if int(S.err.item()):
            raise RuntimeError(f"device error flag {int(S.err.item())}")
    kv_layer = kv_bytes(S, S.ctx)
    extra = B * (q_len - 1) * sh.n_q * sh.d * (2 + 4)
    alg = attn_alg_bytes(S, S.ctx) + extra              # logical: the prefix once per reader
    alg_u = alg - kv_layer + unique_kv_bytes(S, S.ctx)  # the bytes HBM must deliver
    cpu = rows_cpu_baseline(torch, S.k_pool[L - 1], S.v_pool[L - 1], q[L - 1], out[L - 1],
                            S.bt.cpu().numpy(), S.ctx, q_len, sh.n_kv, sh.scale, 0,
                            cpu_seconds) if cpu_seconds > 0 else None
    return {"cpu_baseline": cpu, "ms_per_step": ms, "step_mode": mode, "eager_ms_per_step": eager_ms,
            "kv_gbs": kv_layer * L / (ms * 1e-3) / 1e9,
            "kv_gbs_unique": unique_kv_bytes(S, S.ctx) * L / (ms * 1e-3) / 1e9,
            "write_us": write_us,
            "verify_us": verify_us, "accept_us": accept_us, "verify_alg_bytes": alg_u,
            "verify_alg_bytes_logical": alg,
            "verify_gbs": alg_u / (verify_us * 1e-6) / 1e9,
            "verify_gbs_logical": alg / (verify_us * 1e-6) / 1e9,
            "query_tokens_per_s": B * q_len / (ms * 1e-3),
            "verify_call": ("pkv_paged_attn_verify_prefix over the sequences past the prefix"
                            if use_prefix else "pkv_paged_attn_verify")}


def prefill_bench(pkv, torch, shape, seed, chunk, batch, steps, warmup, graph=True, cpu_seconds=0.0):
    """Chunked prefill at a model shape: batch sequences each take a chunk
    of `chunk` prompt tokens on top of 1,024..6,144 tokens already cached
    (uniform), all layers. Per layer: pkv_kv_write of the chunk's keys and
    values (batch * chunk tokens), then pkv_paged_prefill. Seeded N(0,1)
    values drawn on the device, fragmented pool. Algorithmic flops of one
    layer's prefill: for every (sequence, chunk token i, query head), 4 * d
    per visible position (q.k and p.v, 2 flops per multiply-add), positions
    0 .. ctx - chunk + i."""
    L, n_q, n_kv, d = shape.n_layers, shape.n_q, shape.n_kv, shape.d
    g = w.rng(seed, 20)
    ctx = (g.integers(1024, 6145, batch) + chunk).astype(np.int32)
    sh1 = w.Shape(shape.name, 1, n_q, n_kv, d, batch, 1, 1)
    t = w.build_tables(sh1, seed, context_lens=ctx)
    dev = torch.device("cuda")
    ks, vs = w.pool_shapes(t.num_blocks, n_kv, d)
    kp = [w.device_normal_bf16_(torch.empty(ks, dtype=torch.bfloat16, device=dev), seed * 100 + 2 * l)
          for l in range(L)]
    vp = [w.device_normal_bf16_(torch.empty(vs, dtype=torch.bfloat16, device=dev), seed * 100 + 2 * l + 1)
          for l in range(L)]
    q = w.device_normal_bf16_(torch.empty((L, batch, chunk, n_q, d), dtype=torch.bfloat16, device=dev), 31)
    k_src = w.device_normal_bf16_(torch.empty((L, batch * chunk, n_kv, d), dtype=torch.bfloat16,
                                              device=dev), 32)
    v_src = w.device_normal_bf16_(torch.empty_like(k_src), 33)
    out = torch.empty((L, batch, chunk, n_q, d), dtype=torch.float32, device=dev)
    bt = torch.from_numpy(t.block_tables).to(dev)
    cl = torch.from_numpy(ctx).to(dev)
    rows = torch.arange(batch, dtype=torch.int32, device=dev).repeat_interleave(chunk)
    pos = (cl.repeat_interleave(chunk) - chunk +
           torch.arange(chunk, dtype=torch.int32, device=dev).repeat(batch)).to(torch.int32)
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    max_ctx = int(ctx.max())

    def write(l):
        pkv.pkv_kv_write(kp[l], vp[l], k_src[l], v_src[l], bt, rows, pos, err_flag=err)

    def prefill(l):
        pkv.pkv_paged_prefill(out[l], q[l], kp[l], vp[l], bt, cl, shape.scale, max_ctx, err_flag=err)

    for _ in range(warmup):
        for l in range(L):
            write(l)
            prefill(l)
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(L * steps)]
    t0 = time.perf_counter()
    for i in range(steps):
        for l in range(L):
            e = ev[i * L + l]
            e[0].record()
            write(l)
            e[1].record()
            prefill(l)
            e[2].record()
    torch.cuda.synchronize()
    eager_ms = (time.perf_counter() - t0) * 1e3 / steps
    if int(err.item()):
        raise RuntimeError(f"device error flag {int(err.item())}")
    write_us = float(np.mean([e[0].elapsed_time(e[1]) for e in ev])) * 1e3
    prefill_us = float(np.mean([e[1].elapsed_time(e[2]) for e in ev])) * 1e3
    ms, mode = eager_ms, "eager"
    if graph:
        gr = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gr):
            for l in range(L):
                write(l)
                prefill(l)
        gr.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            gr.replay()
        torch.cuda.synchronize()
        ms, mode = (time.perf_counter() - t0) * 1e3 / steps, "hip-graph"
        if int(err.item()):
            raise RuntimeError(f"device error flag {int(err.item())}")
    seen = sum(int(c) - chunk + (chunk + 1) / 2 for c in ctx) * chunk   # visible positions, all rows of a head
    flops_layer = 4.0 * d * n_q * seen
    tflops = flops_layer / (prefill_us * 1e-6) / 1e12
    traffic, why = (stored_traffic(f"llama3-8b-prefill{chunk}x{batch}", "paged_prefill",
                                   kernel_file="paged_prefill")
                    if shape.name == w.CONFIGS[4].name and seed == 0 else (None, "other workload"))
    cpu = rows_cpu_baseline(torch, kp[L - 1], vp[L - 1], q[L - 1], out[L - 1], t.block_tables, ctx,
                               chunk, n_kv, shape.scale, seed, cpu_seconds) if cpu_seconds > 0 else None
    return {
        "metric": "chunked prefill against the paged cache: TFLOP/s of the attention",
        "value": flops_layer * L / (ms * 1e-3) / 1e12, "unit": "TFLOP/s", "n_gpus": 1,
        "steps": steps, "warmup": warmup, "ms_per_step": ms, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"prefill-{chunk}x{batch}-llama3-8b-gqa-32layer-ctx1024..6144",
                   "layers": L, "batch": batch, "chunk_tokens": chunk, "n_q_heads": n_q,
                   "n_kv_heads": n_kv, "head_dim": d, "cached_tokens": [1024, 6144], "seed": seed},
        "step_mode": mode, "prompt_tokens_per_s": batch * chunk / (ms * 1e-3),
        "kernels_us": {"kv_write": write_us, "paged_prefill": prefill_us},
        "roofline": {"kernel": "paged_prefill", "bound": "mfma", "achieved": tflops,
                     "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": tflops / MFMA_BF16_PEAK_TFLOPS, "traffic": traffic,
                     "traffic_gbs": measured_gbs(traffic, prefill_us),
                     "traffic_note": why, "alg_flops_per_launch": flops_layer},
        "cpu_baseline": cpu,
    }


def rows_cpu_baseline(torch, kp, vp, q, out, tables, ctx, chunk, n_kv, scale, seed, budget_s):
    """The oracle beside a multi-token pass (a prefill chunk, or the
    verification pass's query tokens: `chunk` tokens per sequence, the last
    of its context), on a bounded sample of the last layer's final state:
    rows (sequence, token, query head) drawn at random, the first and last
    token of every sequence first, each recomputed by the single-threaded
    C oracle in float64 (the row's attention over positions 0 .. ctx -
    chunk + token) until budget_s seconds; its rate in the pass's own flop
    count, and the largest difference from the GPU's rows."""
    import oracle
    orc = oracle.default()
    k_h = kp.view(torch.int16).cpu().numpy().view(np.uint16)
    v_h = vp.view(torch.int16).cpu().numpy().view(np.uint16)
    q_h = q.view(torch.int16).cpu().numpy().view(np.uint16)
    got = out.cpu().numpy()
    B, C, n_q, d = q_h.shape
    G = n_q // n_kv
    rnd = np.random.default_rng(seed + 77)
    picks = [(s, 0, 0) for s in range(B)] + [(s, C - 1, n_q - 1) for s in range(B)]
    rows, flops, err, spent = 0, 0.0, 0.0, 0.0
    while spent < budget_s:
        s, i, j = picks[rows] if rows < len(picks) else \
            (int(rnd.integers(B)), int(rnd.integers(C)), int(rnd.integers(n_q)))
        seen = int(ctx[s]) - chunk + i + 1
        t0 = time.perf_counter()
        want, rc = orc.decode_row(q_h[s, i, j], k_h, v_h, tables[s], seen, n_kv, j // G, scale)
        spent += time.perf_counter() - t0
        if rc != 0:
            raise RuntimeError(f"oracle status {rc}")
        err = max(err, float(np.abs(got[s, i, j] - want).max()))
        flops += 4.0 * d * seen
        rows += 1
    return {"value": flops / spent / 1e9, "unit": "GFLOP/s", "cores": 1, "kind": "oracle",
            "sample": f"{rows} (sequence, token, query head) rows of the last layer, "
                      f"{spent:.1f} s of single-threaded C oracle time in float64",
            "parity_max_abs": err, "parity_rows": rows}


def prefix_cache_bench(pkv, seed, n_req=2000):
    """The prefix cache on the host, with a multi-turn chat workload at the
    LLaMA-3-8B context sizes. 64 conversations each share one of four
    2,048-token system prompts. Every request extends its conversation's
    last request by 50..400 tokens (the user's turn), generates 64..256
    tokens, and ends the conversation at 8,192 tokens. Per request: match
    (all but the last prompt token), grow the table, insert the whole
    sequence at the end, release it. The pool holds 16,384 blocks, so the
    cache evicts. Times are host wall-clock."""
    rnd = np.random.default_rng(seed)
    n_blocks, max_blocks = 16384, 8192 // BLOCK
    alloc = pkv.Allocator(n_blocks)
    pc = pkv.PrefixCache(alloc)
    systems = [rnd.integers(0, 128256, 2048).astype(np.int32) for _ in range(4)]
    convs = [systems[i % 4].copy() for i in range(64)]
    table = np.full(max_blocks, -1, np.int32)
    t_match = t_insert = t_evict = 0.0
    prompt_tokens = matched_tokens = 0
    for r in range(n_req):
        c = int(rnd.integers(64))
        turn = rnd.integers(0, 128256, int(rnd.integers(50, 401))).astype(np.int32)
        gen = rnd.integers(0, 128256, int(rnd.integers(64, 257))).astype(np.int32)
        prompt = np.concatenate([convs[c], turn])
        if len(prompt) + len(gen) > 8192:
            prompt = np.concatenate([systems[c % 4], turn])
        tokens = np.concatenate([prompt, gen])
        t0 = time.perf_counter()
        m = pc.match(prompt[:-1], max_blocks)
        t_match += time.perf_counter() - t0
        prompt_tokens += len(prompt)
        matched_tokens += BLOCK * len(m)
        table[:] = -1
        table[:len(m)] = m
        need = -(-len(tokens) // BLOCK) - len(m)
        if need > alloc.pkv_num_free():
            t0 = time.perf_counter()
            pc.evict(need - alloc.pkv_num_free())
            t_evict += time.perf_counter() - t0
        st, nb, _, _ = alloc.pkv_seq_grow(table, len(m), len(tokens))
        if st != pkv.PKV_OK:
            raise RuntimeError("pool too small for one request")
        t0 = time.perf_counter()
        pc.insert(tokens, table[:nb])
        t_insert += time.perf_counter() - t0
        alloc.pkv_seq_release(table, nb)
        convs[c] = tokens
    return {
        "metric": "prefix cache: prompt tokens served from cache, host time per operation",
        "value": matched_tokens / prompt_tokens, "unit": "fraction of prompt tokens",
        "n_gpus": 1, "steps": n_req, "warmup": 0, "ms_per_step": None,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "int32",
        "data": "synthetic",
        "config": {"workload": "multi-turn chat, 64 conversations, 4 x 2048-token system prompts, "
                               "contexts up to 8192, 16384-block pool", "seed": seed},
        "us_per_match": 1e6 * t_match / n_req, "us_per_insert": 1e6 * t_insert / n_req,
        "evict_ms_total": 1e3 * t_evict, "prompt_tokens": prompt_tokens,
        "matched_tokens": matched_tokens, "cached_blocks_end": pc.cached_blocks(),
    }


def loop_bench(pkv, torch, shape, name, seed, steps, warmup, graphs=False, prefix_kernel=True):
    """Continuous batching at a model shape: requests with prompts uniform in
    [prefix, ctx_hi - 256] tokens (all beginning with the shared prefix when
    the shape has one) and 32..256 generated tokens, queued ahead; the
    batcher keeps max_batch of them resident, finished ones release their
    blocks and waiting ones are admitted with their prompt keys/values
    written (pkv_kv_write). Every step is the whole loop: the batcher's
    plan, its upload, per layer copies + prompt writes + pkv_decode_step,
    and a synchronisation (a server samples from the outputs before the
    next step). Keys, values and queries are seeded N(0,1) on the device,
    in the loop's own input buffers. With graphs, the decode launches of a
    step are replayed from a HIP graph cached per row count (the loop's
    copies and prompt writes stay eager); measured slower than issuing them
    eagerly, whose launches the host already queues ahead of the GPU."""
    from paged_kv_cache_468_amd.loop import ServingLoop
    L, B, n_kv, d = shape.n_layers, shape.batch, shape.n_kv, shape.d
    max_blocks = -(-shape.ctx_hi // BLOCK)
    prefix = shape.prefix_tokens
    num_blocks = B * max_blocks + -(-prefix // BLOCK)
    b = pkv.Batcher(num_blocks, B, max_blocks, prefix)
    rnd = np.random.default_rng(seed)
    n_req = 4000
    lo = max(prefix, shape.ctx_lo)
    prompts = rnd.integers(lo, shape.ctx_hi - 256 + 1, n_req)
    gens = rnd.integers(32, 257, n_req)
    for rid in range(n_req):
        b.submit(rid, int(prompts[rid]), int(gens[rid]), prefix > 0)
    ks, vs = w.pool_shapes(num_blocks, n_kv, d)
    kp = [torch.empty(ks, dtype=torch.bfloat16, device="cuda") for _ in range(L)]
    vp = [torch.empty(vs, dtype=torch.bfloat16, device="cuda") for _ in range(L)]
    for l in range(L):
        w.device_normal_bf16_(kp[l], seed * 1000 + 2 * l)
        w.device_normal_bf16_(vp[l], seed * 1000 + 2 * l + 1)
    cap = B * BLOCK * max_blocks
    src_k = torch.empty((cap, n_kv, d), dtype=torch.bfloat16, device="cuda")
    src_v = torch.empty_like(src_k)
    w.device_normal_bf16_(src_k, seed * 1000 + 900)
    w.device_normal_bf16_(src_v, seed * 1000 + 901)
    loop = ServingLoop(b, kp, vp, shape.n_q, shape.scale, B, graphs=graphs,
                       prefix_kernel=prefix_kernel)
    for i, t in enumerate(loop.inputs()):
        w.device_normal_bf16_(t, seed * 1000 + 950 + i)
    if prefix:
        loop.write_prefix([src_k[:prefix]] * L, [src_v[:prefix]] * L)
    stream = loop.stream
    per_token = 2 * n_kv * d * 2 * L          # K and V bytes of one cached token, all layers
    # the prefix's whole blocks (allocated when the batcher is created)
    pre_ids = (b.prefix_table()[0][:prefix // BLOCK].copy() if prefix
               else np.zeros(0, np.int32))

    def one_step(acc):
        t = time.perf_counter()
        p = loop.schedule()
        acc["host_s"] += time.perf_counter() - t
        n, n_fill = p.num_seqs, len(p.fill_rows)
        loop.run(lambda l: (src_k[:n_fill], src_v[:n_fill]), None, None, None)
        stream.synchronize()
        acc["tokens"] += n
        acc["members"] += loop.members[1]
        acc["kv_bytes"] += per_token * int(p.context_lens.astype(np.int64).sum())
        # the bytes HBM must deliver: the prefix's blocks once, however many
        # rows hold them
        held = int((p.block_tables[:n, :len(pre_ids)] == pre_ids).sum()) if len(pre_ids) else 0
        acc["kv_bytes_unique"] += per_token * (int(p.context_lens.astype(np.int64).sum())
                                               - BLOCK * held + (BLOCK * len(pre_ids) if held else 0))
        acc["fill"] += n_fill
        ids = set(p.request_ids.tolist())
        acc["admitted"] += len(ids - acc["prev"])
        acc["prev"] = ids
        acc["finished"] += len(p.finished_ids)
        acc["cow"] += len(p.cow_src)

    def fresh():
        return dict(host_s=0.0, tokens=0, members=0, kv_bytes=0, kv_bytes_unique=0, fill=0,
                    admitted=0, finished=0, cow=0, prev=set())

    acc = fresh()
    for _ in range(warmup):
        one_step(acc)
    torch.cuda.synchronize()
    prev = acc["prev"]
    acc = fresh()
    acc["prev"] = prev
    t0 = time.perf_counter()
    for i in range(steps):
        one_step(acc)
        if (i + 1) % 100 == 0:
            log(f"[loop] {i + 1}/{steps} steps")
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    assert int(loop.err.item()) == 0, "device error flag set in the loop"
    return {
        "metric": "continuous-batching decode tokens/s (whole loop)",
        "value": acc["tokens"] / dt, "unit": "tokens/s", "n_gpus": 1, "steps": steps,
        "warmup": warmup, "ms_per_step": 1e3 * dt / steps, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "continuous-batching-" + name, "layers": L, "max_batch": B, "n_q_heads": shape.n_q,
                   "n_kv_heads": n_kv, "head_dim": d, "prefix_tokens": prefix,
                   "prompt_tokens": [int(lo), int(shape.ctx_hi - 256)], "gen_tokens": [32, 256],
                   "blocks_per_layer": num_blocks, "seed": seed},
        "kv_gbs_logical": acc["kv_bytes"] / dt / 1e9,
        "kv_gbs_unique": acc["kv_bytes_unique"] / dt / 1e9,
        "pct_hbm_peak": 100 * acc["kv_bytes_unique"] / dt / 1e9 / HBM_PEAK_GBS,
        "pct_hbm_peak_logical": 100 * acc["kv_bytes"] / dt / 1e9 / HBM_PEAK_GBS,
        "bytes_note": ("logical: K and V of every row's whole context; unique: the shared "
                       "prefix's whole blocks once per step (the bytes HBM must deliver)"),
        "rows_per_step": acc["tokens"] / steps,
        "host_ms_per_step": 1e3 * acc["host_s"] / steps,
        "prompt_tokens_written_per_step": acc["fill"] / steps,
        "admitted_per_step": acc["admitted"] / steps,
        "finished_per_step": acc["finished"] / steps,
        "cow_per_step": acc["cow"] / steps,
        "decode_call": ("pkv_decode_step_prefix over the rows holding the shared prefix"
                        if loop.n_pre else "pkv_decode_step"),
        "prefix_member_rows_per_step": acc["members"] / steps,
        "decode_launches": "hip-graph, cached per row count" if graphs else "eager",
        "graph_captures": loop.graph_captures, "graph_replays_from_cache": loop.graph_hits,
    }


def copy_calibration(torch, mib):
    """A plain device copy of mib MiB, three times: the reference the
    counter runs scale FETCH_SIZE and WRITE_SIZE by."""
    if mib <= 0:
        return
    a = torch.empty(mib << 20, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    a.fill_(1)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    del a, b


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", type=int, default=4, choices=sorted(w.CONFIGS))
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--shard", type=int, default=1,
                    help="time one GPU's share of the shape split by KV head over this many GPUs")
    ap.add_argument("--partition-tokens", type=int, default=0)
    ap.add_argument("--no-share", action="store_true", help="main run with private prefix copies")
    ap.add_argument("--skip-no-share", action="store_true", help="skip the second, unshared run")
    ap.add_argument("--no-graph", action="store_true", help="time the step eagerly instead of replaying a HIP graph")
    ap.add_argument("--no-prefix-kernel", action="store_true",
                    help="shared prefix: pkv_decode_step (every sequence reads the prefix through "
                         "its own table) instead of pkv_decode_step_prefix")
    ap.add_argument("--valu", action="store_true",
                    help="decode without a shared prefix with the partition kernel's scores and "
                         "P.V on the vector ALUs (pkv_decode_step_partition_valu) instead of "
                         "the matrix cores, for comparison")
    ap.add_argument("--unfused", action="store_true",
                    help="three launches per layer (kv_append, partition, merge) instead of pkv_decode_step")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="one-core oracle budget; 0 skips the oracle")
    ap.add_argument("--cpu-threads-seconds", type=float, default=8.0,
                    help="budget of the oracle on the host's threads over whole layers (at least "
                         "one layer); 0 skips it")
    ap.add_argument("--verify-tokens", type=int, default=0,
                    help="speculative verification instead: this many query tokens per sequence")
    ap.add_argument("--verify-prefix-kernel", action="store_true",
                    help="verification pass: pkv_paged_attn_verify_prefix over the sequences past "
                         "the shared prefix instead of pkv_paged_attn_verify")
    ap.add_argument("--prefill-chunk", type=int, default=0,
                    help="chunked prefill instead: chunk tokens per sequence on top of cached context")
    ap.add_argument("--prefill-batch", type=int, default=8)
    ap.add_argument("--prefix-cache", action="store_true",
                    help="host benchmark of the prefix cache on a multi-turn chat workload")
    ap.add_argument("--loop", action="store_true",
                    help="continuous batching instead: the batcher's plans carried out step by step")
    ap.add_argument("--loop-no-prefix-kernel", action="store_true",
                    help="serving loop: pkv_decode_step for every row, the shared prefix "
                         "included, instead of pkv_decode_step_prefix")
    ap.add_argument("--loop-graphs", action="store_true",
                    help="continuous batching with the decode launches replayed from cached graphs")
    ap.add_argument("--loop-steps", type=int, default=300)
    ap.add_argument("--loop-warmup", type=int, default=300)
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="also run a plain device copy of this many MiB (counter calibration)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py: the library runs on one GPU only; --gpus {args.gpus} is not supported "
              "(no collectives or sharding are implemented).", file=sys.stderr)
        sys.exit(2)

    if args.prefix_cache:   # host only
        import paged_kv_cache_468_amd as pkv
        print(json.dumps(prefix_cache_bench(pkv, args.seed)), flush=True)
        return
    import torch
    if not torch.cuda.is_available():
        print("bench.py: needs a GPU", file=sys.stderr)
        sys.exit(1)
    import paged_kv_cache_468_amd as pkv
    torch.cuda.set_device(0)
    shape = w.tp_shard(w.CONFIGS[args.config], args.shard)
    wname = WORKLOAD_NAMES[args.config] + (f"-shard1of{args.shard}-by-kv-head" if args.shard > 1 else "")
    stored = args.shard in (1, 4)     # the workloads the counter records cover
    if args.loop:
        log(f"[bench] continuous batching, {wname}")
        line = loop_bench(pkv, torch, shape, wname, args.seed, args.loop_steps, args.loop_warmup,
                          graphs=args.loop_graphs, prefix_kernel=not args.loop_no_prefix_kernel)
        print(json.dumps(line), flush=True)
        return
    if args.prefill_chunk > 0:
        log(f"[bench] chunked prefill, {args.prefill_chunk}-token chunks x {args.prefill_batch}")
        line = prefill_bench(pkv, torch, shape, args.seed, args.prefill_chunk, args.prefill_batch,
                             args.steps, args.warmup, graph=not args.no_graph,
                             cpu_seconds=min(args.cpu_seconds, 10.0))
        if line["cpu_baseline"] is not None:
            cb = line["cpu_baseline"]
            log(f"[bench] oracle {cb['value']:.2f} GFLOP/s on 1 thread, parity max-abs "
                f"{cb['parity_max_abs']:.2e} over {cb['parity_rows']} rows")
            if not cb["parity_max_abs"] <= 1e-3:
                raise RuntimeError(f"prefill parity {cb['parity_max_abs']:.3e} > 1e-3")
        copy_calibration(torch, args.copy_calibration_mib)
        print(json.dumps(line), flush=True)
        return
    extra = args.warmup + 2 * args.steps + 1   # one token per step: eager, graph warm-up, graph
    if args.verify_tokens > 0:
        log(f"[bench] verification pass, {args.verify_tokens} query tokens, {wname}")
        share_v = shape.prefix_tokens > 0 and not args.no_share
        S = build_state(pkv, torch, shape, args.seed, share_v, extra, 0,
                        prefix_kernel=not args.no_prefix_kernel)
        dec = run(pkv, torch, S, args.steps, args.warmup, graph=not args.no_graph)
        log(f"[bench] decode on the same state: {dec['ms_per_step']:.3f} ms/step")
        vr = verify_bench(pkv, torch, S, args.verify_tokens, args.steps, args.warmup,
                          graph=not args.no_graph, prefix_kernel=args.verify_prefix_kernel,
                          cpu_seconds=min(args.cpu_seconds, 10.0))
        if vr["cpu_baseline"] is not None:
            cb = vr["cpu_baseline"]
            log(f"[bench] oracle {cb['value']:.2f} GFLOP/s on 1 thread, parity max-abs "
                f"{cb['parity_max_abs']:.2e} over {cb['parity_rows']} rows")
            if not cb["parity_max_abs"] <= 1e-3:
                raise RuntimeError(f"verification parity {cb['parity_max_abs']:.3e} > 1e-3")
        log(f"[bench] verify: {vr['ms_per_step']:.3f} ms/step, write {vr['write_us']:.1f} us, "
            f"verify {vr['verify_us']:.1f} us per layer")
        vtraffic, vwhy = (stored_traffic(f"llama3-8b-verify{args.verify_tokens}", "paged_attn_verify",
                                         "paged_attn_verify")
                          if args.config == 4 and args.shard == 1 and share_v
                          else (None, "other workload"))
        line = {
            "metric": "speculative verification pass: KV GB/s and time vs one decode step",
            "value": vr["kv_gbs"], "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": vr["ms_per_step"], "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
            "config": {"workload": "verify-" + wname,
                       "query_tokens": args.verify_tokens, "layers": shape.n_layers,
                       "batch": S_batch(shape), "n_q_heads": shape.n_q, "n_kv_heads": shape.n_kv,
                       "head_dim": shape.d, "shared_prefix_tokens": shape.prefix_tokens if share_v else 0},
            "step_mode": vr["step_mode"], "decode_ms_per_step": dec["ms_per_step"],
            "verify_over_decode": vr["ms_per_step"] / dec["ms_per_step"],
            "verify_call": vr["verify_call"],
            "kv_gbs_logical": vr["kv_gbs"], "kv_gbs_unique": vr["kv_gbs_unique"],
            "query_tokens_per_s": vr["query_tokens_per_s"],
            "kernels_us": {"kv_write": vr["write_us"], "paged_attn_verify": vr["verify_us"],
                           "spec_accept": vr["accept_us"]},
            "vocab": VOCAB, "cpu_baseline": vr["cpu_baseline"],
            "roofline": {"kernel": "paged_attn_verify", "bound": "hbm", "achieved": vr["verify_gbs"],
                         "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": vr["verify_gbs"] / HBM_PEAK_GBS, "traffic": vtraffic,
                         "traffic_gbs": measured_gbs(vtraffic, vr["verify_us"]),
                         "traffic_note": vwhy, "alg_bytes_per_launch": vr["verify_alg_bytes"],
                         "achieved_logical": vr["verify_gbs_logical"],
                         "alg_bytes_per_launch_logical": vr["verify_alg_bytes_logical"],
                         "note": "events around each pkv_paged_attn_verify call (verify and merge "
                                 "kernels); achieved counts the bytes HBM must deliver (the "
                                 "shared prefix once), achieved_logical every reader's copy"},
        }
        del S
        torch.cuda.empty_cache()
        copy_calibration(torch, args.copy_calibration_mib)
        print(json.dumps(line), flush=True)
        return

    share_main = (not args.no_share) and shape.prefix_tokens > 0
    log(f"[bench] building {wname} share={share_main}")
    S = build_state(pkv, torch, shape, args.seed, share_main, extra, args.partition_tokens,
                    fused=not args.unfused, prefix_kernel=not args.no_prefix_kernel,
                    valu=args.valu)
    log(f"[bench] {S.num_blocks} blocks/layer, partition {S.partition} (0: balanced over {S.split_waves} waves), cow {S.n_cow}; timing")
    main_r = run(pkv, torch, S, args.steps, args.warmup, graph=not args.no_graph)
    log(f"[bench] main: {main_r['ms_per_step']:.3f} ms/step ({main_r['step_mode']}), "
        f"{main_r['kv_gbs']:.0f} GB/s; {main_r['dominant']} {main_r['dominant_us']:.1f} us = "
        f"{main_r['dominant_gbs']:.0f} GB/s; kernels {main_r['kernels_us']}")

    cpu, parity, n_par, parity_full = None, None, 0, None
    if args.cpu_seconds > 0:
        log("[bench] cpu oracle baseline")
        cpu, parity, n_par, parity_full = cpu_baseline(torch, S, args.cpu_seconds,
                                                       args.cpu_threads_seconds)
        log(f"[bench] oracle {cpu['value']:.3f} GB/s on {cpu['cores']} threads, parity max-abs "
            f"{parity:.2e} over {n_par} (sequence, layer) pairs"
            + (f", {parity_full:.2e} over {cpu['full_layers_checked']} whole layers"
               if parity_full is not None else ""))
    del S
    torch.cuda.empty_cache()

    extra_runs = {}
    if shape.prefix_tokens > 0 and share_main and not args.skip_no_share:
        log("[bench] no-share run")
        S2 = build_state(pkv, torch, shape, args.seed, False, extra, args.partition_tokens,
                         fused=not args.unfused, valu=args.valu)
        r2 = run(pkv, torch, S2, args.steps, args.warmup, graph=not args.no_graph)
        log(f"[bench] no-share: {r2['ms_per_step']:.3f} ms/step ({r2['step_mode']}), "
            f"{r2['kv_gbs']:.0f} GB/s; {r2['dominant']} {r2['dominant_us']:.1f} us = "
            f"{r2['dominant_gbs']:.0f} GB/s; kernels {r2['kernels_us']}")
        t2, why2 = (stored_traffic(counter_workload(args.config, args.shard, False), r2["dominant"])
                    if stored else (None, "other workload"))
        extra_runs["no_share"] = {
            "value": r2["kv_gbs"], "unit": "GB/s", "ms_per_step": r2["ms_per_step"],
            "step_mode": r2["step_mode"], "eager_ms_per_step": r2["eager_ms_per_step"],
            "steps_per_s": r2["steps_per_s"],
            "ms_per_step_median": r2["ms_per_step_median"], "ms_per_step_min": r2["ms_per_step_min"],
            "kv_gbs_logical": r2["kv_gbs"], "kv_gbs_unique": r2["kv_gbs_unique"],
            "pct_hbm_peak": 100 * r2["kv_gbs_unique"] / HBM_PEAK_GBS,
            "pct_hbm_peak_logical": 100 * r2["kv_gbs"] / HBM_PEAK_GBS,
            "kernels_us": r2["kernels_us"],
            "roofline": {"kernel": r2["dominant"], "bound": "hbm", "achieved": r2["dominant_gbs"],
                         "duration_us": r2["dominant_us"], "timing": r2["dominant_timing"],
                         "us_per_launch_events_in_step": r2["dominant_us_per_launch_events"],
                         "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": r2["dominant_gbs"] / HBM_PEAK_GBS, "traffic": t2,
                         "traffic_gbs": measured_gbs(t2, r2["dominant_us"]),
                         "traffic_note": why2, "alg_bytes_per_launch": r2["dominant_alg_bytes"]},
            "num_blocks_per_layer": r2["num_blocks_per_layer"],
        }
        del S2
        torch.cuda.empty_cache()

    copy_calibration(torch, args.copy_calibration_mib)

    traffic, why = (stored_traffic(counter_workload(args.config, args.shard, share_main),
                                   main_r["dominant"]) if stored else (None, "other workload"))
    line = {
        "metric": "paged decode-attention KV GB/s (% of HBM peak) + steps/s, Llama-3-8B shape",
        "value": main_r["kv_gbs"],
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": main_r["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": wname,
            "layers": shape.n_layers, "batch": S_batch(shape), "n_q_heads": shape.n_q,
            "n_kv_heads": shape.n_kv, "head_dim": shape.d, "block_tokens": BLOCK,
            "context": ([int(c) for c in shape.fixed_ctx] if shape.fixed_ctx else [shape.ctx_lo, shape.ctx_hi]),
            "shared_prefix_tokens": shape.prefix_tokens if share_main else 0,
            "seed": args.seed, "partition_tokens": main_r["partition_tokens"],
            "split_waves": main_r["split_waves"],
        },
        "step_mode": main_r["step_mode"],
        "eager_ms_per_step": main_r["eager_ms_per_step"],
        "steps_per_s": main_r["steps_per_s"],
        "seq_tokens_per_s": main_r["seq_tokens_per_s"],
        "tokens_per_s": main_r["tokens_per_s"],
        "ms_per_step_median": main_r["ms_per_step_median"],
        "ms_per_step_min": main_r["ms_per_step_min"],
        "ms_per_step_max": main_r["ms_per_step_max"],
        "kv_gbs_logical": main_r["kv_gbs"],
        "kv_gbs_unique": main_r["kv_gbs_unique"],
        "pct_hbm_peak": 100 * main_r["kv_gbs_unique"] / HBM_PEAK_GBS,
        "pct_hbm_peak_logical": 100 * main_r["kv_gbs"] / HBM_PEAK_GBS,
        "bytes_note": ("value and kv_gbs_logical count K and V of every sequence's whole context "
                       "(a shared prefix once per sequence that reads it); kv_gbs_unique and "
                       "pct_hbm_peak count each physical block once (the bytes HBM must deliver), "
                       "over the same step time; pct_hbm_peak_logical is the logical rate over "
                       "8 TB/s and exceeds 100 when a shared prefix is read once"),
        "kv_bytes_per_step": main_r["kv_bytes_per_step"],
        "kv_bytes_unique_per_step": main_r["kv_bytes_unique_per_step"],
        "kernels_us": main_r["kernels_us"],
        "roofline": {
            "kernel": main_r["dominant"],
            "bound": "hbm",
            "achieved": main_r["dominant_gbs"],
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": main_r["dominant_gbs"] / HBM_PEAK_GBS,
            "traffic": traffic,
            "traffic_gbs": measured_gbs(traffic, main_r["dominant_us"]),
            "traffic_note": why,
            "alg_bytes_per_launch": main_r["dominant_alg_bytes"],
            "duration_us": main_r["dominant_us"],
            "timing": main_r["dominant_timing"],
            "us_per_launch_events_in_step": main_r["dominant_us_per_launch_events"],
            "note": ("decode_step_prefix: the whole call (prefix, partition and merge kernels) "
                     "against the bytes it must move, the shared prefix counted once; value "
                     "counts every sequence's whole context (logical KV bytes). no_share gives "
                     "the partition kernel alone with every byte unique"
                     if main_r["dominant"] == "decode_step_prefix" else
                     "with a shared prefix the algorithmic bytes count every sequence's whole "
                     "context while the shared blocks are re-read from cache, so achieved can "
                     "exceed HBM peak (no_share gives the all-unique case)"),
        },
        "cpu_baseline": cpu,
        "parity_sample_max_abs": parity,
        "parity_full_layers_max_abs": parity_full,
        **extra_runs,
    }
    print(json.dumps(line), flush=True)


def S_batch(shape):
    return len(shape.fixed_ctx) if shape.fixed_ctx else shape.batch


if __name__ == "__main__":
    main()
