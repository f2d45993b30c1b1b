"""Continuous batching on the device: the batcher's plan, carried out.

Each step ("Designing an LLM serving system", "Continuous batching": before
every token step finished sequences release their blocks, waiting requests
are admitted, one decode step runs for the resident batch):
  1. pkv_batcher_step (native, host): releases, growth, preemption,
     admission; the plan;
  2. the plan's tables, context lengths, copy pairs and fill coordinates go
     to the device from pinned staging buffers, asynchronously, on the
     loop's stream;
  3. for every layer, in stream order: pkv_copy_blocks for the plan's
     copy-on-write pairs, pkv_kv_write for the prompt tokens admitted this
     step (their keys and values come from the caller: a prefill's output,
     or a preempted request's recomputed tokens), pkv_decode_step for the
     resident rows (the new token's key/value appended inside the
     attention); with the batcher's shared prefix, pkv_decode_step_prefix
     over the longest run of rows whose tables start with the prefix's
     blocks (found on the host from the plan), so the prefix's tiles are
     read once for all of them.
Everything runs in the library's kernels and its native batcher; this
module only moves arguments. The keys, values and queries are the
caller's: in a model they come from the layers' projections.

The staging buffers are reused every step: schedule() waits until the
previous step's uploads have left them (an event, not a device-wide sync).

With graphs=True the decode launches of all layers are replayed from a HIP
graph captured for the step's row count and input addresses (a few kept,
the least recently used dropped): once the batch is full and the caller
writes the step's queries and new keys/values into the loop's own input
buffers (inputs()), every step replays the same graph. The copies and
prompt writes of a step run first, eagerly (their counts change from step
to step); each touches only its layer's pools, so running them before the
decodes keeps every layer's order.
"""
from collections import OrderedDict

import numpy as np

from . import (Batcher, _torch, pkv_copy_blocks, pkv_decode_prefix_workspace_bytes,
               pkv_decode_step, pkv_decode_step_prefix, pkv_decode_workspace_bytes, pkv_kv_write)


class ServingLoop:
    """Device state for one batcher: per-layer pools and outputs, device
    tables, one workspace sized for the largest batch and context."""

    def __init__(self, batcher: Batcher, k_pools, v_pools, n_q: int, scale: float,
                 max_batch: int, stream=None, graphs: bool = False, max_graphs: int = 4,
                 prefix_kernel: bool = True):
        torch = _torch()
        self.b = batcher
        self.k_pools, self.v_pools = k_pools, v_pools
        self.n_layers = len(k_pools)
        _, self.n_kv, _, self.d = k_pools[0].shape
        self.n_q, self.scale = n_q, scale
        self.max_batch = max_batch
        self.max_blocks = batcher.max_blocks_per_seq
        self.max_ctx = 16 * self.max_blocks
        dev = k_pools[0].device
        self.dev = dev
        self.stream = stream if stream is not None else torch.cuda.current_stream(dev)
        i32 = torch.int32
        self.bt = torch.full((max_batch, self.max_blocks), -1, dtype=i32, device=dev)
        self.cl = torch.ones((max_batch,), dtype=i32, device=dev)
        self.bt_h = torch.empty((max_batch, self.max_blocks), dtype=i32, pin_memory=True)
        self.cl_h = torch.empty((max_batch,), dtype=i32, pin_memory=True)
        # copy pairs (src, dst) and fill coordinates (row, position); grown on demand
        self.cow_h = self.cow = self.fill_h = self.fill = None
        self._size_cow(2 * max_batch)
        self._size_fill(max_batch * 16)
        self.out = torch.empty((self.n_layers, max_batch, n_q, self.d), dtype=torch.float32,
                               device=dev)
        self.err = torch.zeros(1, dtype=i32, device=dev)
        ws = pkv_decode_workspace_bytes(max_batch, n_q, self.n_kv, self.d, self.max_ctx, 0)
        # the shared prefix's whole blocks, read once per step for the rows
        # that hold them (a partly filled last block is copied by every
        # request that shares the prefix, so it is not shared)
        table, _ = batcher.prefix_table()
        n_pre = batcher.prefix_tokens // 16
        self.n_pre = n_pre if prefix_kernel else 0
        self.pre_h = table[:n_pre].copy()
        self.pre_table = None
        self.members = (0, 0)   # (first row, count) of this step's prefix call
        if self.n_pre:
            self.pre_table = torch.from_numpy(self.pre_h).to(dev)
            ws = max(ws, pkv_decode_prefix_workspace_bytes(max_batch, n_q, self.n_kv, self.d,
                                                           self.max_ctx, self.n_pre, max_batch))
        self.ws = torch.empty(max(ws, 1), dtype=torch.uint8, device=dev)
        self.uploaded = torch.cuda.Event()
        self.uploaded.record(self.stream)
        self.plan = None
        self.graphs = OrderedDict() if graphs else None
        self.max_graphs = max_graphs
        self.graph_hits = self.graph_captures = 0
        self._inputs = None

    def inputs(self):
        """The loop's own input buffers (q [L][max_batch, n_q, d], k_new and
        v_new [L][max_batch, n_kv, d], bf16): write a step's rows 0 .. n-1
        into them and call run() with q = k_new = v_new = None."""
        if self._inputs is None:
            torch = _torch()
            bf = torch.bfloat16
            L, B = self.n_layers, self.max_batch
            self._inputs = (torch.zeros((L, B, self.n_q, self.d), dtype=bf, device=self.dev),
                            torch.zeros((L, B, self.n_kv, self.d), dtype=bf, device=self.dev),
                            torch.zeros((L, B, self.n_kv, self.d), dtype=bf, device=self.dev))
        return self._inputs

    def _size_cow(self, n):
        if self.cow_h is None or self.cow_h.shape[1] < n:
            torch = _torch()
            self.cow_h = torch.empty((2, n), dtype=torch.int32, pin_memory=True)
            self.cow = torch.empty((2, n), dtype=torch.int32, device=self.dev)

    def _size_fill(self, n):
        if self.fill_h is None or self.fill_h.shape[1] < n:
            torch = _torch()
            self.fill_h = torch.empty((2, n), dtype=torch.int32, pin_memory=True)
            self.fill = torch.empty((2, n), dtype=torch.int32, device=self.dev)

    def write_prefix(self, k_src, v_src):
        """Keys and values of the shared prefix ([L][prefix_tokens, n_kv, d]
        bf16, per layer) into the prefix's blocks."""
        torch = _torch()
        table, n = self.b.prefix_table()
        if n == 0:
            return
        with torch.cuda.stream(self.stream):
            bt = torch.from_numpy(table.reshape(1, -1)).to(self.dev)
            n_tok = k_src[0].shape[0]
            rows = torch.zeros(n_tok, dtype=torch.int32, device=self.dev)
            pos = torch.arange(n_tok, dtype=torch.int32, device=self.dev)
            for l in range(self.n_layers):
                pkv_kv_write(self.k_pools[l], self.v_pools[l], k_src[l], v_src[l], bt, rows, pos,
                             err_flag=self.err, stream=self.stream)

    def schedule(self):
        """Host half of a step: the batcher's plan, its arrays uploaded
        (asynchronously, on the loop's stream)."""
        torch = _torch()
        p = self.b.step()
        self.plan = p
        n, n_cow, n_fill = p.num_seqs, len(p.cow_src), len(p.fill_rows)
        self.members = self._member_run(p) if self.n_pre and n else (0, 0)
        self.uploaded.synchronize()       # the staging buffers are free again
        self._size_cow(n_cow)
        self._size_fill(n_fill)
        with torch.cuda.stream(self.stream):
            if n:
                self.bt_h.numpy()[:n] = p.block_tables
                self.cl_h.numpy()[:n] = p.context_lens
                self.bt[:n].copy_(self.bt_h[:n], non_blocking=True)
                self.cl[:n].copy_(self.cl_h[:n], non_blocking=True)
            if n_cow:
                self.cow_h.numpy()[0, :n_cow] = p.cow_src
                self.cow_h.numpy()[1, :n_cow] = p.cow_dst
                self.cow[:, :n_cow].copy_(self.cow_h[:, :n_cow], non_blocking=True)
            if n_fill:
                self.fill_h.numpy()[0, :n_fill] = p.fill_rows
                self.fill_h.numpy()[1, :n_fill] = p.fill_positions
                self.fill[:, :n_fill].copy_(self.fill_h[:, :n_fill], non_blocking=True)
            self.uploaded.record(self.stream)
        return p

    def _member_run(self, p):
        """The longest run of rows whose contexts extend past the shared
        prefix and whose tables start with its blocks (rows whose contexts
        end inside it may sit in the run too: they read their own blocks)."""
        pre = self.n_pre
        holds = (p.block_tables[:, :pre] == self.pre_h).all(axis=1)
        ok = holds | ((p.context_lens.astype(np.int64) - 1) // 16 < pre)
        best, start = (0, 0), None
        for i, v in enumerate(list(ok) + [False]):
            if v and start is None:
                start = i
            elif not v and start is not None:
                if i - start > best[1]:
                    best = (start, i - start)
                start = None
        return best

    def run(self, fill_kv, q, k_new, v_new):
        """Device half of the scheduled step. fill_kv(l) -> (k_src, v_src)
        bf16 [n_fill, n_kv, d] for the plan's fill tokens of layer l (not
        called when there are none); q [L][n, n_q, d], k_new / v_new
        [L][n, n_kv, d] for the plan's rows. Returns the outputs
        [L][n, n_q, d] (a view, valid until the next run)."""
        torch = _torch()
        p = self.plan
        n, n_cow, n_fill = p.num_seqs, len(p.cow_src), len(p.fill_rows)
        if q is None:
            qb, kb, vb = self.inputs()
            q, k_new, v_new = qb[:, :n], kb[:, :n], vb[:, :n]
        if self.graphs is None:
            with torch.cuda.stream(self.stream):
                for l in range(self.n_layers):
                    self._writes(l, n, n_cow, n_fill, fill_kv)
                    if n:
                        self._decode(l, n, q, k_new, v_new, self.stream)
            return self.out[:, :n]
        with torch.cuda.stream(self.stream):
            for l in range(self.n_layers):
                self._writes(l, n, n_cow, n_fill, fill_kv)
            if n:
                key = (n,) + self.members + tuple(t.data_ptr() for x in (q, k_new, v_new)
                                                  for t in (x[l] for l in range(self.n_layers)))
                g = self.graphs.pop(key, None)
                if g is None:
                    g = torch.cuda.CUDAGraph()
                    # the calls name the current stream, which is the capture
                    # stream inside the capture
                    with torch.cuda.graph(g):
                        for l in range(self.n_layers):
                            self._decode(l, n, q, k_new, v_new, None)
                    self.graph_captures += 1
                    while len(self.graphs) >= self.max_graphs:
                        self.graphs.popitem(last=False)
                else:
                    self.graph_hits += 1
                self.graphs[key] = g
                g.replay()
        return self.out[:, :n]

    def _writes(self, l, n, n_cow, n_fill, fill_kv):
        if n_cow:
            pkv_copy_blocks(self.k_pools[l], self.v_pools[l], self.cow[0, :n_cow],
                            self.cow[1, :n_cow], err_flag=self.err, stream=self.stream)
        if n_fill:
            k_src, v_src = fill_kv(l)
            pkv_kv_write(self.k_pools[l], self.v_pools[l], k_src, v_src, self.bt[:n],
                         self.fill[0, :n_fill], self.fill[1, :n_fill], err_flag=self.err,
                         stream=self.stream)

    def _decode(self, l, n, q, k_new, v_new, stream):
        first, count = self.members
        if count:
            pkv_decode_step_prefix(self.out[l, :n], q[l], k_new[l], v_new[l], self.k_pools[l],
                                   self.v_pools[l], self.bt[:n], self.cl[:n], self.scale,
                                   self.max_ctx, self.pre_table, first, count, workspace=self.ws,
                                   err_flag=self.err, stream=stream)
            return
        pkv_decode_step(self.out[l, :n], q[l], k_new[l], v_new[l], self.k_pools[l],
                        self.v_pools[l], self.bt[:n], self.cl[:n], self.scale, self.max_ctx, 0,
                        workspace=self.ws, err_flag=self.err, stream=stream)
