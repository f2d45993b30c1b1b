"""Continuous batching on the device: the batcher's plan, carried out.

Each step ("Designing an LLM serving system", "Continuous batching": before
every token step finished sequences release their blocks, waiting requests
are admitted, one decode step runs for the resident batch):
  1. pkv_batcher_step (native, host): releases, growth, preemption,
     admission; the plan;
  2. the plan's tables and context lengths go to the device;
  3. for every layer, in stream order: pkv_copy_blocks for the plan's
     copy-on-write pairs, pkv_kv_write for the prompt tokens admitted this
     step (their keys and values come from the caller: a prefill's output,
     or a preempted request's recomputed tokens), pkv_decode_step for the
     resident rows (the new token's key/value appended inside the
     attention).
Everything runs in the library's kernels and its native batcher; this
module only moves arguments. The keys, values and queries are the
caller's: in a model they come from the layers' projections.
"""
import numpy as np

from . import (Batcher, _torch, pkv_copy_blocks, pkv_decode_step, pkv_decode_workspace_bytes,
               pkv_kv_write)


class ServingLoop:
    """Device state for one batcher: per-layer pools and outputs, device
    tables, one workspace sized for the largest batch and context."""

    def __init__(self, batcher: Batcher, k_pools, v_pools, n_q: int, scale: float,
                 max_batch: int, stream=None):
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
        self.stream = stream
        self.bt = torch.full((max_batch, self.max_blocks), -1, dtype=torch.int32, device=dev)
        self.cl = torch.ones((max_batch,), dtype=torch.int32, device=dev)
        self.out = torch.empty((self.n_layers, max_batch, n_q, self.d), dtype=torch.float32,
                               device=dev)
        self.err = torch.zeros(1, dtype=torch.int32, device=dev)
        ws = pkv_decode_workspace_bytes(max_batch, n_q, self.n_kv, self.d, self.max_ctx, 0)
        self.ws = torch.empty(max(ws, 1), dtype=torch.uint8, device=dev)
        self.plan = None

    def write_prefix(self, k_src, v_src):
        """Keys and values of the shared prefix ([L][prefix_tokens, n_kv, d]
        bf16, per layer) into the prefix's blocks."""
        torch = _torch()
        table, n = self.b.prefix_table()
        if n == 0:
            return
        dev = self.k_pools[0].device
        bt = torch.from_numpy(table.reshape(1, -1)).to(dev)
        n_tok = k_src[0].shape[0]
        rows = torch.zeros(n_tok, dtype=torch.int32, device=dev)
        pos = torch.arange(n_tok, dtype=torch.int32, device=dev)
        for l in range(self.n_layers):
            pkv_kv_write(self.k_pools[l], self.v_pools[l], k_src[l], v_src[l], bt, rows, pos,
                         err_flag=self.err, stream=self.stream)

    def schedule(self):
        """Host half of a step: the batcher's plan, tables uploaded."""
        torch = _torch()
        p = self.b.step()
        self.plan = p
        n = p.num_seqs
        if n:
            self.bt[:n].copy_(torch.from_numpy(p.block_tables))
            self.cl[:n].copy_(torch.from_numpy(p.context_lens))
        return p

    def run(self, fill_kv, q, k_new, v_new):
        """Device half of the scheduled step. fill_kv(l) -> (k_src, v_src)
        bf16 [n_fill, n_kv, d] for the plan's fill tokens of layer l (None
        if none); q [L][n, n_q, d], k_new / v_new [L][n, n_kv, d] for the
        plan's rows. Returns the outputs [L][n, n_q, d] (views)."""
        torch = _torch()
        p = self.plan
        n = p.num_seqs
        dev = self.k_pools[0].device
        src = dst = rows = pos = None
        if len(p.cow_src):
            src = torch.from_numpy(p.cow_src).to(dev)
            dst = torch.from_numpy(p.cow_dst).to(dev)
        if len(p.fill_rows):
            rows = torch.from_numpy(p.fill_rows).to(dev)
            pos = torch.from_numpy(p.fill_positions).to(dev)
        for l in range(self.n_layers):
            if src is not None:
                pkv_copy_blocks(self.k_pools[l], self.v_pools[l], src, dst, err_flag=self.err,
                                stream=self.stream)
            if rows is not None:
                k_src, v_src = fill_kv(l)
                pkv_kv_write(self.k_pools[l], self.v_pools[l], k_src, v_src, self.bt[:n], rows,
                             pos, err_flag=self.err, stream=self.stream)
            if n:
                pkv_decode_step(self.out[l, :n], q[l], k_new[l], v_new[l], self.k_pools[l],
                                self.v_pools[l], self.bt[:n], self.cl[:n], self.scale,
                                self.max_ctx, 0, workspace=self.ws, err_flag=self.err,
                                stream=self.stream)
        return self.out[:, :n]
