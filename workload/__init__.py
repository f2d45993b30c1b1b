"""Seeded synthetic inputs for paged decode attention.

This module is shared by the tests, the benchmark and the oracle runs. It
only draws random numbers and lays them out in the documented pool layout;
it holds none of the attention arithmetic, and imports neither the oracle
nor the GPU library.

Shapes come from the model shapes the pages size KV caches for:
  * "Scaling LLM serving", "The KV cache": the author's 0.5B model, 24
    layers, 20 query / 4 KV heads, head size 64.
  * "Module 23: Serving", 23.1: LLaMA-2 7B (32 layers, 32 KV heads, d 128,
    L = 4096) and LLaMA-3 8B (32 layers, 8 KV heads, d 128, L = 8192).
  * "Designing an LLM serving system", "What it must do, and at what size":
    80 layers, 8 KV heads, d 128, 8,000-token requests, ~60 of them.
The pages measure on no dataset; context lengths are drawn uniformly where
the workload has a range (a stand-in for "widely varying" request lengths).

Recipe (every draw is seeded):
  * rng(seed, stream) = numpy PCG64 seeded with [seed, stream]; streams:
    0 context lengths, 1 block permutation, 2 pool values (drawn per
    logical block, so neither the physical permutation nor the sharing mode
    changes any sequence's bytes), 3 q / k_new / v_new.
  * context lengths: integer-uniform, inclusive bounds.
  * physical block ids: a random permutation of the pool, handed out in
    (prefix blocks, then sequence-major, logical-block order).
  * values: N(0, 1) in float32, rounded to bf16 with round-to-nearest-even.
    Large pools are drawn on the GPU with a seeded torch.Generator instead;
    the oracle receives the same bytes by copying them back.
  * unused slots (past a sequence's context in its last block) and unused
    blocks hold a bf16 NaN (0x7FC0) in parity runs: they must never reach
    a result.
  * shared prefix (LLaMA-3-8B shape): 2,048 tokens = 128 blocks owned by the
    prefix. Sequence s shares the prefix blocks strictly before the block
    that holds its newest position ctx_s - 1, i.e. min(128, (ctx_s-1)//16)
    blocks; the block it writes is its own (a copy of the prefix block when
    ctx_s <= 2048). With share=False every sequence gets private copies of
    the same bytes.
"""
from dataclasses import dataclass, field, replace
import math

import numpy as np

BLOCK = 16
BF16_NAN = 0x7FC0


@dataclass(frozen=True)
class Shape:
    name: str
    n_layers: int
    n_q: int
    n_kv: int
    d: int
    batch: int
    ctx_lo: int
    ctx_hi: int
    prefix_tokens: int = 0
    fixed_ctx: tuple = ()       # explicit per-sequence lengths (tiny case)
    pool_blocks: int = 0        # 0: exactly the blocks needed

    @property
    def group(self):
        return self.n_q // self.n_kv

    @property
    def scale(self):
        return 1.0 / math.sqrt(self.d)

    @property
    def max_blocks(self):
        hi = max(self.fixed_ctx) if self.fixed_ctx else self.ctx_hi
        return -(-hi // BLOCK)


CONFIGS = {
    1: Shape("tiny: 1 layer, 20q/4kv, d64, ctx 17/40/77/130, 64-block pool",
             1, 20, 4, 64, 4, 17, 130, fixed_ctx=(17, 40, 77, 130), pool_blocks=64),
    2: Shape("0.5B: 24 layers, 20q/4kv, d64, B128, ctx U[512,2048]",
             24, 20, 4, 64, 128, 512, 2048),
    3: Shape("llama2-7b MHA: 32 layers, 32q/32kv, d128, B32, ctx 4096",
             32, 32, 32, 128, 32, 4096, 4096),
    4: Shape("llama3-8b GQA: 32 layers, 32q/8kv, d128, B64, ctx U[1024,8192], 2048-token shared prefix",
             32, 32, 8, 128, 64, 1024, 8192, prefix_tokens=2048),
    5: Shape("80-layer GQA: 80 layers, 64q/8kv, d128, B60, ctx 8000",
             80, 64, 8, 128, 60, 8000, 8000),
}


def tp_shard(shape: Shape, tp: int) -> Shape:
    """One GPU's share of a shape split by KV head over tp GPUs: n_kv / tp
    KV heads and the n_q / tp query heads that read them, everything else
    (layers, batch, contexts) unchanged."""
    if tp < 1 or shape.n_kv % tp:
        raise ValueError(f"{shape.n_kv} KV heads do not split over {tp} GPUs")
    if tp == 1:
        return shape
    return replace(shape, name=f"{shape.name}; one of {tp} shards by KV head",
                   n_q=shape.n_q // tp, n_kv=shape.n_kv // tp)


def rng(seed: int, stream: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64([seed, stream]))


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round to nearest even."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    out = rounded.astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        out[nan] = BF16_NAN
    return out


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def normal_bf16(gen: np.random.Generator, shape) -> np.ndarray:
    return bf16_bits(gen.standard_normal(shape, dtype=np.float32))


@dataclass
class Tables:
    """Block tables and the bookkeeping the generator used to build them.

    Contents are drawn per LOGICAL block (prefix blocks first, then each
    sequence's own blocks in order), so the bytes a sequence sees do not
    depend on the permutation of physical ids or on whether the prefix is
    shared: fresh_phys[i] is the physical block that receives logical block
    i's draw, and copies lists (dst, src) physical pairs whose contents are
    copies (private copies of prefix blocks)."""
    context_lens: np.ndarray          # int32 [B]
    block_tables: np.ndarray          # int32 [B, max_blocks], -1 padded
    num_blocks: int                   # pool size
    fresh_phys: np.ndarray            # int32 [n_logical]
    copies: np.ndarray                # int32 [n_copies, 2] (dst, src)
    used: np.ndarray                  # bool [num_blocks]
    prefix_phys: np.ndarray           # int32 [n_prefix] physical prefix blocks


def context_lengths(shape: Shape, seed: int) -> np.ndarray:
    if shape.fixed_ctx:
        return np.asarray(shape.fixed_ctx, dtype=np.int32)
    g = rng(seed, 0)
    return g.integers(shape.ctx_lo, shape.ctx_hi, size=shape.batch, endpoint=True).astype(np.int32)


def build_tables(shape: Shape, seed: int, context_lens=None, share: bool = True,
                 max_blocks: int = None, spare_blocks: int = 0, permute: bool = True) -> Tables:
    """Assign physical blocks for every sequence; see the module docstring."""
    cl = context_lengths(shape, seed) if context_lens is None else np.asarray(context_lens, np.int32)
    B = len(cl)
    need_mb = int(-(-int(cl.max()) // BLOCK)) if B else 1
    mb = max_blocks or max(shape.max_blocks, need_mb)
    if mb < need_mb:
        raise ValueError("max_blocks too small for the context lengths")
    n_prefix = shape.prefix_tokens // BLOCK
    # plan per sequence: ("prefix", i) shares prefix block i; ("copy", i) is a
    # private copy of prefix block i; ("fresh", -1) holds its own draw
    plan = []
    for s in range(B):
        nb = -(-int(cl[s]) // BLOCK)
        shared = min(n_prefix, (int(cl[s]) - 1) // BLOCK) if (n_prefix and share) else 0
        entries = []
        for b in range(nb):
            if b < shared:
                entries.append(("prefix", b))
            elif b < n_prefix:
                entries.append(("copy", b))
            else:
                entries.append(("fresh", -1))
        plan.append(entries)
    n_phys = n_prefix + sum(1 for e in plan for kind, _ in e if kind != "prefix")
    pool = shape.pool_blocks or (n_phys + spare_blocks)
    if pool < n_phys:
        raise ValueError(f"pool of {pool} blocks < {n_phys} needed")
    perm = (rng(seed, 1).permutation(pool) if permute else np.arange(pool)).astype(np.int32)
    cursor = n_prefix
    prefix_phys = perm[:n_prefix]
    fresh = list(prefix_phys)
    copies = []
    tables = np.full((B, mb), -1, dtype=np.int32)
    for s, entries in enumerate(plan):
        for b, (kind, src) in enumerate(entries):
            if kind == "prefix":
                tables[s, b] = prefix_phys[src]
                continue
            tables[s, b] = perm[cursor]
            cursor += 1
            if kind == "copy":
                copies.append((int(tables[s, b]), int(prefix_phys[src])))
            else:
                fresh.append(int(tables[s, b]))
    used = np.zeros(pool, dtype=bool)
    used[perm[:cursor]] = True
    return Tables(cl, tables, pool, np.asarray(fresh, np.int32),
                  np.asarray(copies, np.int32).reshape(-1, 2), used,
                  prefix_phys.astype(np.int32))


# ---------------------------------------------------------------------------
# host pools (small cases)

def pool_shapes(num_blocks, n_kv, d):
    """Shaped views of the documented layouts: K [nb, h, 16, d], V [nb, h, d, 16]."""
    return (num_blocks, n_kv, BLOCK, d), (num_blocks, n_kv, d, BLOCK)


@dataclass
class HostCase:
    shape: Shape
    tables: Tables
    q: np.ndarray        # uint16 [B, n_q, d]
    k_pool: np.ndarray   # uint16 [nb, n_kv, 16, d]
    v_pool: np.ndarray   # uint16 [nb, n_kv, d, 16]
    k_new: np.ndarray    # uint16 [B, n_kv, d]
    v_new: np.ndarray


def fill_unused_nan(k_pool, v_pool, tables: Tables):
    """NaN in unused blocks and in the slots past each context."""
    k_pool[~tables.used] = BF16_NAN
    v_pool[~tables.used] = BF16_NAN
    for s, ctx in enumerate(tables.context_lens):
        ctx = int(ctx)
        last = tables.block_tables[s, (ctx - 1) // BLOCK]
        fill = ctx - ((ctx - 1) // BLOCK) * BLOCK    # slots in use in the last block
        k_pool[last, :, fill:, :] = BF16_NAN
        v_pool[last, :, :, fill:] = BF16_NAN


def host_case(shape: Shape, seed: int, share: bool = True, context_lens=None,
              nan_fill: bool = True, spare_blocks: int = 0, max_blocks: int = None,
              permute: bool = True) -> HostCase:
    t = build_tables(shape, seed, context_lens=context_lens, share=share,
                     spare_blocks=spare_blocks, max_blocks=max_blocks, permute=permute)
    ks, vs = pool_shapes(t.num_blocks, shape.n_kv, shape.d)
    g = rng(seed, 2)
    n_logical = len(t.fresh_phys)
    k_logical = normal_bf16(g, (n_logical,) + ks[1:])
    v_logical = normal_bf16(g, (n_logical,) + vs[1:])
    k_pool = np.full(ks, BF16_NAN, dtype=np.uint16)
    v_pool = np.full(vs, BF16_NAN, dtype=np.uint16)
    k_pool[t.fresh_phys] = k_logical
    v_pool[t.fresh_phys] = v_logical
    for dst, src in t.copies:
        k_pool[dst] = k_pool[src]
        v_pool[dst] = v_pool[src]
    g3 = rng(seed, 3)
    B = len(t.context_lens)
    q = normal_bf16(g3, (B, shape.n_q, shape.d))
    k_new = normal_bf16(g3, (B, shape.n_kv, shape.d))
    v_new = normal_bf16(g3, (B, shape.n_kv, shape.d))
    if nan_fill:
        fill_unused_nan(k_pool, v_pool, t)
    return HostCase(shape, t, q, k_pool, v_pool, k_new, v_new)


def gather_contiguous(case_k_pool, case_v_pool, tables: Tables, s: int):
    """Contiguous K [n_kv, ctx, d] and V [n_kv, ctx, d] (uint16) of sequence s,
    read back out of the pools through its table (for library-routine pins)."""
    ctx = int(tables.context_lens[s])
    nb = -(-ctx // BLOCK)
    ids = tables.block_tables[s, :nb]
    k = case_k_pool[ids]                         # [nb, h, 16, d]
    v = case_v_pool[ids]                         # [nb, h, d, 16]
    k = np.transpose(k, (1, 0, 2, 3)).reshape(k.shape[1], nb * BLOCK, k.shape[3])[:, :ctx]
    v = np.transpose(v, (1, 0, 3, 2)).reshape(v.shape[1], nb * BLOCK, v.shape[2])[:, :ctx]
    return np.ascontiguousarray(k), np.ascontiguousarray(v)


def scatter_contiguous(k_seq, v_seq, tables: Tables, s: int, k_pool, v_pool):
    """Inverse of gather_contiguous: write contiguous K/V [n_kv, ctx, d] of
    sequence s into the pools through its table."""
    ctx = k_seq.shape[1]
    for t in range(ctx):
        blk = tables.block_tables[s, t // BLOCK]
        k_pool[blk, :, t % BLOCK, :] = k_seq[:, t, :]
        v_pool[blk, :, :, t % BLOCK] = v_seq[:, t, :]


# ---------------------------------------------------------------------------
# device pools (large cases): torch is plumbing here, for memory and RNG only

def device_normal_bf16_(t, seed: int, chunk: int = 1 << 28):
    """Fill a CUDA bf16 tensor in place with N(0,1) draws from a seeded
    torch.Generator (float32 draws rounded to bf16, chunk by chunk)."""
    import torch
    g = torch.Generator(device=t.device)
    g.manual_seed(seed)
    flat = t.view(-1)
    for start in range(0, flat.numel(), chunk):
        n = min(chunk, flat.numel() - start)
        flat[start:start + n].copy_(torch.randn(n, generator=g, device=t.device, dtype=torch.float32))
    return t
