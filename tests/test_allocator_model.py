"""Pins of the reference allocator model (oracle/allocator_model.py), no GPU.

What the pages fix:
  * "Module 23: Serving", 23.4 and Exercises: blocks of 16 tokens handed out
    only as tokens arrive, so a sequence holds ceil(ctx/16) blocks and wastes
    at most one partly filled block.
  * "Designing an LLM serving system", Paged attention: shared prefix blocks,
    copied on write when a sequence writes into one; Continuous batching: a
    finished sequence releases its blocks, which can then serve anyone.
The 96-block, eight-request figure of 23.4 prints no request lengths, so it
pins nothing here (parity unpinned for that figure).
"""
import random

import pytest

from oracle.allocator_model import AllocatorModel, OutOfBlocks


def test_blocks_follow_context():
    a = AllocatorModel(64)
    table = []
    for ctx in range(1, 16 * 10 + 1):
        src, dst = a.seq_grow(table, ctx, max_blocks=10)
        assert (src, dst) == (-1, -1)
        assert len(table) == -(-ctx // 16)             # ceil: at most one partial block
        assert 16 * len(table) - ctx < 16
    assert a.num_free() == 64 - 10
    assert table == list(range(10))                    # documented order: 0, 1, 2, ...


def test_fork_and_copy_on_write():
    a = AllocatorModel(16)
    parent = []
    for ctx in range(1, 41):                            # 3 blocks, last one partial
        a.seq_grow(parent, ctx, 8)
    child = list(parent)
    a.seq_fork(child)
    assert [a.refcount[b] for b in parent] == [2, 2, 2]
    # the child writes position 40 (inside the shared third block) -> CoW
    src, dst = a.seq_grow(child, 41, 8)
    assert src == parent[2] and dst not in parent
    assert a.refcount[parent[2]] == 1 and a.refcount[dst] == 1
    assert child[:2] == parent[:2] and child[2] == dst
    # the parent writes its own next position: no copy needed any more
    assert a.seq_grow(parent, 41, 8) == (-1, -1)
    # the child crosses into a new block: fresh block, no copy
    for ctx in range(42, 50):
        assert a.seq_grow(child, ctx, 8) == (-1, -1)
    assert len(child) == 4


def test_release_returns_everything():
    a = AllocatorModel(32)
    seqs = []
    for n in (5, 17, 33):
        t = []
        for ctx in range(1, n + 1):
            a.seq_grow(t, ctx, 4)
        seqs.append(t)
    shared = list(seqs[2][:2])
    a.seq_fork(shared)
    for t in seqs:
        a.seq_release(t)
    assert a.num_free() == 32 - 2
    a.seq_release(shared)
    assert a.num_free() == 32 and all(r == 0 for r in a.refcount)


def test_out_of_blocks_is_clean():
    a = AllocatorModel(3)
    t = []
    for ctx in range(1, 49):
        a.seq_grow(t, ctx, 8)
    with pytest.raises(OutOfBlocks):
        a.seq_grow(t, 49, 8)
    assert len(t) == 3 and a.num_free() == 0
    a.seq_release(t[:1])
    a.seq_grow(t, 49, 8)
    assert len(t) == 4


def test_errors():
    a = AllocatorModel(4)
    with pytest.raises(ValueError):
        a.incref(0)                                    # free block
    b = a.alloc()
    a.decref(b)
    with pytest.raises(ValueError):
        a.decref(b)
    with pytest.raises(ValueError):
        a.seq_release([b])
    with pytest.raises(ValueError):
        a.seq_grow([], 0, 4)


def test_random_conservation():
    """Refcounts always equal the number of table references, and the free
    stack holds exactly the blocks nobody references."""
    rnd = random.Random(7)
    a = AllocatorModel(200)
    live = []                                          # (table, ctx)
    for step in range(3000):
        op = rnd.random()
        if op < 0.1 and len(live) < 20:
            live.append(([], 0))
        elif op < 0.15 and live:
            t, c = live[rnd.randrange(len(live))]
            if t:
                child = list(t)
                a.seq_fork(child)
                live.append((child, c))
        elif op < 0.22 and live:
            t, c = live.pop(rnd.randrange(len(live)))
            a.seq_release(t)
        elif live:
            i = rnd.randrange(len(live))
            t, c = live[i]
            if c < 16 * 12:
                try:
                    a.seq_grow(t, c + 1, 12)
                    live[i] = (t, c + 1)
                except OutOfBlocks:
                    pass
        refs = {}
        for t, _ in live:
            for b in t:
                refs[b] = refs.get(b, 0) + 1
        assert all(a.refcount[b] == refs.get(b, 0) for b in range(200))
        assert sorted(a.free) == sorted(b for b in range(200) if b not in refs)
