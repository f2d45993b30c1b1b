"""Reference model of the refcounted block allocator -- TEST INFRASTRUCTURE ONLY.

Plain Python, written from the pages' description of paged KV memory:
  * "Scaling LLM serving", "Managing the cache: PagedAttention": fixed-size
    blocks, not contiguous, allocated as the sequence grows; requests can
    share blocks.
  * "Module 23: Serving", 23.4 "Paged Attention": 16-token blocks and a
    per-sequence table from positions to blocks; Exercises: paging wastes
    less than one block per request (only its last block is partly filled).
  * "Designing an LLM serving system", "Paged attention": shared prefix
    blocks are copied on write when sequences diverge; "Continuous
    batching": a finished sequence releases its blocks.

The free-block order is the one the library documents (a LIFO stack; a new
pool hands out 0, 1, 2, ...), so the model and the library can be compared
entry by entry.
"""

BLOCK_TOKENS = 16


class OutOfBlocks(Exception):
    pass


class AllocatorModel:
    def __init__(self, num_blocks: int):
        if num_blocks < 1:
            raise ValueError("num_blocks must be >= 1")
        self.num_blocks = num_blocks
        self.refcount = [0] * num_blocks
        # top of the stack is the end of the list: block 0 comes out first
        self.free = list(range(num_blocks - 1, -1, -1))

    # -- single blocks -------------------------------------------------------
    def alloc(self) -> int:
        if not self.free:
            raise OutOfBlocks()
        b = self.free.pop()
        self.refcount[b] = 1
        return b

    def incref(self, b: int) -> None:
        if not (0 <= b < self.num_blocks) or self.refcount[b] == 0:
            raise ValueError(f"incref of free or invalid block {b}")
        self.refcount[b] += 1

    def decref(self, b: int) -> None:
        if not (0 <= b < self.num_blocks) or self.refcount[b] == 0:
            raise ValueError(f"decref of free or invalid block {b}")
        self.refcount[b] -= 1
        if self.refcount[b] == 0:
            self.free.append(b)

    def num_free(self) -> int:
        return len(self.free)

    # -- sequences -----------------------------------------------------------
    def seq_grow(self, table: list, new_context_len: int, max_blocks: int):
        """Make position new_context_len - 1 writable. Mutates `table` (the
        list of blocks in use). Returns (cow_src, cow_dst) or (-1, -1).
        Raises OutOfBlocks with the blocks allocated so far left in table."""
        if not (1 <= new_context_len <= BLOCK_TOKENS * max_blocks):
            raise ValueError("context length out of range")
        need = -(-new_context_len // BLOCK_TOKENS)  # ceil
        while len(table) < need:
            table.append(self.alloc())
        idx = (new_context_len - 1) // BLOCK_TOKENS
        old = table[idx]
        if self.refcount[old] > 1:
            new = self.alloc()  # raises before anything changes
            self.decref(old)
            table[idx] = new
            return old, new
        return -1, -1

    def seq_fork(self, table: list) -> None:
        for b in table:
            if not (0 <= b < self.num_blocks) or self.refcount[b] == 0:
                raise ValueError("fork of a free or invalid block")
        for b in table:
            self.refcount[b] += 1

    def seq_release(self, table: list) -> None:
        need = {}
        for b in table:
            need[b] = need.get(b, 0) + 1
        for b, n in need.items():
            if not (0 <= b < self.num_blocks) or self.refcount[b] < n:
                raise ValueError("release of a free or invalid block")
        for b in table:
            self.decref(b)
