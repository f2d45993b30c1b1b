"""CPU oracle for paged decode attention -- TEST INFRASTRUCTURE ONLY.

Only the tests, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package. The product path (the
``paged_kv_cache_468_amd`` package and its HIP library) never imports, links or
runs anything here, and nothing here imports the product path.

Contents
  * ``liboracle.so`` (built from ``oracle.c`` by ``oracle/build.py``): append,
    multi-token write, copy-on-write, decode and the multi-token verification
    attention in double precision, the decode's single-precision twin (the
    naive fp32 loop), the KV-size closed form.
  * ``speculative``: the acceptance rule of speculative decoding (accept,
    leftover distribution, replacement draw) in plain Python.
  * ``allocator_model``: a pure-Python reference model of the refcounted
    block allocator; ``batcher_model``: the continuous-batching scheduler.

Inputs are numpy arrays; bf16 tensors travel as their uint16 bit patterns.
Pinning: every function is checked in tests/test_oracle_pins.py against
values printed on the pages (tests/golden/), closed forms, special cases
that reduce to a library routine (torch's scaled_dot_product_attention in
float64) and invariants (permutation of physical blocks, shared = private
copies, grouped heads = repeated heads).
"""
import ctypes
import os

import numpy as np

from .allocator_model import AllocatorModel, OutOfBlocks  # noqa: F401

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")


def _bind(path):
    lib = ctypes.CDLL(path)
    u16p = ctypes.POINTER(ctypes.c_uint16)
    i32p = ctypes.POINTER(ctypes.c_int32)
    f64p = ctypes.POINTER(ctypes.c_double)
    c_int = ctypes.c_int
    lib.oracle_kv_bytes.restype = ctypes.c_uint64
    lib.oracle_kv_bytes.argtypes = [ctypes.c_int64] * 6
    lib.oracle_kv_append.restype = c_int
    lib.oracle_kv_append.argtypes = [u16p, u16p, u16p, u16p, i32p, i32p,
                                     c_int, c_int, c_int, c_int, c_int]
    lib.oracle_kv_write.restype = c_int
    lib.oracle_kv_write.argtypes = [u16p, u16p, u16p, u16p, i32p, i32p, i32p, c_int, c_int,
                                    c_int, c_int, c_int, c_int]
    lib.oracle_copy_blocks.restype = c_int
    lib.oracle_copy_blocks.argtypes = [u16p, u16p, i32p, i32p, c_int, c_int,
                                       c_int, c_int]
    lib.oracle_decode_row.restype = c_int
    lib.oracle_decode_row.argtypes = [f64p, u16p, u16p, u16p, i32p, c_int,
                                      c_int, c_int, c_int, c_int,
                                      ctypes.c_double]
    lib.oracle_decode.restype = c_int
    lib.oracle_decode.argtypes = [f64p, u16p, u16p, u16p, i32p, i32p, c_int,
                                  c_int, c_int, c_int, c_int, c_int,
                                  ctypes.c_double]
    f32p = ctypes.POINTER(ctypes.c_float)
    lib.oracle_decode_row_f32.restype = c_int
    lib.oracle_decode_row_f32.argtypes = [f32p, u16p, u16p, u16p, i32p, c_int,
                                          c_int, c_int, c_int, c_int, ctypes.c_float]
    lib.oracle_decode_f32.restype = c_int
    lib.oracle_decode_f32.argtypes = [f32p, u16p, u16p, u16p, i32p, i32p, c_int,
                                      c_int, c_int, c_int, c_int, c_int, ctypes.c_float]
    lib.oracle_verify.restype = c_int
    lib.oracle_verify.argtypes = [f64p, u16p, u16p, u16p, i32p, i32p, c_int, c_int,
                                  c_int, c_int, c_int, c_int, c_int, ctypes.c_double]
    return lib


def _ptr(a, ctype):
    return a.ctypes.data_as(ctypes.POINTER(ctype))


def _u16(a, name):
    a = np.ascontiguousarray(a)
    if a.dtype != np.uint16:
        raise TypeError(f"{name}: expected uint16 bf16 bit patterns, got {a.dtype}")
    return a


def _i32(a, name):
    a = np.ascontiguousarray(a)
    if a.dtype != np.int32:
        raise TypeError(f"{name}: expected int32, got {a.dtype}")
    return a


class Oracle:
    """numpy front end of one build of oracle.c (the default build, or a
    deliberately mutated copy the pin tests use to show they catch
    mistakes)."""

    def __init__(self, path=_LIB_PATH):
        self.path = path
        self.lib = _bind(path)

    def kv_bytes(self, n_layers, n_kv_heads, d_head, context_len=1, batch=1, bytes_per_value=2):
        """KV-cache bytes: 2 x layers x kv_heads x d_head x L x B x bytes
        ("Module 23: Serving", 23.1, the KV-memory equation)."""
        return int(self.lib.oracle_kv_bytes(n_layers, n_kv_heads, d_head,
                                            context_len, batch, bytes_per_value))

    def kv_append(self, k_pool, v_pool, k_new, v_new, block_tables, context_lens):
        """In-place append into host pools (contiguous uint16 arrays).
        k_new/v_new: uint16 [num_seqs, n_kv, d]. Returns the C status
        (0 ok, -1 some sequence invalid and skipped)."""
        k_new = _u16(k_new, "k_new")
        v_new = _u16(v_new, "v_new")
        bt = _i32(block_tables, "block_tables")
        cl = _i32(context_lens, "context_lens")
        if not (k_pool.flags.c_contiguous and v_pool.flags.c_contiguous):
            raise ValueError("pools must be contiguous (they are written in place)")
        if k_pool.dtype != np.uint16 or v_pool.dtype != np.uint16:
            raise TypeError("pools must be uint16")
        num_seqs, n_kv, d = k_new.shape
        num_blocks = k_pool.size // (n_kv * 16 * d)
        return self.lib.oracle_kv_append(
            _ptr(k_pool, ctypes.c_uint16), _ptr(v_pool, ctypes.c_uint16),
            _ptr(k_new, ctypes.c_uint16), _ptr(v_new, ctypes.c_uint16),
            _ptr(bt, ctypes.c_int32), _ptr(cl, ctypes.c_int32),
            num_seqs, bt.shape[1], num_blocks, n_kv, d)

    def kv_write(self, k_pool, v_pool, k_src, v_src, block_tables, seq_rows, positions):
        """In-place write of token i of k_src/v_src (uint16 [n, n_kv, d]) at
        row seq_rows[i], position positions[i]. Returns the C status (0 ok,
        -1 some token skipped)."""
        k_src = _u16(k_src, "k_src")
        v_src = _u16(v_src, "v_src")
        bt = _i32(block_tables, "block_tables")
        rows = _i32(seq_rows, "seq_rows")
        pos = _i32(positions, "positions")
        if k_pool.dtype != np.uint16 or v_pool.dtype != np.uint16 or not (
                k_pool.flags.c_contiguous and v_pool.flags.c_contiguous):
            raise TypeError("pools must be contiguous uint16 (written in place)")
        n, n_kv, d = k_src.shape
        num_blocks = k_pool.size // (n_kv * 16 * d)
        return self.lib.oracle_kv_write(
            _ptr(k_pool, ctypes.c_uint16), _ptr(v_pool, ctypes.c_uint16),
            _ptr(k_src, ctypes.c_uint16), _ptr(v_src, ctypes.c_uint16),
            _ptr(bt, ctypes.c_int32), _ptr(rows, ctypes.c_int32), _ptr(pos, ctypes.c_int32),
            n, bt.shape[0], bt.shape[1], num_blocks, n_kv, d)

    def copy_blocks(self, k_pool, v_pool, src, dst, n_kv, d):
        """In-place copy-on-write of whole blocks src[p] -> dst[p]."""
        src = _i32(src, "src")
        dst = _i32(dst, "dst")
        num_blocks = k_pool.size // (n_kv * 16 * d)
        return self.lib.oracle_copy_blocks(
            _ptr(k_pool, ctypes.c_uint16), _ptr(v_pool, ctypes.c_uint16),
            _ptr(src, ctypes.c_int32), _ptr(dst, ctypes.c_int32),
            len(src), num_blocks, n_kv, d)

    def decode(self, q, k_pool, v_pool, block_tables, context_lens, n_kv, scale):
        """Decode attention of one layer in double precision.
        q: uint16 [num_seqs, n_q, d]; pools uint16; block_tables int32
        [num_seqs, max_blocks]; context_lens int32 [num_seqs].
        Returns (out float64 [num_seqs, n_q, d], status)."""
        q = _u16(q, "q")
        k_pool = _u16(k_pool, "k_pool")
        v_pool = _u16(v_pool, "v_pool")
        bt = _i32(block_tables, "block_tables")
        cl = _i32(context_lens, "context_lens")
        num_seqs, n_q, d = q.shape
        num_blocks = k_pool.size // (n_kv * 16 * d)
        out = np.empty((num_seqs, n_q, d), dtype=np.float64)
        rc = self.lib.oracle_decode(
            _ptr(out, ctypes.c_double), _ptr(q, ctypes.c_uint16),
            _ptr(k_pool, ctypes.c_uint16), _ptr(v_pool, ctypes.c_uint16),
            _ptr(bt, ctypes.c_int32), _ptr(cl, ctypes.c_int32),
            num_seqs, bt.shape[1], num_blocks, n_q, n_kv, d, float(scale))
        if rc == -2:
            raise MemoryError("oracle_decode: out of host memory")
        if rc == -3:
            raise ValueError("oracle_decode: n_q must be a multiple of n_kv")
        return out, rc

    def decode_f32(self, q, k_pool, v_pool, block_tables, context_lens, n_kv, scale):
        """decode() as the naive loop in single precision (its float64
        twin is decode()). Returns (out float32 [num_seqs, n_q, d], status)."""
        q = _u16(q, "q")
        k_pool = _u16(k_pool, "k_pool")
        v_pool = _u16(v_pool, "v_pool")
        bt = _i32(block_tables, "block_tables")
        cl = _i32(context_lens, "context_lens")
        num_seqs, n_q, d = q.shape
        num_blocks = k_pool.size // (n_kv * 16 * d)
        out = np.empty((num_seqs, n_q, d), dtype=np.float32)
        rc = self.lib.oracle_decode_f32(
            _ptr(out, ctypes.c_float), _ptr(q, ctypes.c_uint16),
            _ptr(k_pool, ctypes.c_uint16), _ptr(v_pool, ctypes.c_uint16),
            _ptr(bt, ctypes.c_int32), _ptr(cl, ctypes.c_int32),
            num_seqs, bt.shape[1], num_blocks, n_q, n_kv, d, float(scale))
        if rc == -2:
            raise MemoryError("oracle_decode_f32: out of host memory")
        if rc == -3:
            raise ValueError("oracle_decode_f32: n_q must be a multiple of n_kv")
        return out, rc

    def verify(self, q, k_pool, v_pool, block_tables, context_lens, n_kv, scale):
        """Verification attention of q_len query tokens per sequence, query
        token i at position ctx - q_len + i seeing tokens [0, ctx - q_len + i].
        q: uint16 [num_seqs, q_len, n_q, d]. Returns (out float64
        [num_seqs, q_len, n_q, d], status)."""
        q = _u16(q, "q")
        k_pool = _u16(k_pool, "k_pool")
        v_pool = _u16(v_pool, "v_pool")
        bt = _i32(block_tables, "block_tables")
        cl = _i32(context_lens, "context_lens")
        num_seqs, q_len, n_q, d = q.shape
        num_blocks = k_pool.size // (n_kv * 16 * d)
        out = np.empty((num_seqs, q_len, n_q, d), dtype=np.float64)
        rc = self.lib.oracle_verify(
            _ptr(out, ctypes.c_double), _ptr(q, ctypes.c_uint16),
            _ptr(k_pool, ctypes.c_uint16), _ptr(v_pool, ctypes.c_uint16),
            _ptr(bt, ctypes.c_int32), _ptr(cl, ctypes.c_int32),
            num_seqs, q_len, bt.shape[1], num_blocks, n_q, n_kv, d, float(scale))
        if rc == -2:
            raise MemoryError("oracle_verify: out of host memory")
        if rc == -3:
            raise ValueError("oracle_verify: bad heads or q_len")
        return out, rc

    def decode_sharded(self, q, k_pool, v_pool, block_tables, context_lens, n_kv, scale,
                       threads):
        """decode() with the sequences split into `threads` contiguous shards,
        each shard one call of the same single-threaded C function on its
        own host thread (ctypes releases the interpreter lock for the call).
        The rows are computed exactly as by decode(): each row's arithmetic
        depends only on its own sequence. Returns (out, worst status)."""
        from concurrent.futures import ThreadPoolExecutor
        q = _u16(q, "q")
        k_pool = _u16(k_pool, "k_pool")
        v_pool = _u16(v_pool, "v_pool")
        bt = _i32(block_tables, "block_tables")
        cl = _i32(context_lens, "context_lens")
        B = q.shape[0]
        threads = max(1, min(int(threads), B))
        cuts = [B * i // threads for i in range(threads + 1)]
        parts = [(a, b) for a, b in zip(cuts[:-1], cuts[1:]) if b > a]
        with ThreadPoolExecutor(max_workers=len(parts)) as pool:
            res = list(pool.map(lambda ab: self.decode(q[ab[0]:ab[1]], k_pool, v_pool,
                                                       bt[ab[0]:ab[1]], cl[ab[0]:ab[1]], n_kv,
                                                       scale), parts))
        out = np.concatenate([r[0] for r in res]) if res else np.empty(q.shape, np.float64)
        return out, min((r[1] for r in res), default=0)

    def decode_row_f32(self, q_row, k_pool, v_pool, table_row, ctx, n_kv, h, scale):
        """decode_row() in single precision (float32 row, status)."""
        q_row = _u16(q_row, "q_row")
        k_pool = _u16(k_pool, "k_pool")
        v_pool = _u16(v_pool, "v_pool")
        table_row = _i32(table_row, "table_row")
        d = q_row.shape[-1]
        num_blocks = k_pool.size // (n_kv * 16 * d)
        out = np.empty(d, dtype=np.float32)
        rc = self.lib.oracle_decode_row_f32(
            _ptr(out, ctypes.c_float), _ptr(q_row, ctypes.c_uint16),
            _ptr(k_pool, ctypes.c_uint16), _ptr(v_pool, ctypes.c_uint16),
            _ptr(table_row, ctypes.c_int32), int(ctx), num_blocks, n_kv, int(h),
            d, float(scale))
        if rc == -2:
            raise MemoryError("oracle_decode_row_f32: out of host memory")
        return out, rc

    def decode_row(self, q_row, k_pool, v_pool, table_row, ctx, n_kv, h, scale):
        """One output row (one sequence, one query head, KV head h)."""
        q_row = _u16(q_row, "q_row")
        k_pool = _u16(k_pool, "k_pool")
        v_pool = _u16(v_pool, "v_pool")
        table_row = _i32(table_row, "table_row")
        d = q_row.shape[-1]
        num_blocks = k_pool.size // (n_kv * 16 * d)
        out = np.empty(d, dtype=np.float64)
        rc = self.lib.oracle_decode_row(
            _ptr(out, ctypes.c_double), _ptr(q_row, ctypes.c_uint16),
            _ptr(k_pool, ctypes.c_uint16), _ptr(v_pool, ctypes.c_uint16),
            _ptr(table_row, ctypes.c_int32), int(ctx), num_blocks, n_kv, int(h),
            d, float(scale))
        if rc == -2:
            raise MemoryError("oracle_decode_row: out of host memory")
        return out, rc


_default = None


def default() -> Oracle:
    """The oracle built from oracle.c (built on first use if missing)."""
    global _default
    if _default is None:
        if not os.path.exists(_LIB_PATH):
            from .build import build
            build()
        _default = Oracle(_LIB_PATH)
    return _default


def kv_bytes(*a, **k):
    return default().kv_bytes(*a, **k)


def kv_append(*a, **k):
    return default().kv_append(*a, **k)


def copy_blocks(*a, **k):
    return default().copy_blocks(*a, **k)


def kv_write(*a, **k):
    return default().kv_write(*a, **k)


def decode(*a, **k):
    return default().decode(*a, **k)


def decode_f32(*a, **k):
    return default().decode_f32(*a, **k)


def decode_sharded(*a, **k):
    return default().decode_sharded(*a, **k)


def host_threads(cap=16):
    """Threads for a sharded oracle run: the CPUs this process may use, at
    most cap."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(cap, n))


def verify(*a, **k):
    return default().verify(*a, **k)


def decode_row(*a, **k):
    return default().decode_row(*a, **k)


def decode_row_f32(*a, **k):
    return default().decode_row_f32(*a, **k)
