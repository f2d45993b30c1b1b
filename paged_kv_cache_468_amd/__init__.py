"""paged_kv_cache_468_amd -- paged decode attention on AMD MI355X (gfx950).

A thin ctypes binding of libpkv.so (the C ABI in include/pkv.h). Every
function here only marshals arguments: checks that tensors have the
documented dtype, shape, device and contiguity, and passes their device
pointers, sizes and torch's current HIP stream to the library. All compute
runs in the library's HIP kernels; there is no fallback. If libpkv.so is
missing the import fails with an error that says how to build it.

Functions keep the C names (pkv_*). Tensors:
  k_pool  torch.bfloat16 [num_blocks, n_kv, 16, head_dim]   (token-major)
  v_pool  torch.bfloat16 [num_blocks, n_kv, head_dim, 16]   (dim-major)
  q       torch.bfloat16 [num_seqs, n_q, head_dim]
  k_new / v_new torch.bfloat16 [num_seqs, n_kv, head_dim]
  out     torch.float32 [num_seqs, n_q, head_dim]
  block_tables torch.int32 [num_seqs, max_blocks]; context_lens torch.int32 [num_seqs]
  err_flag torch.int32 [1] or None
The allocator works on host numpy int32 tables.
"""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpkv.so")

PKV_OK, PKV_EINVAL, PKV_EUNSUPPORTED, PKV_ENOMEM, PKV_EWORKSPACE, PKV_EHIP = 0, -1, -2, -3, -4, -5
PKV_DEVERR_BLOCK_ID, PKV_DEVERR_CONTEXT, PKV_DEVERR_COPY_PAIR, PKV_DEVERR_TOKEN = 1, 2, 4, 8
PKV_DEVERR_PREFIX = 16
BLOCK_TOKENS = 16

# every symbol include/pkv.h declares, with its ctypes signature
_vp, _i32, _i64, _u64, _sz, _f32 = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64,
                                    ctypes.c_uint64, ctypes.c_size_t, ctypes.c_float)
_i32p = ctypes.POINTER(ctypes.c_int32)
SIGNATURES = {
    "pkv_strerror": (ctypes.c_char_p, [ctypes.c_int]),
    "pkv_kv_bytes_per_token": (_u64, [_i32, _i32, _i32, _i32]),
    "pkv_kv_cache_bytes": (_u64, [_i32, _i32, _i32, _i64, _i64, _i32]),
    "pkv_pool_bytes": (_u64, [_i32, _i32, _i32]),
    "pkv_kv_append": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32,
                                     _vp, _vp]),
    "pkv_decode_workspace_bytes": (_sz, [_i32, _i32, _i32, _i32, _i32, _i32]),
    "pkv_paged_attn_decode": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32,
                                             _i32, _i32, _f32, _i32, _i32, _vp, _sz, _vp, _vp]),
    "pkv_paged_attn_partition": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32,
                                                _i32, _i32, _i32, _f32, _i32, _i32, _vp, _sz, _vp,
                                                _vp]),
    "pkv_paged_attn_merge": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32,
                                            _i32, _i32, _f32, _i32, _i32, _vp, _sz, _vp, _vp]),
    "pkv_decode_split_waves": (_i32, [_i32, _i32, _i32, _i32, _i32]),
    "pkv_decode_step": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32,
                                       _i32, _i32, _i32, _f32, _i32, _i32, _vp, _sz, _vp, _vp]),
    "pkv_decode_step_noalloc": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32,
                                               _i32, _i32, _i32, _i32, _f32, _i32, _vp, _vp]),
    "pkv_decode_step_partition": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32,
                                                 _i32, _i32, _i32, _i32, _i32, _f32, _i32, _i32,
                                                 _vp, _sz, _vp, _vp]),
    "pkv_decode_step_partition_valu": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                                      _i32, _i32, _i32, _i32, _i32, _i32, _f32,
                                                      _i32, _i32, _vp, _sz, _vp, _vp]),
    "pkv_decode_prefix_workspace_bytes": (_sz, [_i32, _i32, _i32, _i32, _i32, _i32, _i32]),
    "pkv_decode_step_prefix": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32,
                                              _i32, _i32, _i32, _i32, _f32, _i32, _vp, _i32, _i32,
                                              _i32, _vp, _sz, _vp, _vp]),
    "pkv_verify_workspace_bytes": (_sz, [_i32, _i32, _i32, _i32, _i32, _i32]),
    "pkv_paged_attn_verify": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32,
                                             _i32, _i32, _i32, _f32, _i32, _vp, _sz, _vp, _vp]),
    "pkv_verify_prefix_workspace_bytes": (_sz, [_i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32]),
    "pkv_paged_attn_verify_prefix": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32,
                                                    _i32, _i32, _i32, _i32, _f32, _i32, _vp, _i32,
                                                    _i32, _i32, _vp, _sz, _vp, _vp]),
    "pkv_paged_prefill": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32,
                                         _i32, _i32, _f32, _i32, _vp, _vp]),
    "pkv_spec_accept_workspace_bytes": (_sz, [_i32, _i32]),
    "pkv_spec_accept": (ctypes.c_int, [_vp, _vp, _vp, _vp, _i32, _i32, _i32, _vp, _vp, _vp, _sz,
                                       _vp, _vp]),
    "pkv_copy_blocks": (ctypes.c_int, [_vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _vp, _vp]),
    "pkv_kv_write": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32,
                                    _i32, _vp, _vp]),
    "pkv_batcher_enable_prefix_cache": (ctypes.c_int, [_vp]),
    "pkv_batcher_submit_tokens": (ctypes.c_int, [_vp, _i64, _i32p, _i32, _i32]),
    "pkv_batcher_cached_blocks": (_i32, [_vp]),
    "pkv_prefix_cache_create": (ctypes.c_int, [_vp, ctypes.POINTER(_vp)]),
    "pkv_prefix_cache_destroy": (None, [_vp]),
    "pkv_prefix_match": (_i32, [_vp, _i32p, _i32, _i32p, _i32]),
    "pkv_prefix_insert": (_i32, [_vp, _i32p, _i32, _i32p, _i32]),
    "pkv_prefix_evict": (_i32, [_vp, _i32]),
    "pkv_prefix_cached_blocks": (_i32, [_vp]),
    "pkv_allocator_create": (ctypes.c_int, [_i32, ctypes.POINTER(_vp)]),
    "pkv_allocator_destroy": (None, [_vp]),
    "pkv_block_alloc": (ctypes.c_int, [_vp, _i32p]),
    "pkv_block_incref": (ctypes.c_int, [_vp, _i32]),
    "pkv_block_decref": (ctypes.c_int, [_vp, _i32]),
    "pkv_block_refcount": (_i32, [_vp, _i32]),
    "pkv_num_free": (_i32, [_vp]),
    "pkv_num_blocks": (_i32, [_vp]),
    "pkv_seq_grow": (ctypes.c_int, [_vp, _i32p, _i32p, _i32, _i32, _i32p, _i32p]),
    "pkv_seq_fork": (ctypes.c_int, [_vp, _i32p, _i32]),
    "pkv_seq_release": (ctypes.c_int, [_vp, _i32p, _i32]),
    "pkv_batcher_create": (ctypes.c_int, [_i32, _i32, _i32, _i32, ctypes.POINTER(_vp)]),
    "pkv_batcher_destroy": (None, [_vp]),
    "pkv_batcher_prefix_table": (_i32, [_vp, ctypes.POINTER(_i32p)]),
    "pkv_batcher_submit": (ctypes.c_int, [_vp, _i64, _i32, _i32, _i32]),
    "pkv_batcher_step": (ctypes.c_int, [_vp, ctypes.c_void_p]),
}


class StepPlan(ctypes.Structure):
    """pkv_step_plan (include/pkv.h)."""
    _fields_ = [
        ("num_seqs", ctypes.c_int32), ("max_blocks_per_seq", ctypes.c_int32),
        ("block_tables", ctypes.POINTER(ctypes.c_int32)),
        ("context_lens", ctypes.POINTER(ctypes.c_int32)),
        ("request_ids", ctypes.POINTER(ctypes.c_int64)),
        ("n_cow", ctypes.c_int32), ("cow_src", ctypes.POINTER(ctypes.c_int32)),
        ("cow_dst", ctypes.POINTER(ctypes.c_int32)),
        ("n_fill", ctypes.c_int32), ("fill_rows", ctypes.POINTER(ctypes.c_int32)),
        ("fill_positions", ctypes.POINTER(ctypes.c_int32)),
        ("n_finished", ctypes.c_int32), ("finished_ids", ctypes.POINTER(ctypes.c_int64)),
        ("n_preempted", ctypes.c_int32), ("preempted_ids", ctypes.POINTER(ctypes.c_int64)),
        ("num_free_blocks", ctypes.c_int32), ("num_waiting", ctypes.c_int32),
        ("n_cached_tokens", ctypes.c_int32),
    ]


class PkvError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        super().__init__(f"{where}: {strerror(status)} ({status})")


def _load():
    # torch first: libpkv.so then binds to the HIP runtime torch already
    # loaded (same soname), so torch's device pointers and stream handles are
    # valid in the library. Loaded the other way round, the process would
    # hold two HIP runtimes and torch's streams would be foreign handles.
    import torch  # noqa: F401
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with `python -c 'import __graft_entry__ as g; g.build()'` "
            "or `python paged_kv_cache_468_amd/build.py` (hipcc, gfx950). There is no fallback.")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


lib = _load()


def strerror(status: int) -> str:
    return lib.pkv_strerror(int(status)).decode()


def _check(status, where):
    if status != PKV_OK:
        raise PkvError(status, where)


# ---------------------------------------------------------------------------
# tensor marshalling

def _torch():
    import torch
    return torch


def _dev(t, name, dtype, ndim=None):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name}: expected a torch tensor")
    if not t.is_cuda:
        raise ValueError(f"{name}: must be on the GPU")
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name}: expected {ndim} dims, got shape {tuple(t.shape)}")
    return ctypes.c_void_p(t.data_ptr())


def _flag(err_flag):
    if err_flag is None:
        return None
    return _dev(err_flag, "err_flag", _torch().int32)


def _stream(stream):
    torch = _torch()
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _pool_dims(k_pool, v_pool):
    torch = _torch()
    _dev(k_pool, "k_pool", torch.bfloat16, 4)
    _dev(v_pool, "v_pool", torch.bfloat16, 4)
    nb, n_kv, bt, d = k_pool.shape
    if bt != BLOCK_TOKENS or tuple(v_pool.shape) != (nb, n_kv, d, BLOCK_TOKENS):
        raise ValueError(f"pools: expected K [nb, n_kv, 16, d] and V [nb, n_kv, d, 16], got "
                         f"{tuple(k_pool.shape)} and {tuple(v_pool.shape)}")
    return nb, n_kv, d


# ---------------------------------------------------------------------------
# C ABI, same names

def pkv_kv_bytes_per_token(n_layers, n_kv_heads, head_dim, bytes_per_value=2):
    return int(lib.pkv_kv_bytes_per_token(n_layers, n_kv_heads, head_dim, bytes_per_value))


def pkv_kv_cache_bytes(n_layers, n_kv_heads, head_dim, context_len, batch, bytes_per_value=2):
    return int(lib.pkv_kv_cache_bytes(n_layers, n_kv_heads, head_dim, context_len, batch,
                                      bytes_per_value))


def pkv_pool_bytes(num_blocks, n_kv_heads, head_dim):
    return int(lib.pkv_pool_bytes(num_blocks, n_kv_heads, head_dim))


def pkv_kv_append(k_pool, v_pool, k_new, v_new, block_tables, context_lens, err_flag=None,
                  stream=None):
    torch = _torch()
    nb, n_kv, d = _pool_dims(k_pool, v_pool)
    _dev(k_new, "k_new", torch.bfloat16, 3)
    _dev(v_new, "v_new", torch.bfloat16, 3)
    num_seqs = k_new.shape[0]
    if tuple(k_new.shape) != (num_seqs, n_kv, d) or tuple(v_new.shape) != (num_seqs, n_kv, d):
        raise ValueError("k_new / v_new: expected [num_seqs, n_kv, head_dim]")
    bt = _dev(block_tables, "block_tables", torch.int32, 2)
    cl = _dev(context_lens, "context_lens", torch.int32, 1)
    if block_tables.shape[0] != num_seqs or context_lens.shape[0] != num_seqs:
        raise ValueError("block_tables / context_lens: first dim must be num_seqs")
    _check(lib.pkv_kv_append(_dev(k_pool, "k_pool", torch.bfloat16),
                             _dev(v_pool, "v_pool", torch.bfloat16),
                             _dev(k_new, "k_new", torch.bfloat16),
                             _dev(v_new, "v_new", torch.bfloat16), bt, cl, num_seqs,
                             block_tables.shape[1], nb, n_kv, d, _flag(err_flag),
                             _stream(stream)), "pkv_kv_append")


def pkv_decode_workspace_bytes(num_seqs, n_q_heads, n_kv_heads, head_dim, max_context_len,
                               partition_tokens=0):
    return int(lib.pkv_decode_workspace_bytes(num_seqs, n_q_heads, n_kv_heads, head_dim,
                                              max_context_len, partition_tokens))


def pkv_decode_split_waves(num_seqs, n_q_heads, n_kv_heads, head_dim, max_context_len):
    """Wavefronts of the balanced split (partition_tokens == 0) on the
    current device; negative PKV_E* codes pass through."""
    return int(lib.pkv_decode_split_waves(num_seqs, n_q_heads, n_kv_heads, head_dim,
                                          max_context_len))


_NO_WORKSPACE = False   # workspace argument of a call that takes none (nothing is allocated)


def _decode_args(out, q, k_pool, v_pool, block_tables, context_lens, scale, max_context_len,
                 partition_tokens, workspace, err_flag, stream):
    torch = _torch()
    nb, n_kv, d = _pool_dims(k_pool, v_pool)
    _dev(q, "q", torch.bfloat16, 3)
    num_seqs, n_q, dq = q.shape
    if dq != d:
        raise ValueError("q: head_dim differs from the pools'")
    _dev(out, "out", torch.float32, 3)
    if tuple(out.shape) != (num_seqs, n_q, d):
        raise ValueError("out: expected [num_seqs, n_q, head_dim] float32")
    bt = _dev(block_tables, "block_tables", torch.int32, 2)
    cl = _dev(context_lens, "context_lens", torch.int32, 1)
    if block_tables.shape[0] != num_seqs or context_lens.shape[0] != num_seqs:
        raise ValueError("block_tables / context_lens: first dim must be num_seqs")
    need = pkv_decode_workspace_bytes(num_seqs, n_q, n_kv, d, max_context_len, partition_tokens)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_ptr, ws_bytes = None, 0
    if workspace is not None and workspace is not _NO_WORKSPACE:
        ws_ptr = _dev(workspace, "workspace", torch.uint8)
        ws_bytes = workspace.numel()
    return (_dev(out, "out", torch.float32), _dev(q, "q", torch.bfloat16),
            _dev(k_pool, "k_pool", torch.bfloat16), _dev(v_pool, "v_pool", torch.bfloat16), bt, cl,
            num_seqs, block_tables.shape[1], nb, n_q, n_kv, d, float(scale), int(max_context_len),
            int(partition_tokens), ws_ptr, ws_bytes, _flag(err_flag), _stream(stream)), workspace


def pkv_paged_attn_decode(out, q, k_pool, v_pool, block_tables, context_lens, scale,
                          max_context_len, partition_tokens=0, workspace=None, err_flag=None,
                          stream=None):
    """out <- attention of q over the paged cache. workspace: a torch uint8
    CUDA tensor of at least pkv_decode_workspace_bytes(...) bytes, or None
    to have one allocated here (by torch's caching allocator)."""
    args, _ = _decode_args(out, q, k_pool, v_pool, block_tables, context_lens, scale,
                           max_context_len, partition_tokens, workspace, err_flag, stream)
    _check(lib.pkv_paged_attn_decode(*args), "pkv_paged_attn_decode")


def _step_args(out, q, k_new, v_new, k_pool, v_pool, block_tables, context_lens, scale,
               max_context_len, partition_tokens, workspace, err_flag, stream):
    torch = _torch()
    args, ws = _decode_args(out, q, k_pool, v_pool, block_tables, context_lens, scale,
                            max_context_len, partition_tokens, workspace, err_flag, stream)
    _, n_kv, d = _pool_dims(k_pool, v_pool)
    for name, t in (("k_new", k_new), ("v_new", v_new)):
        _dev(t, name, torch.bfloat16, 3)
        if tuple(t.shape) != (q.shape[0], n_kv, d):
            raise ValueError(f"{name}: expected [num_seqs, n_kv, head_dim]")
    # C order: out, q, k_new, v_new, k_pool, v_pool, then as the decode
    step = (args[0], args[1], _dev(k_new, "k_new", torch.bfloat16),
            _dev(v_new, "v_new", torch.bfloat16), args[2], args[3]) + args[4:]
    return step, ws


def pkv_decode_step(out, q, k_new, v_new, k_pool, v_pool, block_tables, context_lens, scale,
                    max_context_len, partition_tokens=0, workspace=None, err_flag=None,
                    stream=None):
    """kv_append of (k_new, v_new) and the decode attention of one layer;
    with the balanced split the append runs inside the partition kernel.
    workspace as for pkv_paged_attn_decode."""
    args, _ = _step_args(out, q, k_new, v_new, k_pool, v_pool, block_tables, context_lens, scale,
                         max_context_len, partition_tokens, workspace, err_flag, stream)
    _check(lib.pkv_decode_step(*args), "pkv_decode_step")


NOALLOC_SCRATCH_BYTES = 64 << 20   # PKV_NOALLOC_SCRATCH_BYTES


def pkv_decode_step_noalloc(out, q, k_new, v_new, k_pool, v_pool, block_tables, context_lens,
                            scale, max_context_len, err_flag=None, stream=None):
    """pkv_decode_step (balanced split) with no workspace: the library's own
    device array of NOALLOC_SCRATCH_BYTES per GPU serves as one; nothing is
    allocated, here or in the library. Overlapping calls on one GPU race."""
    args, _ = _step_args(out, q, k_new, v_new, k_pool, v_pool, block_tables, context_lens, scale,
                         max_context_len, 0, _NO_WORKSPACE, err_flag, stream)
    # C order: the step's arguments without partition_tokens, workspace and its size
    _check(lib.pkv_decode_step_noalloc(*(args[:16] + args[19:])), "pkv_decode_step_noalloc")


def pkv_decode_step_partition_valu(out, q, k_new, v_new, k_pool, v_pool, block_tables,
                                   context_lens, scale, max_context_len, workspace=None,
                                   err_flag=None, stream=None):
    """pkv_decode_step_partition (balanced split) with the scores and P.V
    on the vector ALUs instead of the matrix cores; at most 8 query heads
    per KV head. pkv_paged_attn_merge with the same arguments and workspace
    finishes the step. Returns the workspace used."""
    args, ws = _step_args(out, q, k_new, v_new, k_pool, v_pool, block_tables, context_lens, scale,
                          max_context_len, 0, workspace, err_flag, stream)
    _check(lib.pkv_decode_step_partition_valu(*args), "pkv_decode_step_partition_valu")
    return ws


def pkv_decode_prefix_workspace_bytes(num_seqs, n_q_heads, n_kv_heads, head_dim, max_context_len,
                                      prefix_blocks, prefix_num_seqs):
    return int(lib.pkv_decode_prefix_workspace_bytes(num_seqs, n_q_heads, n_kv_heads, head_dim,
                                                     max_context_len, prefix_blocks,
                                                     prefix_num_seqs))


def _prefix_step_args(out, q, k_new, v_new, k_pool, v_pool, block_tables, context_lens, scale,
                      max_context_len, prefix_table, prefix_first_seq, prefix_num_seqs, workspace,
                      err_flag, stream):
    torch = _torch()
    pt = _dev(prefix_table, "prefix_table", torch.int32, 1)
    n_pre = prefix_table.shape[0]
    _, n_kv, d = _pool_dims(k_pool, v_pool)
    _dev(q, "q", torch.bfloat16, 3)
    if workspace is None:
        need = pkv_decode_prefix_workspace_bytes(q.shape[0], q.shape[1], n_kv, d, max_context_len,
                                                 n_pre, prefix_num_seqs)
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    args, ws = _step_args(out, q, k_new, v_new, k_pool, v_pool, block_tables, context_lens, scale,
                          max_context_len, 0, workspace, err_flag, stream)
    # C order: the step's arguments up to max_context_len, then the prefix
    # (table, blocks, first member, member count) in place of partition_tokens
    return args[:16] + (pt, n_pre, int(prefix_first_seq), int(prefix_num_seqs)) + args[17:], ws


def pkv_decode_step_prefix(out, q, k_new, v_new, k_pool, v_pool, block_tables, context_lens, scale,
                           max_context_len, prefix_table, prefix_first_seq, prefix_num_seqs,
                           workspace=None, err_flag=None, stream=None):
    """pkv_decode_step for a batch whose sequences prefix_first_seq ..
    prefix_first_seq + prefix_num_seqs - 1 share the blocks prefix_table
    (device int32 [prefix_blocks]) as the start of their tables: the
    prefix's tiles are read once for all members. workspace: at least
    pkv_decode_prefix_workspace_bytes(...) bytes, or None."""
    args, _ = _prefix_step_args(out, q, k_new, v_new, k_pool, v_pool, block_tables, context_lens,
                                scale, max_context_len, prefix_table, prefix_first_seq,
                                prefix_num_seqs, workspace, err_flag, stream)
    _check(lib.pkv_decode_step_prefix(*args), "pkv_decode_step_prefix")


def pkv_decode_step_partition(out, q, k_new, v_new, k_pool, v_pool, block_tables, context_lens,
                              scale, max_context_len, partition_tokens=0, workspace=None,
                              err_flag=None, stream=None):
    """The append and the partition kernel of pkv_decode_step; returns the
    workspace used (pass it to pkv_paged_attn_merge to finish the step)."""
    args, ws = _step_args(out, q, k_new, v_new, k_pool, v_pool, block_tables, context_lens, scale,
                          max_context_len, partition_tokens, workspace, err_flag, stream)
    _check(lib.pkv_decode_step_partition(*args), "pkv_decode_step_partition")
    return ws


def pkv_paged_attn_partition(out, q, k_pool, v_pool, block_tables, context_lens, scale,
                             max_context_len, partition_tokens=0, workspace=None, err_flag=None,
                             stream=None):
    """First kernel of the decode; returns the workspace it used (pass the
    same one to pkv_paged_attn_merge)."""
    args, ws = _decode_args(out, q, k_pool, v_pool, block_tables, context_lens, scale,
                            max_context_len, partition_tokens, workspace, err_flag, stream)
    _check(lib.pkv_paged_attn_partition(*args), "pkv_paged_attn_partition")
    return ws


def pkv_paged_attn_merge(out, q, k_pool, v_pool, block_tables, context_lens, scale,
                         max_context_len, partition_tokens=0, workspace=None, err_flag=None,
                         stream=None):
    args, _ = _decode_args(out, q, k_pool, v_pool, block_tables, context_lens, scale,
                           max_context_len, partition_tokens, workspace, err_flag, stream)
    _check(lib.pkv_paged_attn_merge(*args), "pkv_paged_attn_merge")


def pkv_verify_workspace_bytes(num_seqs, q_len, n_q_heads, n_kv_heads, head_dim, max_context_len):
    return int(lib.pkv_verify_workspace_bytes(num_seqs, q_len, n_q_heads, n_kv_heads, head_dim,
                                              max_context_len))


def pkv_paged_attn_verify(out, q, k_pool, v_pool, block_tables, context_lens, scale,
                          max_context_len, workspace=None, err_flag=None, stream=None):
    """Verification pass: q bf16 [num_seqs, q_len, n_q, d] (the last q_len
    cached tokens of each sequence, already written), out fp32 of the same
    shape; query token i sees positions [0, ctx - q_len + i]. workspace: a
    torch uint8 CUDA tensor of at least pkv_verify_workspace_bytes(...)
    bytes, or None to have one allocated here. Returns the workspace."""
    torch = _torch()
    nb, n_kv, d = _pool_dims(k_pool, v_pool)
    _dev(q, "q", torch.bfloat16, 4)
    _dev(out, "out", torch.float32, 4)
    B, q_len, n_q, dq = q.shape
    if dq != d or tuple(out.shape) != tuple(q.shape):
        raise ValueError("q / out: expected [num_seqs, q_len, n_q, head_dim], the same shape")
    bt = _dev(block_tables, "block_tables", torch.int32, 2)
    cl = _dev(context_lens, "context_lens", torch.int32, 1)
    if block_tables.shape[0] != B or context_lens.shape[0] != B:
        raise ValueError("block_tables / context_lens: one row per sequence")
    need = pkv_verify_workspace_bytes(B, q_len, n_q, n_kv, d, max_context_len) if B else 0
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    ws = _dev(workspace, "workspace", torch.uint8, 1)
    _check(lib.pkv_paged_attn_verify(_dev(out, "out", torch.float32), _dev(q, "q", torch.bfloat16),
                                     _dev(k_pool, "k_pool", torch.bfloat16),
                                     _dev(v_pool, "v_pool", torch.bfloat16), bt, cl, B, q_len,
                                     block_tables.shape[1], nb, n_q, n_kv, d, float(scale),
                                     int(max_context_len), ws, workspace.numel(), _flag(err_flag),
                                     _stream(stream)), "pkv_paged_attn_verify")
    return workspace


def pkv_verify_prefix_workspace_bytes(num_seqs, q_len, n_q_heads, n_kv_heads, head_dim,
                                      max_context_len, prefix_blocks, prefix_num_seqs):
    return int(lib.pkv_verify_prefix_workspace_bytes(num_seqs, q_len, n_q_heads, n_kv_heads,
                                                     head_dim, max_context_len, prefix_blocks,
                                                     prefix_num_seqs))


def pkv_paged_attn_verify_prefix(out, q, k_pool, v_pool, block_tables, context_lens, scale,
                                 max_context_len, prefix_table, prefix_first_seq,
                                 prefix_num_seqs, workspace=None, err_flag=None, stream=None):
    """The verification pass with a shared prefix read once for the member
    sequences prefix_first_seq .. + prefix_num_seqs - 1: prefix_table a
    torch int32 CUDA tensor of the prefix's block ids (its length is the
    prefix's block count). Other arguments as for pkv_paged_attn_verify;
    workspace of at least pkv_verify_prefix_workspace_bytes(...) bytes, or
    None to have one allocated here. Returns the workspace."""
    torch = _torch()
    nb, n_kv, d = _pool_dims(k_pool, v_pool)
    _dev(q, "q", torch.bfloat16, 4)
    _dev(out, "out", torch.float32, 4)
    B, q_len, n_q, dq = q.shape
    if dq != d or tuple(out.shape) != tuple(q.shape):
        raise ValueError("q / out: expected [num_seqs, q_len, n_q, head_dim], the same shape")
    bt = _dev(block_tables, "block_tables", torch.int32, 2)
    cl = _dev(context_lens, "context_lens", torch.int32, 1)
    if block_tables.shape[0] != B or context_lens.shape[0] != B:
        raise ValueError("block_tables / context_lens: one row per sequence")
    pt = _dev(prefix_table, "prefix_table", torch.int32, 1)
    n_pre = prefix_table.shape[0]
    need = pkv_verify_prefix_workspace_bytes(B, q_len, n_q, n_kv, d, max_context_len, n_pre,
                                             prefix_num_seqs) if B else 0
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    ws = _dev(workspace, "workspace", torch.uint8, 1)
    _check(lib.pkv_paged_attn_verify_prefix(
        _dev(out, "out", torch.float32), _dev(q, "q", torch.bfloat16),
        _dev(k_pool, "k_pool", torch.bfloat16), _dev(v_pool, "v_pool", torch.bfloat16), bt, cl, B,
        q_len, block_tables.shape[1], nb, n_q, n_kv, d, float(scale), int(max_context_len), pt,
        n_pre, int(prefix_first_seq), int(prefix_num_seqs), ws, workspace.numel(),
        _flag(err_flag), _stream(stream)), "pkv_paged_attn_verify_prefix")
    return workspace


def pkv_paged_prefill(out, q, k_pool, v_pool, block_tables, context_lens, scale, max_context_len,
                      err_flag=None, stream=None):
    """Chunked prefill: q bf16 [num_seqs, chunk_len, n_q, d] (the last
    chunk_len cached tokens of each sequence, already written), out fp32 of
    the same shape; chunk token i sees positions [0, ctx - chunk_len + i]."""
    torch = _torch()
    nb, n_kv, d = _pool_dims(k_pool, v_pool)
    _dev(q, "q", torch.bfloat16, 4)
    _dev(out, "out", torch.float32, 4)
    B, C, n_q, dq = q.shape
    if dq != d or tuple(out.shape) != tuple(q.shape):
        raise ValueError("q / out: expected [num_seqs, chunk_len, n_q, head_dim], the same shape")
    bt = _dev(block_tables, "block_tables", torch.int32, 2)
    cl = _dev(context_lens, "context_lens", torch.int32, 1)
    if block_tables.shape[0] != B or context_lens.shape[0] != B:
        raise ValueError("block_tables / context_lens: one row per sequence")
    _check(lib.pkv_paged_prefill(_dev(out, "out", torch.float32), _dev(q, "q", torch.bfloat16),
                                 _dev(k_pool, "k_pool", torch.bfloat16),
                                 _dev(v_pool, "v_pool", torch.bfloat16), bt, cl, B, C,
                                 block_tables.shape[1], nb, n_q, n_kv, d, float(scale),
                                 int(max_context_len), _flag(err_flag), _stream(stream)),
           "pkv_paged_prefill")


def pkv_spec_accept_workspace_bytes(num_seqs, vocab):
    return int(lib.pkv_spec_accept_workspace_bytes(num_seqs, vocab))


def pkv_spec_accept(p_target, q_draft, draft_tokens, uniforms, n_accepted, next_token,
                    workspace=None, err_flag=None, stream=None):
    """The acceptance rule: p_target fp32 [B, gamma+1, V], q_draft fp32
    [B, gamma, V], draft_tokens int32 [B, gamma], uniforms fp32 [B, gamma+1];
    writes n_accepted and next_token (int32 [B]). workspace: a torch uint8
    CUDA tensor of at least pkv_spec_accept_workspace_bytes(B, V) bytes, or
    None to have one allocated here. Returns the workspace."""
    torch = _torch()
    _dev(p_target, "p_target", torch.float32, 3)
    B, g1, V = p_target.shape
    gamma = g1 - 1
    if tuple(uniforms.shape) != (B, g1):
        raise ValueError("uniforms: expected [num_seqs, gamma + 1]")
    if gamma > 0:
        _dev(q_draft, "q_draft", torch.float32, 3)
        _dev(draft_tokens, "draft_tokens", torch.int32, 2)
        if tuple(q_draft.shape) != (B, gamma, V) or tuple(draft_tokens.shape) != (B, gamma):
            raise ValueError("q_draft / draft_tokens: expected [B, gamma, V] / [B, gamma]")
    for name, t in (("n_accepted", n_accepted), ("next_token", next_token)):
        _dev(t, name, torch.int32, 1)
        if t.shape[0] != B:
            raise ValueError(f"{name}: one entry per sequence")
    if workspace is None:
        workspace = torch.empty(max(pkv_spec_accept_workspace_bytes(B, V), 1), dtype=torch.uint8,
                                device=p_target.device)
    ws = _dev(workspace, "workspace", torch.uint8, 1)
    _check(lib.pkv_spec_accept(_dev(p_target, "p_target", torch.float32),
                               _dev(q_draft, "q_draft", torch.float32) if gamma > 0 else None,
                               _dev(draft_tokens, "draft_tokens", torch.int32) if gamma > 0 else None,
                               _dev(uniforms, "uniforms", torch.float32), B, gamma, V,
                               _dev(n_accepted, "n_accepted", torch.int32),
                               _dev(next_token, "next_token", torch.int32), ws, workspace.numel(),
                               _flag(err_flag), _stream(stream)), "pkv_spec_accept")
    return workspace


def pkv_kv_write(k_pool, v_pool, k_src, v_src, block_tables, seq_rows, positions, err_flag=None,
                 stream=None):
    """Token t of k_src / v_src ([n, n_kv, d] bf16) into row seq_rows[t] at
    position positions[t] (both int32 [n] on the device)."""
    torch = _torch()
    nb, n_kv, d = _pool_dims(k_pool, v_pool)
    _dev(k_src, "k_src", torch.bfloat16, 3)
    _dev(v_src, "v_src", torch.bfloat16, 3)
    n = k_src.shape[0]
    if tuple(k_src.shape) != (n, n_kv, d) or tuple(v_src.shape) != (n, n_kv, d):
        raise ValueError("k_src / v_src: expected [n_tokens, n_kv, head_dim]")
    bt = _dev(block_tables, "block_tables", torch.int32, 2)
    rows = _dev(seq_rows, "seq_rows", torch.int32, 1)
    pos = _dev(positions, "positions", torch.int32, 1)
    if seq_rows.shape[0] != n or positions.shape[0] != n:
        raise ValueError("seq_rows / positions: one entry per token")
    _check(lib.pkv_kv_write(_dev(k_pool, "k_pool", torch.bfloat16),
                            _dev(v_pool, "v_pool", torch.bfloat16),
                            _dev(k_src, "k_src", torch.bfloat16), _dev(v_src, "v_src", torch.bfloat16),
                            bt, rows, pos, n, block_tables.shape[0], block_tables.shape[1], nb, n_kv,
                            d, _flag(err_flag), _stream(stream)), "pkv_kv_write")


def pkv_copy_blocks(k_pool, v_pool, src, dst, err_flag=None, stream=None):
    torch = _torch()
    nb, n_kv, d = _pool_dims(k_pool, v_pool)
    s = _dev(src, "src", torch.int32, 1)
    t = _dev(dst, "dst", torch.int32, 1)
    if src.shape != dst.shape:
        raise ValueError("src / dst: same length required")
    _check(lib.pkv_copy_blocks(_dev(k_pool, "k_pool", torch.bfloat16),
                               _dev(v_pool, "v_pool", torch.bfloat16), s, t, src.shape[0], nb,
                               n_kv, d, _flag(err_flag), _stream(stream)), "pkv_copy_blocks")


# ---------------------------------------------------------------------------
# host allocator

def _i32_host(a, name):
    if not isinstance(a, np.ndarray) or a.dtype != np.int32 or not a.flags.c_contiguous:
        raise TypeError(f"{name}: expected a contiguous numpy int32 array")
    return a.ctypes.data_as(_i32p)


class Allocator:
    """Owner of a pkv_allocator handle (host memory, one thread)."""

    def __init__(self, num_blocks: int):
        h = ctypes.c_void_p()
        _check(lib.pkv_allocator_create(num_blocks, ctypes.byref(h)), "pkv_allocator_create")
        self._h = h

    def close(self):
        if self._h:
            lib.pkv_allocator_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def pkv_block_alloc(self) -> int:
        out = ctypes.c_int32()
        _check(lib.pkv_block_alloc(self._h, ctypes.byref(out)), "pkv_block_alloc")
        return out.value

    def pkv_block_incref(self, b):
        _check(lib.pkv_block_incref(self._h, int(b)), "pkv_block_incref")

    def pkv_block_decref(self, b):
        _check(lib.pkv_block_decref(self._h, int(b)), "pkv_block_decref")

    def pkv_block_refcount(self, b) -> int:
        return int(lib.pkv_block_refcount(self._h, int(b)))

    def pkv_num_free(self) -> int:
        return int(lib.pkv_num_free(self._h))

    def pkv_num_blocks(self) -> int:
        return int(lib.pkv_num_blocks(self._h))

    def pkv_seq_grow(self, table: np.ndarray, n_blocks: int, new_context_len: int):
        """Returns (status, n_blocks, cow_src, cow_dst); status is PKV_OK or
        PKV_ENOMEM (other codes raise)."""
        nb = ctypes.c_int32(n_blocks)
        src, dst = ctypes.c_int32(), ctypes.c_int32()
        st = lib.pkv_seq_grow(self._h, _i32_host(table, "table"), ctypes.byref(nb),
                              table.shape[0], int(new_context_len), ctypes.byref(src),
                              ctypes.byref(dst))
        if st not in (PKV_OK, PKV_ENOMEM):
            raise PkvError(st, "pkv_seq_grow")
        return st, nb.value, src.value, dst.value

    def pkv_seq_fork(self, table: np.ndarray, n_blocks: int):
        _check(lib.pkv_seq_fork(self._h, _i32_host(table, "table"), int(n_blocks)), "pkv_seq_fork")

    def pkv_seq_release(self, table: np.ndarray, n_blocks: int):
        _check(lib.pkv_seq_release(self._h, _i32_host(table, "table"), int(n_blocks)),
               "pkv_seq_release")


# ---------------------------------------------------------------------------
# pre-marshalled calls for loops that issue the same call many times

class PreparedCall:
    """One C-ABI call whose arguments were checked and marshalled once.

    Built by prepare_*; calling it re-issues the C function with the same
    pointers (the tensors must stay alive and keep their storage), which
    removes the per-call Python checks from a step loop. Raises PkvError on
    a non-OK status like the plain wrappers."""

    __slots__ = ("name", "fn", "args", "keep")

    def __init__(self, name, args, keep=()):
        self.name = name
        self.fn = getattr(lib, name)
        self.args = args
        self.keep = keep

    def __call__(self):
        st = self.fn(*self.args)
        if st != PKV_OK:
            raise PkvError(st, self.name)


def prepare_kv_append(k_pool, v_pool, k_new, v_new, block_tables, context_lens, err_flag=None,
                      stream=None):
    torch = _torch()
    nb, n_kv, d = _pool_dims(k_pool, v_pool)
    _dev(k_new, "k_new", torch.bfloat16, 3)
    _dev(v_new, "v_new", torch.bfloat16, 3)
    num_seqs = k_new.shape[0]
    if tuple(k_new.shape) != (num_seqs, n_kv, d) or tuple(v_new.shape) != (num_seqs, n_kv, d):
        raise ValueError("k_new / v_new: expected [num_seqs, n_kv, head_dim]")
    bt = _dev(block_tables, "block_tables", torch.int32, 2)
    cl = _dev(context_lens, "context_lens", torch.int32, 1)
    if block_tables.shape[0] != num_seqs or context_lens.shape[0] != num_seqs:
        raise ValueError("block_tables / context_lens: first dim must be num_seqs")
    args = (_dev(k_pool, "k_pool", torch.bfloat16), _dev(v_pool, "v_pool", torch.bfloat16),
            _dev(k_new, "k_new", torch.bfloat16), _dev(v_new, "v_new", torch.bfloat16), bt, cl,
            num_seqs, block_tables.shape[1], nb, n_kv, d, _flag(err_flag), _stream(stream))
    return PreparedCall("pkv_kv_append", args,
                        (k_pool, v_pool, k_new, v_new, block_tables, context_lens, err_flag))


def _prepare_decode(name, out, q, k_pool, v_pool, block_tables, context_lens, scale,
                    max_context_len, partition_tokens=0, workspace=None, err_flag=None,
                    stream=None):
    args, ws = _decode_args(out, q, k_pool, v_pool, block_tables, context_lens, scale,
                            max_context_len, partition_tokens, workspace, err_flag, stream)
    return PreparedCall(name, args,
                        (out, q, k_pool, v_pool, block_tables, context_lens, ws, err_flag))


def prepare_decode_step(out, q, k_new, v_new, k_pool, v_pool, block_tables, context_lens, scale,
                        max_context_len, partition_tokens=0, workspace=None, err_flag=None,
                        stream=None):
    args, ws = _step_args(out, q, k_new, v_new, k_pool, v_pool, block_tables, context_lens, scale,
                          max_context_len, partition_tokens, workspace, err_flag, stream)
    return PreparedCall("pkv_decode_step", args,
                        (out, q, k_new, v_new, k_pool, v_pool, block_tables, context_lens, ws,
                         err_flag))


def prepare_decode_step_partition(out, q, k_new, v_new, k_pool, v_pool, block_tables,
                                  context_lens, scale, max_context_len, partition_tokens=0,
                                  workspace=None, err_flag=None, stream=None):
    """The first half of prepare_decode_step; prepare_paged_attn_merge with
    the same arguments (and call.keep[8], the workspace) finishes it."""
    args, ws = _step_args(out, q, k_new, v_new, k_pool, v_pool, block_tables, context_lens, scale,
                          max_context_len, partition_tokens, workspace, err_flag, stream)
    return PreparedCall("pkv_decode_step_partition", args,
                        (out, q, k_new, v_new, k_pool, v_pool, block_tables, context_lens, ws,
                         err_flag))


def prepare_decode_step_partition_valu(out, q, k_new, v_new, k_pool, v_pool, block_tables,
                                       context_lens, scale, max_context_len, workspace=None,
                                       err_flag=None, stream=None):
    """prepare_decode_step_partition with the scores and P.V on the vector
    ALUs (balanced split only); prepare_paged_attn_merge finishes it."""
    args, ws = _step_args(out, q, k_new, v_new, k_pool, v_pool, block_tables, context_lens, scale,
                          max_context_len, 0, workspace, err_flag, stream)
    return PreparedCall("pkv_decode_step_partition_valu", args,
                        (out, q, k_new, v_new, k_pool, v_pool, block_tables, context_lens, ws,
                         err_flag))


def prepare_decode_step_prefix(out, q, k_new, v_new, k_pool, v_pool, block_tables, context_lens,
                               scale, max_context_len, prefix_table, prefix_first_seq,
                               prefix_num_seqs, workspace=None, err_flag=None, stream=None):
    args, ws = _prefix_step_args(out, q, k_new, v_new, k_pool, v_pool, block_tables, context_lens,
                                 scale, max_context_len, prefix_table, prefix_first_seq,
                                 prefix_num_seqs, workspace, err_flag, stream)
    return PreparedCall("pkv_decode_step_prefix", args,
                        (out, q, k_new, v_new, k_pool, v_pool, block_tables, context_lens,
                         prefix_table, ws, err_flag))


def prepare_paged_attn_decode(*a, **k):
    return _prepare_decode("pkv_paged_attn_decode", *a, **k)


def prepare_paged_attn_partition(*a, **k):
    """The partition kernel alone; pass the same workspace to
    prepare_paged_attn_merge (call.keep[6] is the workspace used)."""
    return _prepare_decode("pkv_paged_attn_partition", *a, **k)


def prepare_paged_attn_merge(*a, **k):
    return _prepare_decode("pkv_paged_attn_merge", *a, **k)


def prepare_copy_blocks(k_pool, v_pool, src, dst, err_flag=None, stream=None):
    torch = _torch()
    nb, n_kv, d = _pool_dims(k_pool, v_pool)
    s = _dev(src, "src", torch.int32, 1)
    t = _dev(dst, "dst", torch.int32, 1)
    if src.shape != dst.shape:
        raise ValueError("src / dst: same length required")
    args = (_dev(k_pool, "k_pool", torch.bfloat16), _dev(v_pool, "v_pool", torch.bfloat16), s, t,
            src.shape[0], nb, n_kv, d, _flag(err_flag), _stream(stream))
    return PreparedCall("pkv_copy_blocks", args, (k_pool, v_pool, src, dst, err_flag))


# ---------------------------------------------------------------------------
# continuous batching (host)

def _arr(ptr, n, dtype):
    if n == 0:
        return np.zeros(0, dtype)
    return np.ctypeslib.as_array(ptr, shape=(n,)).astype(dtype, copy=True)


class PrefixCache:
    """Owner of a pkv_prefix_cache over an Allocator (kept alive here)."""

    def __init__(self, alloc: Allocator):
        h = ctypes.c_void_p()
        _check(lib.pkv_prefix_cache_create(alloc._h, ctypes.byref(h)), "pkv_prefix_cache_create")
        self._h = h
        self.alloc = alloc

    def close(self):
        if self._h:
            lib.pkv_prefix_cache_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def match(self, tokens, max_blocks: int) -> np.ndarray:
        """Block ids of the longest cached whole-block prefix (each with a
        new reference for the caller)."""
        t = np.ascontiguousarray(tokens, dtype=np.int32)
        table = np.full(max(max_blocks, 1), -1, np.int32)
        m = lib.pkv_prefix_match(self._h, _i32_host(t, "tokens"), len(t), _i32_host(table, "table"), max_blocks)
        _check(min(m, 0), "pkv_prefix_match")
        return table[:m].copy()

    def insert(self, tokens, table) -> int:
        t = np.ascontiguousarray(tokens, dtype=np.int32)
        b = np.ascontiguousarray(table, dtype=np.int32)
        r = lib.pkv_prefix_insert(self._h, _i32_host(t, "tokens"), len(t), _i32_host(b, "table"), len(b))
        _check(min(r, 0), "pkv_prefix_insert")
        return int(r)

    def evict(self, n_blocks: int) -> int:
        r = lib.pkv_prefix_evict(self._h, n_blocks)
        _check(min(r, 0), "pkv_prefix_evict")
        return int(r)

    def cached_blocks(self) -> int:
        return int(lib.pkv_prefix_cached_blocks(self._h))


class Plan:
    """One step of pkv_batcher_step, copied into numpy arrays."""

    def __init__(self, c: StepPlan):
        n, mb = c.num_seqs, c.max_blocks_per_seq
        self.num_seqs = n
        self.block_tables = _arr(c.block_tables, n * mb, np.int32).reshape(n, mb)
        self.context_lens = _arr(c.context_lens, n, np.int32)
        self.request_ids = _arr(c.request_ids, n, np.int64)
        self.cow_src = _arr(c.cow_src, c.n_cow, np.int32)
        self.cow_dst = _arr(c.cow_dst, c.n_cow, np.int32)
        self.fill_rows = _arr(c.fill_rows, c.n_fill, np.int32)
        self.fill_positions = _arr(c.fill_positions, c.n_fill, np.int32)
        self.finished_ids = _arr(c.finished_ids, c.n_finished, np.int64)
        self.preempted_ids = _arr(c.preempted_ids, c.n_preempted, np.int64)
        self.num_free_blocks = c.num_free_blocks
        self.num_waiting = c.num_waiting
        self.n_cached_tokens = c.n_cached_tokens


class Batcher:
    """Owner of a pkv_batcher handle (host memory, one thread)."""

    def __init__(self, num_blocks: int, max_batch: int, max_blocks_per_seq: int,
                 prefix_tokens: int = 0):
        h = ctypes.c_void_p()
        _check(lib.pkv_batcher_create(num_blocks, max_batch, max_blocks_per_seq, prefix_tokens,
                                      ctypes.byref(h)), "pkv_batcher_create")
        self._h = h
        self.max_blocks_per_seq = max_blocks_per_seq
        self.prefix_tokens = prefix_tokens

    def close(self):
        if self._h:
            lib.pkv_batcher_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def enable_prefix_cache(self):
        _check(lib.pkv_batcher_enable_prefix_cache(self._h), "pkv_batcher_enable_prefix_cache")

    def submit_tokens(self, request_id: int, tokens, gen_len: int):
        t = np.ascontiguousarray(tokens, dtype=np.int32)
        _check(lib.pkv_batcher_submit_tokens(self._h, int(request_id), _i32_host(t, "tokens"),
                                             len(t), int(gen_len)), "pkv_batcher_submit_tokens")

    def cached_blocks(self) -> int:
        return int(lib.pkv_batcher_cached_blocks(self._h))

    def prefix_table(self):
        """(table int32 [max_blocks_per_seq], number of prefix blocks)."""
        p = _i32p()
        n = lib.pkv_batcher_prefix_table(self._h, ctypes.byref(p))
        if n < 0:
            raise PkvError(n, "pkv_batcher_prefix_table")
        return _arr(p, self.max_blocks_per_seq, np.int32), int(n)

    def submit(self, request_id: int, prompt_len: int, gen_len: int, shares_prefix: bool = False):
        _check(lib.pkv_batcher_submit(self._h, int(request_id), int(prompt_len), int(gen_len),
                                      1 if shares_prefix else 0), "pkv_batcher_submit")

    def step(self) -> Plan:
        c = StepPlan()
        _check(lib.pkv_batcher_step(self._h, ctypes.byref(c)), "pkv_batcher_step")
        return Plan(c)
