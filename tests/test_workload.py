"""The workload generators' shape helpers (host only)."""
import pytest

import workload as w


def test_tp_shard_keeps_group_and_divides_heads():
    """A shard by KV head keeps the query heads with the KV heads they
    read: the group size, layers, batch and contexts are unchanged, and the
    KV bytes per token fall by the shard count."""
    full = w.CONFIGS[5]
    s = w.tp_shard(full, 4)
    assert (s.n_q, s.n_kv) == (16, 2)
    assert s.group == full.group == 8
    assert (s.n_layers, s.batch, s.ctx_lo, s.ctx_hi, s.d) == \
        (full.n_layers, full.batch, full.ctx_lo, full.ctx_hi, full.d)
    assert 4 * s.n_kv * s.d == full.n_kv * full.d
    assert w.tp_shard(full, 1) is full


@pytest.mark.parametrize("tp", [0, 3, 16])
def test_tp_shard_rejects_uneven_splits(tp):
    with pytest.raises(ValueError):
        w.tp_shard(w.CONFIGS[5], tp)
