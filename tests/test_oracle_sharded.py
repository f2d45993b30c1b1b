"""The oracle's sharded driver (the same C function over disjoint shards of
the sequences, one host thread each) gives the single call's rows bit for
bit, for any shard count, including more shards than sequences."""
import numpy as np
import pytest

import workload as w


@pytest.mark.parametrize("threads", [1, 3, 8, 40])
def test_sharded_equals_single_call(orc, threads):
    hc = w.host_case(w.Shape("sharded", 1, 20, 4, 64, 11, 1, 700), 71)
    one, rc1 = orc.decode(hc.q, hc.k_pool, hc.v_pool, hc.tables.block_tables,
                          hc.tables.context_lens, 4, 0.125)
    many, rc2 = orc.decode_sharded(hc.q, hc.k_pool, hc.v_pool, hc.tables.block_tables,
                                   hc.tables.context_lens, 4, 0.125, threads)
    assert rc1 == 0 and rc2 == 0
    assert np.array_equal(one, many)


def test_sharded_reports_invalid_sequences(orc):
    hc = w.host_case(w.Shape("sharded bad", 1, 8, 2, 64, 6, 1, 300), 72)
    cl = hc.tables.context_lens.copy()
    cl[4] = 0
    _, rc1 = orc.decode(hc.q, hc.k_pool, hc.v_pool, hc.tables.block_tables, cl, 2, 0.125)
    _, rc2 = orc.decode_sharded(hc.q, hc.k_pool, hc.v_pool, hc.tables.block_tables, cl, 2, 0.125, 3)
    assert rc1 == rc2 != 0
