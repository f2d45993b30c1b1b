"""Every plausible mistake in the oracle must fail at least one pin.

Each mutant is a one-line textual change to a temporary copy of
oracle/oracle.c (a dropped term, a wrong sign, index or layout, a missing
normalisation), compiled with the same flags; the pin checks of
tests/oracle_pins.py then run against it. Nothing here touches the real
oracle build or the GPU.
"""
import os
import tempfile

import pytest

import oracle
from oracle.build import SRC, build
from oracle_pins import ALL_CHECKS

MUTANTS = {
    "kv_head_modulo": ("ctx, num_blocks, n_kv, j / group,", "ctx, num_blocks, n_kv, j % n_kv,"),
    "verify_kv_head_modulo": ("seen, num_blocks, n_kv, j / group,", "seen, num_blocks, n_kv, j % n_kv,"),
    "dropped_scale": ("z[t] = scale * dot;", "z[t] = dot;"),
    "exp_sign": ("z[t] = exp(z[t] - zmax);", "z[t] = exp(zmax - z[t]);"),
    "max_not_subtracted": ("z[t] = exp(z[t] - zmax);", "z[t] = exp(z[t]);"),
    "v_layout_token_major": ("* d + i) * ORACLE_BLOCK + t);", "* ORACLE_BLOCK + t) * d + i);"),
    "v_slot_from_block_index": ("v_index(blk, h, t % ORACLE_BLOCK, i, n_kv, d)",
                                "v_index(blk, h, t / ORACLE_BLOCK, i, n_kv, d)"),
    "k_dim_slot_swapped": ("bf16_value(k_pool[k_index(blk, h, slot, i, n_kv, d)])",
                           "bf16_value(k_pool[k_index(blk, h, i % ORACLE_BLOCK, slot, n_kv, d)])"),
    "context_off_by_one": ("for (int t = 0; t < ctx; ++t) {\n    int32_t blk",
                           "for (int t = 0; t < ctx - 1; ++t) {\n    int32_t blk"),
    "no_normalisation": ("out_row[i] = num / denom;", "out_row[i] = num;"),
    "append_slot_shift": ("    int slot = pos % ORACLE_BLOCK;\n    for (int h = 0; h < n_kv; ++h) {\n      for (int i = 0; i < d; ++i) {\n        size_t src = ((size_t)s",
                          "    int slot = (pos + 1) % ORACLE_BLOCK;\n    for (int h = 0; h < n_kv; ++h) {\n      for (int i = 0; i < d; ++i) {\n        size_t src = ((size_t)s"),
    "append_table_entry": ("(size_t)s * max_blocks_per_seq + pos / ORACLE_BLOCK];", "(size_t)s * max_blocks_per_seq + ctx / ORACLE_BLOCK];"),
    "write_slot_from_row": ("    int slot = pos % ORACLE_BLOCK;\n    for (int h = 0; h < n_kv; ++h) {\n      for (int i = 0; i < d; ++i) {\n        size_t src = ((size_t)tok",
                            "    int slot = row % ORACLE_BLOCK;\n    for (int h = 0; h < n_kv; ++h) {\n      for (int i = 0; i < d; ++i) {\n        size_t src = ((size_t)tok"),
    "write_source_row": ("        size_t src = ((size_t)tok * n_kv + h) * d + i;", "        size_t src = ((size_t)row * n_kv + h) * d + i;"),
    "copy_k_only": ("      v_pool[(size_t)dst[p] * per_block + e] = v_pool[(size_t)src[p] * per_block + e];\n", ""),
    "verify_no_causal": ("int seen = ctx - q_len + i + 1;", "int seen = ctx;"),
    "verify_seen_off_by_one": ("int seen = ctx - q_len + i + 1;", "int seen = ctx - q_len + i + 2;"),
    "verify_reversed_tokens": ("int seen = ctx - q_len + i + 1;", "int seen = ctx - i;"),
    "verify_query_of_decode_layout": ("int rc = oracle_decode_row(row, q + row_index * d,",
                                      "int rc = oracle_decode_row(row, q + ((size_t)s * n_q + j) * d,"),
    "verify_short_context_accepted": ("int bad_ctx = ctx < q_len ||", "int bad_ctx ="),
    "kv_bytes_no_two": ("return (uint64_t)2 * (uint64_t)n_layers", "return (uint64_t)n_layers"),
    "kv_bytes_no_precision": (" *\n         (uint64_t)bytes_per_value;", ";"),
    "f32_dropped_scale": ("w[p] = scale * qk;", "w[p] = qk;"),
    "f32_exp_sign": ("w[p] = expf(w[p] - top);", "w[p] = expf(top - w[p]);"),
    "f32_max_not_subtracted": ("w[p] = expf(w[p] - top);", "w[p] = expf(w[p]);"),
    "f32_no_normalisation": ("out_row[i] = acc / total;", "out_row[i] = acc;"),
    "f32_kv_head_modulo": ("int kv_head = j / group;", "int kv_head = j % n_kv;"),
    "f32_v_slot_from_dim": ("      acc += w[p] * bf16_float(v_pool[v_index(block, h, in_block, i, n_kv, d)]);",
                            "      acc += w[p] * bf16_float(v_pool[v_index(block, h, i % ORACLE_BLOCK, i, n_kv, d)]);"),
    "f32_context_off_by_one": ("  for (int p = 0; p < ctx; ++p) {\n    int32_t block",
                               "  for (int p = 0; p < ctx - 1; ++p) {\n    int32_t block"),
    "f32_last_token_dropped_from_sum": ("    total += w[p];", "    if (p + 1 < ctx) total += w[p];"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    old, new = MUTANTS[name]
    with open(SRC) as f:
        text = f.read()
    assert text.count(old) == 1, f"mutation anchor for {name} not unique in oracle.c"
    src = tmp_path / "oracle_mutant.c"
    src.write_text(text.replace(old, new))
    lib = tmp_path / "liboracle_mutant.so"
    build(src=str(src), lib=str(lib))
    mutant = oracle.Oracle(str(lib))
    failed = []
    for check in ALL_CHECKS:
        try:
            check(mutant)
        except Exception as e:  # noqa: BLE001 -- any failure counts as caught
            failed.append((check.__name__, type(e).__name__))
    assert failed, f"mutant {name} passed every pin"
