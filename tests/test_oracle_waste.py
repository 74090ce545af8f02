"""Pins of the oracle's allocation arithmetic to numbers the pages print."""

import math
import random

import numpy as np

import oracle


def _pct1(x):
    return round(100.0 * x, 1)


def test_worked_example(golden):
    g = golden("worked_example.json")
    L, bs = g["lengths"], g["block_size"]
    assert int(np.sum(L)) == g["used"]
    assert list(oracle.blocks_for(L, bs)) == g["pages"]
    assert list(oracle.blocks_for(L, bs) * bs) == g["alloc"]
    assert list(oracle.tail_slots(L, bs)) == g["tail_waste"]
    paged = oracle.paged_slots(L, bs)
    naive = oracle.naive_slots(L, g["reserve_max_len"])
    assert paged == g["paged_alloc"]
    assert naive == g["naive_alloc"]
    assert _pct1(oracle.waste_fraction(L, paged)) == g["paged_waste_pct_1dp"]
    assert _pct1(oracle.waste_fraction(L, naive)) == g["naive_waste_pct_1dp"]
    assert oracle.capacity(g["pool_slots"], naive, len(L)) == g["capacity_naive"]
    assert oracle.capacity(g["pool_slots"], paged, len(L)) == g["capacity_paged"]


def test_waste_table(golden):
    g = golden("waste_table.json")
    bs = g["block_size"]
    for row in g["rows"]:
        L = row["length"]
        assert int(oracle.blocks_for(L, bs)) == row["blocks"]
        assert int(oracle.tail_slots(L, bs)) == row["wasted_slots"]
        assert _pct1(oracle.waste_fraction([L], oracle.paged_slots([L], bs))) == row["waste_pct_1dp"]
    # worst case over every length: bs - 1 slots
    Ls = np.arange(1, 5000)
    assert int(oracle.tail_slots(Ls, bs).max()) == g["worst_case_wasted_slots"]
    assert int(oracle.blocks_for(g["note_80_tokens"]["length"], bs)) == g["note_80_tokens"]["blocks"]
    assert int(oracle.blocks_for(g["note_100k"]["length"], bs)) == g["note_100k"]["blocks"]


def test_expected_tail_is_half_block():
    # "Serving: vLLM and PagedAttention" 2.2: the tail averages (B_b - 1) / 2 = 7.5
    # slots at B_b = 16 when L mod B_b is uniform.
    for bs in (8, 16, 32):
        Ls = np.arange(1, bs * 1000 + 1)
        assert float(np.mean(oracle.tail_slots(Ls, bs))) == (bs - 1) / 2


def _page_lengths(max_len, n=2000, seed=0):
    """The page's simulated workload: CPython's random seeded 0, lognormal(5.5, 0.9)
    truncated to an integer and capped at max_len."""
    gen = random.Random(seed)
    out = []
    while len(out) < n:
        out.append(min(max_len, int(gen.lognormvariate(5.5, 0.9))))
    return out


def test_fragmentation_simulation(golden):
    g = golden("fragmentation_sim.json")
    L = _page_lengths(g["max_len"], g["n"])
    assert sum(L) == g["tokens_stored"]
    naive = oracle.naive_slots(L, g["max_len"])
    paged = oracle.paged_slots(L, 16)
    assert naive == g["naive_alloc"]
    assert paged == g["paged_alloc_bs16"]
    assert _pct1(oracle.utilisation(L, naive)) == g["naive_util_pct_1dp"]
    assert _pct1(oracle.utilisation(L, paged)) == g["paged_util_pct_1dp_bs16"]
    assert round(sum(L) / len(L)) == g["mean_length_0dp"]
    assert round((paged - sum(L)) / len(L), 1) == g["wasted_per_seq_1dp"]
    for bs, pct in g["sweep_util_pct_1dp"].items():
        assert _pct1(oracle.utilisation(L, oracle.paged_slots(L, int(bs)))) == pct
    L2 = _page_lengths(32768, g["n"])
    m = g["max_len_32768"]
    assert _pct1(oracle.utilisation(L2, oracle.naive_slots(L2, 32768))) == m["naive_util_pct_1dp"]
    assert _pct1(oracle.utilisation(L2, oracle.paged_slots(L2, 16))) == m["paged_util_pct_1dp_bs16"]


def test_capacity_example(golden):
    g = golden("capacity_example.json")
    per_tok = g["layers"] * g["kv_heads"] * g["head_dim"] * 2 * g["kv_elem_bytes"]
    assert per_tok == g["bytes_per_token"]
    assert per_tok * g["conversation_tokens"] == g["bytes_per_conversation"]
    assert per_tok * g["block_size"] == g["bytes_per_block"]
    assert g["pool_bytes"] // g["bytes_per_block"] == g["pool_blocks"]
    n = int(oracle.blocks_for(g["answer_tokens"], g["block_size"]))
    assert n == g["answer_blocks"]
    last = g["answer_tokens"] - (n - 1) * g["block_size"]
    assert last == g["answer_last_block_tokens"]
    assert int(oracle.tail_slots(g["answer_tokens"], g["block_size"])) == g["answer_last_block_free"]
    assert n * g["bytes_per_block"] // 2**20 == g["answer_mib"]
    p = int(oracle.blocks_for(g["system_prompt_tokens"], g["block_size"]))
    assert p == g["system_prompt_blocks"]
    assert p * g["bytes_per_block"] // 2**20 == g["system_prompt_mib"]


def test_blocks_for_edge_cases():
    assert int(oracle.blocks_for(0, 16)) == 0
    assert int(oracle.blocks_for(-3, 16)) == 0
    assert int(oracle.blocks_for(1, 16)) == 1
    assert int(oracle.blocks_for(16, 16)) == 1
    assert int(oracle.blocks_for(17, 16)) == 2
    assert int(oracle.tail_slots(16, 16)) == 0
    assert int(oracle.tail_slots(17, 16)) == 15
    assert math.isclose(oracle.waste_fraction([16, 32], 48), 0.0)
