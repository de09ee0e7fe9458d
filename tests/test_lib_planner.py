"""The C++ row planner (trainable-mode trie, leaf placement) against the oracle.

Bit-exact: node numbering, seq_last, the row of every sequence and the tokens
of every row, on random forests (both trie modes, both placement modes) and
on the pages' packing example [ART "Does it actually help?"].
"""

import json
import os

import numpy as np
import pytest

import prefix_tree_packed_dfs_amd as lib
from oracle.pack import place_leaves, segments
from oracle.trie import build_trie

from .test_oracle_pack import GOLDEN, _art_example, _random_forest


@pytest.mark.parametrize("seed", range(40))
def test_trainable_trie_matches_oracle(seed):
    rng = np.random.default_rng(500 + seed)
    seqs, train = _random_forest(rng, int(rng.integers(1, 14)), vocab=int(rng.integers(2, 4)), p_train=0.6)
    for ms in (1, 3, 64):
        ref = build_trie(seqs, min_shared=ms, trainable=train)
        parent, seq_last = lib.tree_build_trie(seqs, min_shared=ms, trainable=train)
        assert np.array_equal(parent, ref.parent)
        assert np.array_equal(seq_last, ref.seq_last)


@pytest.mark.parametrize("seed", range(40))
@pytest.mark.parametrize("mode", ["global", "in_order"])
def test_placement_matches_oracle(seed, mode):
    rng = np.random.default_rng(900 + seed)
    seqs, train = _random_forest(rng, int(rng.integers(1, 20)), vocab=int(rng.integers(2, 4)), p_train=0.5)
    tr = build_trie(seqs, min_shared=int(rng.integers(1, 5)), trainable=train if seed % 2 else None)
    grp = rng.integers(0, 5, len(seqs)).astype(np.int32)
    cap = max(len(s) for s in seqs) + int(rng.integers(0, 40))
    ref = place_leaves(segments(tr.parent, tr.seq_last), grp, cap, mode)
    bin_of, tokens = lib.tree_place_leaves(tr.parent, tr.seq_last, grp, cap, mode)
    assert np.array_equal(bin_of, ref.bin_of_seq)
    assert np.array_equal(tokens, ref.bin_tokens)


@pytest.mark.parametrize("mode", ["global", "in_order"])
def test_art_example_rows_library(mode):
    g, seqs, train, grp = _art_example()
    parent, seq_last = lib.tree_build_trie(seqs, trainable=train)
    bin_of, tokens = lib.tree_place_leaves(parent, seq_last, grp, g["row_len"], mode)
    want = g["global_rows" if mode == "global" else "in_order_rows"]
    assert tokens.tolist() == [r["tokens"] for r in want]


def test_placement_errors():
    parent, seq_last = lib.tree_build_trie([np.arange(50, dtype=np.int32)], min_shared=1)
    with pytest.raises(lib.TreeAttnError, match="CAPACITY"):
        lib.tree_place_leaves(parent, seq_last, [0], 49)
    bad = parent.copy()
    bad[3] = 10                                   # a node before its parent
    with pytest.raises(lib.TreeAttnError, match="BAD_TREE"):
        lib.tree_place_leaves(bad, seq_last, [0], 100)
    with pytest.raises(lib.TreeAttnError, match="INVALID_ARG"):
        lib.tree_place_leaves(parent, seq_last, None, 100, "global")   # groups required
    b, t = lib.tree_place_leaves(parent, seq_last, None, 100, "in_order")
    assert b.tolist() == [0] and t.tolist() == [50]


# ---------------------------------------------------------------------------
# tree_plan_rows: TRL's planner (rows grown sample by sample under a budget of forwarded tokens)
# ---------------------------------------------------------------------------

from oracle.pack import grow_rows  # noqa: E402


@pytest.mark.parametrize("seed", range(40))
def test_plan_rows_matches_oracle(seed):
    rng = np.random.default_rng(1300 + seed)
    seqs, _ = _random_forest(rng, int(rng.integers(1, 30)), vocab=int(rng.integers(2, 4)), max_len=60)
    budget = max(len(s) for s in seqs) + int(rng.integers(0, 200))
    for thr in (0, 1, 4, 9, 1024):
        ref = grow_rows(seqs, token_budget=budget, fork_threshold=thr)
        row_of, row_tok, forked = lib.tree_plan_rows(seqs, budget, thr)
        assert np.array_equal(row_of, ref.row_of_seq)
        assert np.array_equal(row_tok, ref.row_tokens)
        assert np.array_equal(forked, ref.forked)


def test_plan_rows_workloads_match_oracle():
    """grpo_group's 16 rollouts and long_history's 8 under budgets that split them, both thresholds."""
    from synth import grpo_group, long_history
    for w, budgets in ((grpo_group(), (18_447, 10_000, 6_000)), (long_history(), (36_864, 30_000))):
        for thr in (64, 1024, 4096):
            for budget in budgets:
                ref = grow_rows(w.sequences, token_budget=budget, fork_threshold=thr)
                row_of, row_tok, forked = lib.tree_plan_rows(w.sequences, budget, thr)
                assert np.array_equal(row_of, ref.row_of_seq) and np.array_equal(row_tok, ref.row_tokens)
                assert np.array_equal(forked, ref.forked)


def test_plan_rows_errors():
    import ctypes as C
    L = lib.lib
    with pytest.raises(lib.TreeAttnError) as e:
        lib.tree_plan_rows([[1, 2, 3], list(range(50))], 40)
    assert e.value.status == 3
    with pytest.raises(lib.TreeAttnError) as e:
        lib.tree_plan_rows([[1, 2]], 0)
    assert e.value.status == 1
    with pytest.raises(lib.TreeAttnError) as e:
        lib.tree_plan_rows([[1, 2]], 10, -1)
    assert e.value.status == 1
    # fewer row slots than rows: TREE_ERR_CAPACITY, the row count and every sample's row still written
    seqs = [np.arange(10 * i, 10 * i + 8, dtype=np.int32) for i in range(5)]
    offs = np.zeros(6, np.int64)
    np.cumsum([8] * 5, out=offs[1:])
    toks = np.concatenate(seqs)
    row_of = np.full(5, -7, np.int32)
    row_tok = np.zeros(2, np.int64)
    n = C.c_int32(0)
    i32, i64 = C.POINTER(C.c_int32), C.POINTER(C.c_int64)
    st = L.tree_plan_rows(5, offs.ctypes.data_as(i64), toks.ctypes.data_as(i32), 1024, 16, row_of.ctypes.data_as(i32),
                          row_tok.ctypes.data_as(i64), 2, C.byref(n), None)
    assert st == 3 and n.value == 3 and row_of.tolist() == [0, 0, 1, 1, 2]
    assert lib.tree_plan_rows([], 10)[1].size == 0
