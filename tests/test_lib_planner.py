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
