"""Pins for the oracle's DFS layout (CPU only)."""

import json
import os

import numpy as np
import pytest

from oracle.brute import ancestor_mask
from oracle.layout import dfs_layout
from oracle.trie import build_trie


def _random_forest(rng, n):
    parent = np.full(n, -1, dtype=np.int64)
    for v in range(1, n):
        parent[v] = -1 if rng.random() < 0.1 else int(rng.integers(0, v))
    perm = rng.permutation(n)                    # arbitrary node numbering
    inv = np.empty(n, dtype=np.int64)
    inv[perm] = np.arange(n)
    p2 = np.full(n, -1, dtype=np.int64)
    for v in range(n):
        if parent[v] >= 0:
            p2[inv[v]] = inv[parent[v]]
    return p2


def test_mask_caption_example(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "art_mask_caption.json")))
    parent = np.asarray(g["parent"])
    lay = dfs_layout(parent, [8, 5], 9)
    assert np.array_equal(lay.slot_node, np.arange(9))
    i = g["query"]
    se = lay.subtree_end
    visible = [j for j in range(9) if j <= i <= se[j]]
    assert visible == g["visible"]
    M = ancestor_mask(parent)
    assert np.nonzero(M[i])[0].tolist() == g["visible"]
    # the root segment is one fully visible block for query 7, its own branch a causal run
    assert all(M[i, j] for j in g["full_block_for_query_7"])
    assert not any(M[i, j] for j in range(3, 6))


@pytest.mark.parametrize("seed", range(20))
def test_layout_invariants(seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(1, 60))
    parent = _random_forest(rng, n)
    R = n + int(rng.integers(0, 5))
    leaves = [v for v in range(n) if not np.any(parent == v)]
    lay = dfs_layout(parent, leaves, R)
    sn, se, pos = lay.slot_node, lay.subtree_end, lay.pos_ids
    slot_parent = np.full(R, -1)
    for s in range(n):
        p = parent[sn[s]]
        slot_parent[s] = -1 if p < 0 else lay.node_slot[p]
        if p >= 0:
            assert slot_parent[s] < s
            assert pos[s] == pos[slot_parent[s]] + 1
        else:
            assert pos[s] == 0
    M = ancestor_mask(slot_parent[:n])
    # interval test == ancestor-or-self from parent pointers
    for i in range(n):
        for j in range(n):
            assert M[i, j] == (j <= i <= se[j])
    # pair count = sum of (depth + 1)
    assert M.sum() == int((pos[:n] + 1).sum())
    # padding
    assert np.all(sn[n:] == -1) and np.array_equal(se[n:], np.arange(n, R)) and np.all(pos[n:] == 0)
    # token_index follows parent pointers back to a root
    for k, leaf in enumerate(leaves):
        ti = lay.token_index[k]
        assert ti[-1] == lay.node_slot[leaf] and slot_parent[ti[0]] == -1
        assert np.array_equal(slot_parent[ti[1:]], ti[:-1])
        assert np.array_equal(pos[ti], np.arange(len(ti)))


def test_trie_layout_depth_is_position():
    rng = np.random.default_rng(3)
    seqs = [rng.integers(0, 3, size=int(rng.integers(1, 12))).tolist() for _ in range(7)]
    trie = build_trie(seqs, min_shared=1)
    lay = dfs_layout(trie.parent, trie.seq_last, trie.n_nodes + 3)
    toks = np.full(lay.row_len, -1)
    toks[:trie.n_nodes] = trie.token[lay.slot_node[:trie.n_nodes]]
    for s, seq in enumerate(seqs):
        assert np.array_equal(toks[lay.token_index[s]], seq)
        assert np.array_equal(lay.pos_ids[lay.token_index[s]], np.arange(len(seq)))


def test_layout_rejects_bad_trees():
    with pytest.raises(ValueError):
        dfs_layout([1, 0], [0], 2)            # a 2-cycle, no root
    with pytest.raises(ValueError):
        dfs_layout([-1, 5], [1], 2)           # parent out of range
    with pytest.raises(ValueError):
        dfs_layout([-1, 0, 1], [2], 2)        # row shorter than the tree


def test_deep_chain_iterative():
    n = 30000
    parent = np.arange(-1, n - 1)
    lay = dfs_layout(parent, [n - 1], n)
    assert lay.pos_ids[-1] == n - 1 and lay.subtree_end[0] == n - 1
