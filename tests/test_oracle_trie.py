"""Pins for the oracle's trie builder and counts (CPU only)."""

import json
import os

import numpy as np
import pytest

from oracle.counts import distinct_prefixes, packing_counts
from oracle.layout import dfs_layout
from oracle.trie import build_trie
from synth import grpo_group, long_history


def _check_paths(seqs, trie):
    for s, seq in enumerate(seqs):
        p = trie.paths[s]
        assert np.all(p >= 0)
        assert np.array_equal(trie.token[p], np.asarray(seq))
        assert trie.parent[p[0]] == -1
        assert np.array_equal(trie.parent[p[1:]], p[:-1])


def test_docs_example_counts(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "trl_docs_example.json")))
    prompt = [11, 12, 13]
    per = g["raw_tokens"] // g["rollouts"]
    comp = per - g["prompt_tokens"]
    seqs = [prompt + [100 + 10 * r + i for i in range(comp)] for r in range(g["rollouts"])]
    trie = build_trie(seqs, min_shared=1)          # the docs example has no minimum run
    lay = dfs_layout(trie.parent, trie.seq_last, trie.n_nodes)
    c = packing_counts(seqs, lay.token_index, trie.n_nodes)
    assert c["raw"] == g["raw_tokens"]
    assert c["forwarded"] == g["forwarded_tokens"]
    assert trie.n_nodes == g["forwarded_tokens"]
    _check_paths(seqs, trie)


def test_back_of_envelope_counts(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "trl_back_of_envelope.json")))
    w = long_history(prefix=g["history_tokens"], n=g["rollouts"], unique=g["new_tokens"])
    trie = build_trie(w.sequences)
    lay = dfs_layout(trie.parent, trie.seq_last, 36864)
    c = packing_counts(w.sequences, lay.token_index, 36864)
    assert c["raw"] == g["raw_tokens"]
    assert c["distinct_prefixes"] == g["distinct_tokens"]
    # one join copy per branch on top of the distinct tokens
    assert c["forwarded"] == g["distinct_tokens"] + g["rollouts"] - 1
    assert round(c["raw"] / c["distinct_prefixes"], 1) == g["ratio_one_decimal"]
    assert round(c["packing_ratio"], 1) == g["ratio_one_decimal"]
    _check_paths(w.sequences, trie)


def test_grpo_counts_closed_form():
    P, n, C = 2048, 16, 1024
    w = grpo_group(prompt=P, n=n, completion=C)
    trie = build_trie(w.sequences)
    # prompt shared minus its last token, which every completion gets a copy of
    assert trie.n_nodes == (P - 1) + n * (C + 1)
    assert sum(len(s) for s in w.sequences) == n * (P + C)


def _dict_trie_fork_extra(seqs):
    """Sum over non-root trie nodes of (k - 1) for k >= 2 branches (a sequence ending there counts as one)."""
    root = {}
    END = object()
    for s in seqs:
        node = root
        for tok in s:
            node = node.setdefault(tok, {})
        node[END] = True
    extra = 0
    stack = [(root, True)]
    while stack:
        node, is_root = stack.pop()
        kids = [v for k, v in node.items() if k is not END]
        k = len(kids) + (1 if (END in node and kids) else 0)
        if not is_root and k >= 2:
            extra += k - 1
        stack.extend((c, False) for c in kids)
    return extra


@pytest.mark.parametrize("seed", range(40))
def test_node_count_brute_force(seed):
    """With min_shared=1: nodes = distinct prefixes + (k-1) join copies per k-way fork."""
    rng = np.random.default_rng(seed)
    n = int(rng.integers(1, 9))
    vocab = int(rng.integers(2, 4))
    seqs = [rng.integers(0, vocab, size=int(rng.integers(1, 9))).tolist() for _ in range(n)]
    trie = build_trie(seqs, min_shared=1)
    assert trie.n_nodes == distinct_prefixes(seqs) + _dict_trie_fork_extra(seqs)
    _check_paths(seqs, trie)
    # emission order is a pre-order: the DFS layout of the trie is the identity
    lay = dfs_layout(trie.parent, trie.seq_last, trie.n_nodes)
    assert np.array_equal(lay.slot_node, np.arange(trie.n_nodes))


def test_min_shared_boundary():
    """A 64-token run that forks stays shared (63 + a copy per branch); 63 tokens are not shared."""
    base = list(range(1000, 1064))
    a = base + [1, 2, 3]
    b = base + [4, 5, 6]
    t64 = build_trie([a, b], min_shared=64)
    assert t64.n_nodes == 63 + 2 * (1 + 3)
    t65 = build_trie([a, b], min_shared=65)
    assert t65.n_nodes == len(a) + len(b)
    assert t65.parent[t65.paths[1][0]] == -1


def test_short_run_copied_then_shared_deeper():
    """A short common run is copied per next-token partition; longer runs below it are shared."""
    short = [7, 7, 7]
    deep = list(range(500, 600))
    seqs = [short + [1] + deep + [10], short + [1] + deep + [11], short + [2, 9]]
    trie = build_trie(seqs, min_shared=64)
    # partition {0,1} shares short+[1]+deep (104 tokens) minus the join, then two 2-token branches
    assert trie.n_nodes == (3 + 1 + 100 - 1) + 2 * 2 + 5
    p0, p1, p2 = trie.paths
    assert np.array_equal(p0[:103], p1[:103]) and p0[103] != p1[103]
    assert p2[0] != p0[0]                         # the short run is not shared with sequence 2
    _check_paths(seqs, trie)


def test_identical_and_prefix_sequences():
    s = list(range(100, 180))
    trie = build_trie([s, list(s)], min_shared=64)
    assert trie.n_nodes == len(s)
    assert np.array_equal(trie.paths[0], trie.paths[1])
    # a strict prefix of another sequence gets its own copy of the join token
    trie = build_trie([s, s + [1, 2]], min_shared=64)
    assert trie.n_nodes == (len(s) - 1) + 1 + 3
    assert trie.paths[0][-1] != trie.paths[1][len(s) - 1]


def test_branch_order_ascending_next_token():
    base = list(range(64))
    seqs = [base + [9, 1], base + [3, 1], base + [5, 1]]
    trie = build_trie(seqs, min_shared=64)
    firsts = [int(trie.paths[s][64]) for s in range(3)]
    order = np.argsort(firsts)
    assert [seqs[i][64] for i in order] == [3, 5, 9]


def test_counts_fields():
    seqs = [[1, 2, 3, 4], [1, 2, 3, 5], [9, 9]]
    trie = build_trie(seqs, min_shared=1)
    lay = dfs_layout(trie.parent, trie.seq_last, 16)
    c = packing_counts(seqs, lay.token_index, 16)
    assert c["raw"] == 10 and c["forwarded"] == trie.n_nodes == 2 + 2 * 2 + 2
    assert c["row_fill"] == trie.n_nodes / 16
    assert c["fork_frac"] == pytest.approx(2 / 3)
