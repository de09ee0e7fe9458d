"""Pins of the row-planner oracle (trainable-mode trie, segments, placement).

Pinned to the pages' worked packing example (exact row fills and contents,
[ART "Does it actually help?"], fixture tests/golden/art_row_placement.json),
to classical best-fit decreasing when nothing is shared (the reduction in
[ART "Appendix: this isn't quite bin packing"]), and to invariants: a row's
load is the size of the union of its leaves' segments, no row is over
capacity, trainable tokens are never shared.
"""

import itertools
import json
import os

import numpy as np
import pytest

from oracle.pack import place_leaves, segments
from oracle.trie import build_trie

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "art_row_placement.json")


def _art_example(seed=0):
    g = json.load(open(GOLDEN))
    rng = np.random.default_rng(seed)
    root = rng.integers(1000, 2000, g["root_tokens"])
    seqs, train, grp = [], [], []
    P = g["group_prefix_tokens"]
    for gi, spec in enumerate(g["groups"]):
        prefix = np.concatenate([[10 + gi], rng.integers(2000, 3000, P - 1)])
        for _ in range(spec["rollouts"]):
            comp = rng.integers(3000, 1 << 20, spec["completion"])
            seqs.append(np.concatenate([root, prefix, comp]))
            train.append(np.concatenate([np.zeros(len(root) + P, bool), np.ones(len(comp), bool)]))
            grp.append(gi)
    return g, seqs, train, np.asarray(grp)


def _contents(g, grp, pl):
    names = [s["name"] for s in g["groups"]]
    out = []
    for b in range(len(pl.bin_tokens)):
        cnt = np.bincount(grp[pl.bin_of_seq == b], minlength=len(names))
        out.append({names[i]: int(c) for i, c in enumerate(cnt) if c})
    return out


@pytest.mark.parametrize("mode", ["global", "in_order"])
def test_art_example_rows(mode):
    g, seqs, train, grp = _art_example()
    tr = build_trie(seqs, trainable=train)
    pl = place_leaves(segments(tr.parent, tr.seq_last), grp, g["row_len"], mode)
    want = g["global_rows" if mode == "global" else "in_order_rows"]
    assert pl.bin_tokens.tolist() == [r["tokens"] for r in want]
    assert _contents(g, grp, pl) == [r["contents"] for r in want]
    assert len(pl.bin_tokens) * g["row_len"] == g["allocated_tokens"][mode]


def test_art_example_trainable_accounting():
    """Root shared whole, 11,999 shared prefix tokens per group, completion + 1 per rollout."""
    g, seqs, train, grp = _art_example()
    tr = build_trie(seqs, trainable=train)
    sg = segments(tr.parent, tr.seq_last)
    for s, path in enumerate(sg.paths):
        lens = [int(sg.seg_len[x]) for x in path]
        comp = g["groups"][grp[s]]["completion"]
        assert lens == [g["root_tokens"], g["group_prefix_tokens"] - 1, comp + 1]
    # every node a trainable token lands on belongs to one sequence only
    users = np.zeros(tr.n_nodes, dtype=np.int64)
    trained = np.zeros(tr.n_nodes, dtype=bool)
    for s, p in enumerate(tr.paths):
        np.add.at(users, p, 1)
        trained[p[train[s]]] = True
    assert np.all(users[trained] == 1)


def test_default_mode_copies_every_join():
    """Without trainable flags every fork copies its join token (one more token per fork)."""
    g, seqs, _, grp = _art_example()
    tr = build_trie(seqs)
    pl = place_leaves(segments(tr.parent, tr.seq_last), grp, g["row_len"], "global")
    # root 4,095 + per group (1 + 11,999) + per rollout (completion + 1): one more than trainable
    # mode per group in a row (its join copy below the root)
    assert pl.bin_tokens.tolist() == [130105 + 1, 122114 + 2]


def _bfd_sizes(sizes, cap):
    """Textbook best-fit decreasing on fixed sizes (stable order for equal sizes)."""
    order = sorted(range(len(sizes)), key=lambda i: -sizes[i])
    free, where = [], [0] * len(sizes)
    for i in order:
        best = None
        for b, f in enumerate(free):
            if sizes[i] <= f and (best is None or f - sizes[i] < free[best] - sizes[i]):
                best = b
        if best is None:
            free.append(cap)
            best = len(free) - 1
        free[best] -= sizes[i]
        where[i] = best
    return where, [cap - f for f in free]


@pytest.mark.parametrize("seed", range(5))
def test_private_segments_reduce_to_classical_bfd(seed):
    rng = np.random.default_rng(seed)
    sizes = rng.integers(1, 60, 30).tolist()
    seqs = [np.full(n, 1000 + i) for i, n in enumerate(sizes)]   # distinct first tokens: nothing shared
    tr = build_trie(seqs, min_shared=1)
    pl = place_leaves(segments(tr.parent, tr.seq_last), np.arange(len(seqs)), 100, "global")
    where, load = _bfd_sizes(sizes, 100)
    assert pl.bin_of_seq.tolist() == where
    assert pl.bin_tokens.tolist() == load


def _random_forest(rng, n_seq, vocab=3, max_len=40, p_train=0.3):
    seqs, train = [], []
    for _ in range(n_seq):
        L = int(rng.integers(1, max_len))
        s = np.repeat(rng.integers(0, vocab, L // 8 + 1), 8)[:L]
        seqs.append(s)
        cut = int(rng.integers(0, L + 1))
        t = np.zeros(L, bool)
        if rng.random() < p_train:
            t[cut:] = True
        train.append(t)
    return seqs, train


@pytest.mark.parametrize("seed", range(8))
@pytest.mark.parametrize("trainable", [False, True])
def test_invariants_random(seed, trainable):
    rng = np.random.default_rng(100 + seed)
    seqs, train = _random_forest(rng, 12)
    tr = build_trie(seqs, min_shared=4, trainable=train if trainable else None)
    # paths still spell every sequence
    for s, p in enumerate(tr.paths):
        assert np.array_equal(tr.token[p], seqs[s])
        assert all(tr.parent[p[i]] == p[i - 1] for i in range(1, len(p)))
    sg = segments(tr.parent, tr.seq_last)
    for s, path in enumerate(sg.paths):
        assert sum(int(sg.seg_len[x]) for x in path) == len(seqs[s])
    grp = rng.integers(0, 4, len(seqs))
    cap = max(len(s) for s in seqs) + 10
    for mode in ("global", "in_order"):
        pl = place_leaves(sg, grp, cap, mode)
        assert np.all(pl.bin_of_seq >= 0)
        for b in range(len(pl.bin_tokens)):
            members = np.nonzero(pl.bin_of_seq == b)[0]
            union = set(x for s in members for x in sg.paths[s])
            assert pl.bin_tokens[b] == sum(int(sg.seg_len[x]) for x in union) <= cap
    if trainable:   # a trainable token is never shared
        users = np.zeros(tr.n_nodes, dtype=np.int64)
        trained = np.zeros(tr.n_nodes, dtype=bool)
        for s, p in enumerate(tr.paths):
            np.add.at(users, p, 1)
            trained[p[train[s]]] = True
        assert np.all(users[trained] == 1)


@pytest.mark.parametrize("seed", range(4))
def test_global_rows_never_below_optimum(seed):
    """Brute force over every assignment of 6 leaves: the heuristic uses at least the optimum."""
    rng = np.random.default_rng(7 + seed)
    seqs, _ = _random_forest(rng, 6, vocab=2, max_len=24, p_train=0.0)
    tr = build_trie(seqs, min_shared=2)
    sg = segments(tr.parent, tr.seq_last)
    cap = max(len(s) for s in seqs) + 4
    pl = place_leaves(sg, np.arange(6), cap, "global")
    best = 6
    for assign in itertools.product(range(6), repeat=6):
        if max(assign) + 1 >= best:
            continue
        ok = True
        for b in set(assign):
            union = set(x for s in range(6) if assign[s] == b for x in sg.paths[s])
            if sum(int(sg.seg_len[x]) for x in union) > cap:
                ok = False
                break
        if ok:
            best = max(assign) + 1
    assert len(pl.bin_tokens) >= best


def test_too_long_sequence_is_an_error():
    tr = build_trie([np.arange(50)], min_shared=1)
    with pytest.raises(ValueError):
        place_leaves(segments(tr.parent, tr.seq_last), [0], 49, "global")


# ---------------------------------------------------------------------------
# TRL's planner: rows grown sample by sample under a forwarded-token budget
# ---------------------------------------------------------------------------

from oracle.pack import grow_rows  # noqa: E402

TRL_DOCS = os.path.join(os.path.dirname(__file__), "golden", "trl_docs_example.json")
TRL_ENVELOPE = os.path.join(os.path.dirname(__file__), "golden", "trl_back_of_envelope.json")


def _docs_rollouts():
    g = json.load(open(TRL_DOCS))
    per = g["raw_tokens"] // g["rollouts"]
    prompt = list(range(1, g["prompt_tokens"] + 1))
    return g, [prompt + [100 * (r + 1) + t for t in range(per - g["prompt_tokens"])] for r in range(g["rollouts"])]


def test_grow_rows_docs_example_and_fork_threshold():
    """[TRL "How tree packing works"]: 10 raw tokens, 8 forwarded once the 3-token prompt is shared
    (a fork threshold of at most 3); with the default threshold of 1024 the prompt is too short to
    share and all 10 are forwarded."""
    g, seqs = _docs_rollouts()
    for thr in (0, 1, 3):
        r = grow_rows(seqs, token_budget=100, fork_threshold=thr)
        assert r.row_tokens.tolist() == [g["forwarded_tokens"]] and r.forked.tolist() == [1, 1]
    for thr in (4, 1024):
        r = grow_rows(seqs, token_budget=100, fork_threshold=thr)
        assert r.row_tokens.tolist() == [g["raw_tokens"]] and r.forked.tolist() == [0, 0]
    # the budget bounds forwarded tokens: 8 fit a budget of 8 when shared, 10 do not
    assert grow_rows(seqs, token_budget=8, fork_threshold=1).row_of_seq.tolist() == [0, 0]
    assert grow_rows(seqs, token_budget=8, fork_threshold=1024).row_of_seq.tolist() == [0, 1]


def test_grow_rows_back_of_envelope_history():
    """[TRL "A back-of-envelope example"]: a 20,000-token history and 8 rollouts of 2,000 own tokens.
    With the default threshold the history is shared: k rollouts in a row forward 19,999 + 2,001 k
    tokens (one join copy per branch), so a 36,864-token budget holds all eight (36,007) and a budget
    of 36,006 closes the row after seven (34,006), the eighth opening a row of its own (22,000)."""
    g = json.load(open(TRL_ENVELOPE))
    H, n, u = g["history_tokens"], g["rollouts"], g["new_tokens"]
    hist = list(range(H))
    seqs = [hist + list(range(10 ** 6 * (r + 1), 10 ** 6 * (r + 1) + u)) for r in range(n)]
    r = grow_rows(seqs, token_budget=36864, fork_threshold=1024)
    assert r.row_tokens.tolist() == [H - 1 + n * (u + 1)] and set(r.forked.tolist()) == {1}
    r = grow_rows(seqs, token_budget=H - 1 + n * (u + 1) - 1, fork_threshold=1024)
    assert r.row_tokens.tolist() == [H - 1 + (n - 1) * (u + 1), H + u]
    assert r.row_of_seq.tolist() == [0] * (n - 1) + [1] and r.forked.tolist() == [1] * (n - 1) + [0]
    assert sum(len(s) for s in seqs) == g["raw_tokens"]


def _next_fit(lengths, cap):
    """Textbook next-fit bin packing: items in order, a new bin when the next item does not fit."""
    bins, loads = [], []
    for L in lengths:
        if not loads or loads[-1] + L > cap:
            loads.append(0)
        loads[-1] += L
        bins.append(len(loads) - 1)
    return bins, loads


@pytest.mark.parametrize("seed", range(20))
def test_grow_rows_without_sharing_is_next_fit(seed):
    """Samples with nothing in common (or a threshold above every common run) forward their raw tokens,
    so growing rows in order reduces to next-fit bin packing on the sample lengths."""
    rng = np.random.default_rng(70 + seed)
    lens = rng.integers(1, 60, int(rng.integers(1, 30)))
    seqs = [list(range(10_000 * i, 10_000 * i + int(L))) for i, L in enumerate(lens)]
    cap = int(lens.max()) + int(rng.integers(0, 100))
    bins, loads = _next_fit(lens, cap)
    r = grow_rows(seqs, token_budget=cap, fork_threshold=1)
    assert r.row_of_seq.tolist() == bins and r.row_tokens.tolist() == loads and not r.forked.any()
    shared = [[7] * 5 + s for s in seqs]          # a 5-token common run, below a threshold of 6
    bins, loads = _next_fit(lens + 5, cap + 5)
    r = grow_rows(shared, token_budget=cap + 5, fork_threshold=6)
    assert r.row_of_seq.tolist() == bins and r.row_tokens.tolist() == loads


@pytest.mark.parametrize("seed", range(25))
def test_grow_rows_invariants(seed):
    """Rows are runs of consecutive samples; each holds the trie of its samples, within the budget; a
    row is closed only when the next sample would not fit; a sample alone in its row has not forked."""
    rng = np.random.default_rng(300 + seed)
    seqs, _ = _random_forest(rng, int(rng.integers(1, 25)), vocab=int(rng.integers(2, 4)))
    budget = max(len(s) for s in seqs) + int(rng.integers(0, 120))
    thr = int(rng.integers(0, 20))
    r = grow_rows(seqs, token_budget=budget, fork_threshold=thr)
    row = r.row_of_seq
    assert row[0] == 0 and np.all(np.diff(row) >= 0) and np.all(np.diff(row) <= 1)
    for k in range(len(r.row_tokens)):
        members = np.nonzero(row == k)[0]
        t = build_trie([seqs[i] for i in members], min_shared=max(1, thr)).n_nodes
        assert t == r.row_tokens[k] <= budget
        if k + 1 < len(r.row_tokens):
            nxt = int(np.nonzero(row == k + 1)[0][0])
            assert build_trie([seqs[i] for i in list(members) + [nxt]], min_shared=max(1, thr)).n_nodes > budget
        if len(members) == 1:
            assert r.forked[members[0]] == 0


def test_grow_rows_rejects_a_sample_beyond_the_budget():
    with pytest.raises(ValueError):
        grow_rows([[1, 2, 3], list(range(50))], token_budget=40)
