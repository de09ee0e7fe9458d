"""Oracle for the row planner: segments of the packed trie and leaf placement.

TEST INFRASTRUCTURE ONLY: used by tests/ and bench.py's CPU baseline, never by
the library.

[ART "Bin packing, with a twist"]: a leaf (one sequence) is the list of
(segment, length) pairs on its root-to-leaf path in the global trie; its cost
of joining a row is the length of the segments that row does not hold yet
(the insertion delta), so a row's load is the size of the union of its
leaves' segments.  Rows are filled by best-fit decreasing over that marginal
cost: groups in decreasing order of their most expensive leaf (a leaf's
standalone cost is its full path length), each leaf into the row that is left
with the least free space after it, a new row when none can take it.
[ART "Does it actually help?"] also describes the packer this replaced:
rows filled one at a time in arrival order, moving on for good when the next
sequence does not fit ("in order" here).

Readings (listed in the design doc):
* a segment is a maximal chain of trie nodes: a node starts a new segment
  when it is a root, when its parent has more than one child, or when its
  parent is the last token of some sequence (so every sequence's path is a
  whole number of segments);
* groups keep the order of their first sequence among equally expensive
  groups (a stable sort); leaves keep input order inside their group; ties
  in free space go to the earliest row;
* in-order rows are measured on the same global segments (a row's union of
  global segments equals the size of a trie rebuilt for that row alone);
* a sequence longer than a row is an error.
"""

from __future__ import annotations

from dataclasses import dataclass
from typing import List

import numpy as np


@dataclass
class Segments:
    seg_of_node: np.ndarray        # [n_nodes] segment id (segments numbered by first node)
    seg_len: np.ndarray            # [n_segments] nodes per segment
    paths: List[List[int]]         # per sequence: segment ids root to leaf


def segments(parent, seq_last) -> Segments:
    parent = np.asarray(parent, dtype=np.int64)
    n = len(parent)
    kids = np.zeros(n, dtype=np.int64)
    for v in range(n):
        if parent[v] >= 0:
            kids[parent[v]] += 1
    ends = np.zeros(n, dtype=bool)
    for x in seq_last:
        if x >= 0:
            ends[x] = True
    # nodes are in DFS pre-order (parent before child), so one pass suffices
    seg_of = np.full(n, -1, dtype=np.int64)
    lens: List[int] = []
    for v in range(n):
        p = parent[v]
        if p < 0 or kids[p] > 1 or ends[p]:
            seg_of[v] = len(lens)
            lens.append(0)
        else:
            seg_of[v] = seg_of[p]
        lens[seg_of[v]] += 1
    first = {}
    for v in range(n):
        first.setdefault(int(seg_of[v]), v)
    paths = []
    for x in seq_last:
        path = []
        v = int(x)
        while v >= 0:
            sg = int(seg_of[v])
            path.append(sg)
            v = int(parent[first[sg]])
        paths.append(path[::-1])
    return Segments(seg_of_node=seg_of, seg_len=np.asarray(lens, dtype=np.int64), paths=paths)


@dataclass
class Placement:
    bin_of_seq: np.ndarray         # [n_seqs] row of each sequence
    bin_tokens: np.ndarray         # [n_bins] tokens each row holds (union of its segments)


def place_leaves(segs: Segments, group, seq_len: int, mode: str = "global") -> Placement:
    paths = segs.paths
    L = segs.seg_len
    n = len(paths)
    cost = [int(sum(L[s] for s in p)) for p in paths]
    for s in range(n):
        if cost[s] > seq_len:
            raise ValueError(f"sequence {s} needs {cost[s]} tokens, more than a row of {seq_len}")
    bins_segs: List[set] = []
    bins_tok: List[int] = []
    where = np.full(n, -1, dtype=np.int64)

    def delta(b, s):
        return sum(int(L[x]) for x in paths[s] if x not in bins_segs[b])

    def add(b, s):
        bins_tok[b] += delta(b, s)
        bins_segs[b].update(paths[s])
        where[s] = b

    def new_bin():
        bins_segs.append(set())
        bins_tok.append(0)
        return len(bins_tok) - 1

    if mode == "in_order":
        cur = -1
        for s in range(n):
            if cur < 0 or bins_tok[cur] + delta(cur, s) > seq_len:
                cur = new_bin()
            add(cur, s)
    elif mode == "global":
        groups: dict = {}
        for s in range(n):
            groups.setdefault(int(group[s]), []).append(s)
        ordered = sorted(groups.values(), key=lambda g: max(cost[s] for s in g), reverse=True)
        for g in ordered:
            for s in g:
                best, best_free = -1, seq_len + 1
                for b in range(len(bins_tok)):
                    c = bins_tok[b] + delta(b, s)
                    if c <= seq_len and seq_len - c < best_free:
                        best, best_free = b, seq_len - c
                if best < 0:
                    best = new_bin()
                add(best, s)
    else:
        raise ValueError(mode)
    return Placement(bin_of_seq=where, bin_tokens=np.asarray(bins_tok, dtype=np.int64))


# ---------------------------------------------------------------------------
# [TRL "How tree packing works"]: the planner grows the trie sample by sample,
# and token_budget bounds a row's unique (forwarded) tokens, not its raw ones;
# [TRL "Limits and caveats to know before you switch"]: fork_threshold_tokens
# (1024 by default) decides how much of a prefix must be common before samples
# share it.  Readings (listed in the design doc): samples are taken in arrival
# order; a sample joins the open row when the trie of the row plus the sample
# holds at most token_budget nodes, else the row is closed for good and the
# sample opens the next one; the trie is the one of oracle.trie with the fork
# threshold as its minimum shared run (a common run shorter than the
# threshold is not shared; a shared one gives each branch its join copy); a
# sample longer than token_budget is an error.  fork_frac is the share of
# samples whose path shares a node with another sample of their row.
# ---------------------------------------------------------------------------

@dataclass
class GrownRows:
    row_of_seq: np.ndarray         # [n_seqs] row of each sample
    row_tokens: np.ndarray         # [n_rows] forwarded tokens (trie nodes) of each row
    forked: np.ndarray             # [n_seqs] 1 if the sample shares a node with another sample of its row


def grow_rows(sequences, token_budget: int, fork_threshold: int = 1024) -> GrownRows:
    from .trie import build_trie

    thr = max(1, int(fork_threshold))
    n = len(sequences)
    row_of = np.full(n, -1, dtype=np.int64)
    rows: List[List[int]] = []
    tokens: List[int] = []
    cur: List[int] = []
    cur_tokens = 0
    for s in range(n):
        if len(sequences[s]) > token_budget:
            raise ValueError(f"sample {s} has {len(sequences[s])} tokens, more than the budget {token_budget}")
        cand = cur + [s]
        t = build_trie([sequences[i] for i in cand], min_shared=thr).n_nodes
        if t <= token_budget:
            cur, cur_tokens = cand, t
        else:
            rows.append(cur)
            tokens.append(cur_tokens)
            cur, cur_tokens = [s], len(sequences[s])
    if cur:
        rows.append(cur)
        tokens.append(cur_tokens)
    forked = np.zeros(n, dtype=np.int64)
    for r, members in enumerate(rows):
        row_of[members] = r
        trie = build_trie([sequences[i] for i in members], min_shared=thr)
        users = np.zeros(trie.n_nodes, dtype=np.int64)
        for p in trie.paths:
            users[np.unique(np.asarray(p, dtype=np.int64))] += 1
        for k, i in enumerate(members):
            p = np.asarray(trie.paths[k], dtype=np.int64)
            forked[i] = int(len(p) > 0 and bool(np.any(users[p] > 1)))
    return GrownRows(row_of_seq=row_of, row_tokens=np.asarray(tokens, dtype=np.int64), forked=forked)
