"""Oracle step 1: the packed trie built from token sequences.

Follows [ART "The tree"]: find the longest run every active sequence agrees
on, emit it once, then partition the rest by their next token and recurse on
each partition.  Two refinements from the same section:

* a shared run shorter than ``min_shared`` tokens (64 by default) is not
  shared: it is copied into every next-token partition, and sharing can
  resume deeper if a partition agrees for longer;
* at every fork each branch keeps its own copy of the last shared token (the
  join token), so each copy has its own query position to predict the
  branch's first own token [ART "The tree"; DAG "The walk": the last common
  node is copied once per child].

Trainable mode (``trainable`` given, one flag per token): [ART "The tree"]
keeps trainable tokens out of sharing, and gives each branch a duplicated
context token at its join point so that the branch's first own token has
its own prediction position.  Read literally:

* a shared run stops at the first position where any active sequence holds
  a trainable token (so trainable tokens are never shared, not even between
  identical sequences);
* at a fork, a branch whose next token is trainable gets its own copy of
  the join token; a branch whose next token is not trainable, and a
  sequence that ends at the fork, hang off the shared token itself;
* a sequence whose next token is trainable forms a branch of its own even
  when another sequence has the same token there.
This is the accounting of the pages' packing example ([ART "Does it
actually help?"]): a 4,096-token system prompt shared whole, 11,999 shared
group-prefix tokens and completion + 1 tokens per rollout.

Readings where the pages are silent (all listed in the design doc):
* the run length compared with ``min_shared`` is measured before the join
  token is split off (a 64-token run that forks stays shared: 63 shared
  tokens plus one copy per branch);
* partitions are visited in ascending order of their next token, stable in
  input order; sequences that end exactly where the others fork form their
  own partition, visited first, and get their own copy of the join token;
* identical sequences share one path.

Nodes are numbered in emission order, which is a depth-first pre-order.
"""

from __future__ import annotations

from dataclasses import dataclass
from typing import List

import numpy as np


@dataclass
class Trie:
    parent: np.ndarray          # [n_nodes] int64, -1 for a root
    token: np.ndarray           # [n_nodes] token id of each node
    paths: List[np.ndarray]     # per sequence: node id of each of its tokens
    seq_last: np.ndarray        # [n_seqs] node of each sequence's last token

    @property
    def n_nodes(self) -> int:
        return int(len(self.parent))


def build_trie(sequences, min_shared: int = 64, trainable=None) -> Trie:
    seqs = [np.asarray(s, dtype=np.int64) for s in sequences]
    if min_shared < 1:
        raise ValueError("min_shared must be >= 1")
    train = None
    if trainable is not None:
        train = [np.asarray(t, dtype=bool) for t in trainable]
        if len(train) != len(seqs) or any(len(t) != len(s) for t, s in zip(train, seqs)):
            raise ValueError("trainable flags must match the sequences")

    def is_train(s, t):
        return train is not None and bool(train[s][t])
    parent: List[int] = []
    token: List[int] = []
    paths = [np.full(len(s), -1, dtype=np.int64) for s in seqs]

    def emit(active, start, end, par):
        """One node per position in [start, end), shared by every sequence in ``active``."""
        if end <= start:
            return par
        first = len(parent)
        for t in range(start, end):
            token.append(int(seqs[active[0]][t]))
            parent.append(par if t == start else len(parent) - 1)
        for s in active:
            paths[s][start:end] = np.arange(first, first + (end - start))
        return len(parent) - 1

    def common_run_end(active, start):
        """Smallest end >= start where the active sequences stop agreeing (or the shortest ends,
        or, in trainable mode, any of them reaches a trainable token)."""
        m = min(len(seqs[s]) for s in active)
        ref = seqs[active[0]][start:m]
        end = m
        for s in active[1:]:
            diff = np.nonzero(seqs[s][start:m] != ref)[0]
            if len(diff):
                end = min(end, start + int(diff[0]))
        if train is not None:
            for s in active:
                tr = np.nonzero(train[s][start:end])[0]
                if len(tr):
                    end = min(end, start + int(tr[0]))
        return end

    def partitions(active, pos):
        """Split by the token at ``pos``; ended sequences first, then ascending token, stable.
        In trainable mode a sequence whose token at ``pos`` is trainable is a branch of its own."""
        ended = [s for s in active if len(seqs[s]) == pos]
        going = [s for s in active if len(seqs[s]) > pos]
        going.sort(key=lambda s: int(seqs[s][pos]))          # stable sort keeps input order
        parts = [ended] if ended else []
        i = 0
        while i < len(going):
            j = i
            while j < len(going) and seqs[going[j]][pos] == seqs[going[i]][pos]:
                j += 1
            shared = [s for s in going[i:j] if not is_train(s, pos)]
            if shared:
                parts.append(shared)
            parts.extend([s] for s in going[i:j] if is_train(s, pos))
            i = j
        return parts

    def walk(active, start, par):
        active = [s for s in active if len(seqs[s]) > start]
        if not active:
            return
        if len(active) == 1:                                  # a private leaf
            emit(active, start, len(seqs[active[0]]), par)
            return
        end = common_run_end(active, start)
        if end == start:                                      # no shared run: split by next token
            for part in partitions(active, start):
                walk(part, start, par)
            return
        if all(len(seqs[s]) == end for s in active):          # identical remainders: no fork
            emit(active, start, end, par)
            return
        if end - start >= min_shared and train is None:       # share the run, copy the join token
            node = emit(active, start, end - 1, par)
            for part in partitions(active, end):
                walk(part, end - 1, node)
        elif end - start >= min_shared:                       # trainable mode: copy where it is needed
            parts = partitions(active, end)
            copy = [len(seqs[p[0]]) > end and is_train(p[0], end) for p in parts]
            if any(copy):
                node = emit(active, start, end - 1, par)
                stay = [s for p, c in zip(parts, copy) if not c for s in p]
                join = emit(stay, end - 1, end, node) if stay else None
                for p, c in zip(parts, copy):
                    if c:
                        walk(p, end - 1, node)
                    else:
                        walk(p, end, join)
            else:
                node = emit(active, start, end, par)
                for p in parts:
                    walk(p, end, node)
        else:                                                 # too short to share: copy it per branch
            for part in partitions(active, end):
                walk(part, start, par)

    walk(list(range(len(seqs))), 0, -1)
    parent_a = np.asarray(parent, dtype=np.int64)
    seq_last = np.asarray([p[-1] if len(p) else -1 for p in paths], dtype=np.int64)
    return Trie(parent=parent_a, token=np.asarray(token, dtype=np.int64), paths=paths,
                seq_last=seq_last)
