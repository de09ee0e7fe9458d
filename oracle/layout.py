"""Oracle step 2: the DFS layout of a packed tree.

From a parent array (a forest; -1 marks a root) this lays the nodes out in
depth-first pre-order [TRL "How tree packing works": the collator lays
tokens out depth-first; DAG "The walk"], gives every slot its depth as
position id [DAG "Positions": the number of transitions from the root; TRL
same section], the last slot of its subtree (the exit half of the
pre-order/exit-order interval of [ART "Token-mixing layers"]), and a
token_index that maps every token of every sequence to its packed slot
[TRL "How tree packing works"].

Readings: children are visited in ascending node id; roots sit at depth 0;
slots past the last node are padding with position 0 and subtree end equal
to their own slot.
"""

from __future__ import annotations

from dataclasses import dataclass
from typing import List

import numpy as np


@dataclass
class Layout:
    slot_node: np.ndarray       # [row_len] node in each slot, -1 for padding
    node_slot: np.ndarray       # [n_nodes]
    pos_ids: np.ndarray         # [row_len] depth
    subtree_end: np.ndarray     # [row_len] last slot of the subtree, inclusive
    token_index: List[np.ndarray]  # per sequence: slot of each token
    n_nodes: int
    row_len: int


def dfs_layout(parent, seq_last, row_len: int) -> Layout:
    parent = np.asarray(parent, dtype=np.int64)
    n = len(parent)
    if row_len < n:
        raise ValueError("row shorter than the tree")
    if np.any((parent < -1) | (parent >= n)):
        raise ValueError("parent out of range")
    children = [[] for _ in range(n)]
    roots = []
    for v in range(n):
        if parent[v] < 0:
            roots.append(v)
        else:
            children[int(parent[v])].append(v)

    # pre-order with an explicit stack (trees here are tens of thousands deep)
    order = []
    stack = list(reversed(roots))
    seen = np.zeros(n, dtype=bool)
    while stack:
        v = stack.pop()
        if seen[v]:
            raise ValueError("not a forest")
        seen[v] = True
        order.append(v)
        stack.extend(reversed(children[v]))
    if len(order) != n:
        raise ValueError("not a forest: some nodes are on a cycle")

    node_slot = np.empty(n, dtype=np.int64)
    node_slot[np.asarray(order, dtype=np.int64)] = np.arange(n)

    depth = np.zeros(n, dtype=np.int64)
    for v in order:                      # a parent comes before its children
        if parent[v] >= 0:
            depth[v] = depth[parent[v]] + 1

    size = np.ones(n, dtype=np.int64)
    for v in reversed(order):            # children before their parent
        if parent[v] >= 0:
            size[parent[v]] += size[v]

    slot_node = np.full(row_len, -1, dtype=np.int64)
    slot_node[:n] = order
    pos_ids = np.zeros(row_len, dtype=np.int64)
    subtree_end = np.arange(row_len, dtype=np.int64)
    for s in range(n):
        v = slot_node[s]
        pos_ids[s] = depth[v]
        subtree_end[s] = s + size[v] - 1

    token_index = []
    for last in np.asarray(seq_last, dtype=np.int64):
        if last < 0:
            token_index.append(np.zeros(0, dtype=np.int64))
            continue
        path = []
        v = int(last)
        while v >= 0:
            path.append(node_slot[v])
            v = int(parent[v])
        token_index.append(np.asarray(path[::-1], dtype=np.int64))
    return Layout(slot_node=slot_node, node_slot=node_slot, pos_ids=pos_ids,
                  subtree_end=subtree_end, token_index=token_index, n_nodes=n, row_len=row_len)
