"""Oracle step 3: token counts of a packed row.

[TRL "How tree packing works"]: raw tokens are summed over the unpacked
sequences, forwarded tokens are the packed ones, and raw / forwarded is the
packing ratio.  [TRL "A back-of-envelope example"] counts distinct prefix
tokens (a token shared by several samples counted once, join copies not
added), so that count is reported too, from a plain dictionary trie.
[TRL "How to evaluate it on your own workload"] names row fill and fork
fraction; readings: row fill = forwarded / row length, fork fraction = share
of sequences whose path shares at least one slot with another sequence.
"""

from __future__ import annotations

import numpy as np


def distinct_prefixes(sequences) -> int:
    """Number of distinct non-empty prefixes: nodes of an uncompressed token trie."""
    root: dict = {}
    count = 0
    for s in sequences:
        node = root
        for tok in np.asarray(s).tolist():
            nxt = node.get(tok)
            if nxt is None:
                nxt = {}
                node[tok] = nxt
                count += 1
            node = nxt
    return count


def packing_counts(sequences, token_index, row_len: int) -> dict:
    raw = int(sum(len(s) for s in sequences))
    slots = np.concatenate([np.asarray(ti) for ti in token_index]) if token_index else np.zeros(0)
    forwarded = int(len(np.unique(slots)))
    use = np.bincount(slots.astype(np.int64), minlength=max(row_len, 1)) if len(slots) else np.zeros(1)
    forked = sum(1 for ti in token_index if len(ti) and np.any(use[np.asarray(ti)] > 1))
    return {
        "raw": raw,
        "forwarded": forwarded,
        "distinct_prefixes": distinct_prefixes(sequences),
        "packing_ratio": raw / forwarded if forwarded else float("nan"),
        "row_fill": forwarded / row_len if row_len else float("nan"),
        "fork_frac": forked / len(token_index) if token_index else float("nan"),
    }
