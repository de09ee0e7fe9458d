"""Seeded synthetic workloads for attention over prefix-tree-packed rows.

This module only makes inputs.  A workload is described the way the pages
describe their batches: a set of token sequences that share prefixes
(a GRPO group sharing one prompt, agentic rollouts branching from a common
history, independent documents).  It is generated as a tree of *segments*
(runs of fresh random tokens hanging off a parent segment); every
root-to-leaf chain of segments is one sequence.  Nothing here builds the
packed trie, lays out a row or computes attention: both the library and the
oracle receive only the sequences plus the per-token tensors below, and
derive everything else on their own.

Per-token tensors stand in for the activations of a causal model:

* q/k/v of a token depend only on its prefix (a causal model gives one
  hidden state per distinct prefix).  ``fid[s][t]`` is the row of the
  feature tables for the prefix ``seq[s][:t+1]``; since sibling segments
  start with distinct tokens, distinct (segment, offset) pairs are distinct
  prefixes.
* the upstream gradient at a token depends on its prefix *and* on what it
  is trained to predict next (its target), as with a next-token loss.
  ``dkey[s][t]`` is the row of the gradient table for (prefix, next token),
  with one extra row per sequence end.

Random numbers: NumPy PCG64.  Tree seed ``1000*c``, q/k/v/dout tables from
``1000*c + 1 .. 4``.  Values are N(0, 1); bf16 workloads round them to the
nearest bf16 (ties to even) and keep them as float32 so every consumer reads
exactly the same numbers.
"""

from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np

TOKEN_HIGH = 2**31  # token ids are uniform in [0, 2**31)


@dataclass
class Workload:
    name: str
    sequences: List[np.ndarray]          # int32 token ids, one array per sequence
    fid: List[np.ndarray]                # int64 feature row of each token's prefix
    dkey: List[np.ndarray]               # int64 gradient row of each (prefix, next token)
    n_feat: int
    n_dkey: int
    Hq: int
    Hkv: int
    D: int
    dtype: str                           # "f32" or "bf16"
    row_len: Optional[int]               # None: pad the packed count to a multiple of row_multiple
    row_multiple: int = 64
    theta: float = 10000.0
    backward: bool = True
    seed_base: int = 0
    notes: dict = field(default_factory=dict)

    @property
    def raw_tokens(self) -> int:
        return int(sum(len(s) for s in self.sequences))

    def row_length(self, n_forwarded: int) -> int:
        """Row capacity for a packed count (the fixed row of the workload, or padding to a multiple)."""
        if self.row_len is not None:
            return self.row_len
        m = self.row_multiple
        return ((n_forwarded + m - 1) // m) * m


# --------------------------------------------------------------------------
# helpers
# --------------------------------------------------------------------------

def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even); returns float32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    u = (u + 0x7FFF + lsb) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32)


class _SegmentTree:
    """Segments of fresh tokens; children of one parent start with distinct tokens."""

    def __init__(self, rng: np.random.Generator):
        self.rng = rng
        self.parent: List[int] = []
        self.tokens: List[np.ndarray] = []
        self.children: List[List[int]] = []

    def first_tokens(self, k: int) -> np.ndarray:
        while True:
            t = self.rng.integers(0, TOKEN_HIGH, size=k, dtype=np.int64)
            if len(set(t.tolist())) == k:
                return t

    def add(self, parent: int, length: int, first: Optional[int] = None) -> int:
        toks = self.rng.integers(0, TOKEN_HIGH, size=length, dtype=np.int64)
        if first is not None and length > 0:
            toks[0] = first
        sid = len(self.tokens)
        self.parent.append(parent)
        self.tokens.append(toks.astype(np.int32))
        self.children.append([])
        if parent >= 0:
            self.children[parent].append(sid)
        return sid

    def add_children(self, parent: int, lengths) -> List[int]:
        firsts = self.first_tokens(len(lengths))
        return [self.add(parent, int(L), int(f)) for L, f in zip(lengths, firsts)]

    def to_sequences(self):
        """Root-to-leaf token sequences, feature rows and gradient rows (leaves in creation order)."""
        base = np.zeros(len(self.tokens) + 1, dtype=np.int64)
        for i, t in enumerate(self.tokens):
            base[i + 1] = base[i] + len(t)
        n_feat = int(base[-1])
        seqs, fids, dkeys = [], [], []
        leaves = [i for i in range(len(self.tokens)) if not self.children[i]]
        for li, leaf in enumerate(leaves):
            chain = []
            s = leaf
            while s >= 0:
                chain.append(s)
                s = self.parent[s]
            chain.reverse()
            toks = np.concatenate([self.tokens[c] for c in chain])
            fid = np.concatenate([base[c] + np.arange(len(self.tokens[c]), dtype=np.int64) for c in chain])
            dk = np.empty_like(fid)
            dk[:-1] = fid[1:]             # (prefix, next token) == prefix one longer
            dk[-1] = n_feat + li          # end of this sequence
            seqs.append(toks)
            fids.append(fid)
            dkeys.append(dk)
        return seqs, fids, dkeys, n_feat, n_feat + len(leaves)


def _finish(name, tree, Hq, Hkv, D, dtype, row_len, seed_base, backward=True, theta=10000.0, notes=None):
    seqs, fids, dkeys, n_feat, n_dkey = tree.to_sequences()
    return Workload(name=name, sequences=seqs, fid=fids, dkey=dkeys, n_feat=n_feat, n_dkey=n_dkey,
                    Hq=Hq, Hkv=Hkv, D=D, dtype=dtype, row_len=row_len, theta=theta,
                    backward=backward, seed_base=seed_base, notes=notes or {})


# --------------------------------------------------------------------------
# the five workloads (sizes are parameters so tests can shrink them)
# --------------------------------------------------------------------------

def tiny_tree(seed_base: int = 1000, n_seqs: int = 8, prefix: int = 128, mid: int = 72,
              leaf_lo: int = 32, leaf_hi: int = 96, Hq: int = 2, Hkv: int = 2, D: int = 64,
              dtype: str = "f32") -> Workload:
    """8 sequences: a shared prefix, two groups that each share a middle run, then leaves.

    The prefix forks into two groups of at least two sequences (random split);
    each group shares ``mid`` more tokens and then forks into its leaves of
    U[leaf_lo, leaf_hi] tokens.  fp32, forward only, depth RoPE theta 10000.
    """
    rng = np.random.Generator(np.random.PCG64(seed_base))
    tree = _SegmentTree(rng)
    root = tree.add(-1, prefix)
    n0 = int(rng.integers(2, n_seqs - 1))
    groups = tree.add_children(root, [mid, mid])
    for g, n in zip(groups, (n0, n_seqs - n0)):
        tree.add_children(g, rng.integers(leaf_lo, leaf_hi + 1, size=n))
    return _finish("tiny_tree", tree, Hq, Hkv, D, dtype, None, seed_base, backward=False)


def grpo_group(seed_base: int = 2000, prompt: int = 2048, n: int = 16, completion: int = 1024,
               Hq: int = 16, Hkv: int = 8, D: int = 128, dtype: str = "bf16",
               row_len: Optional[int] = 32768) -> Workload:
    """A GRPO group: ``n`` rollouts sharing one prompt, each with its own completion."""
    rng = np.random.Generator(np.random.PCG64(seed_base))
    tree = _SegmentTree(rng)
    root = tree.add(-1, prompt)
    tree.add_children(root, [completion] * n)
    return _finish("grpo_group", tree, Hq, Hkv, D, dtype, row_len, seed_base)


def _agentic_tree(seed: int, budget: int, seg_lo: int, seg_hi: int, p_fork: float,
                  kid_lo: int, kid_hi: int):
    """Depth-first growth of a random branching history.

    Segment lengths are U[seg_lo, seg_hi]; at the end of a segment it forks
    with probability ``p_fork`` into U{kid_lo..kid_hi} children, else it is a
    leaf; the root always forks.  Growth stops when the row budget is used,
    truncating the last segment.  A row of ``budget`` slots holds the segment
    tokens plus one slot per branch that hangs off a fork (the copy of the
    token the branch joins at).
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    tree = _SegmentTree(rng)
    used = 0
    root_len = int(rng.integers(seg_lo, seg_hi + 1))
    root_len = min(root_len, budget)
    root = tree.add(-1, root_len)
    used += root_len
    stack = []  # (parent, first token) of segments still to grow, depth first

    def fork(parent, always=False):
        if always or rng.random() < p_fork:
            k = int(rng.integers(kid_lo, kid_hi + 1))
            firsts = tree.first_tokens(k)
            for f in reversed(firsts.tolist()):
                stack.append((parent, f))

    fork(root, always=True)
    while stack and used < budget:
        parent, first = stack.pop()
        L = int(rng.integers(seg_lo, seg_hi + 1))
        room = budget - used - 1          # one slot for this branch's copy of the join token
        if room <= 0:
            break
        L = min(L, room)
        sid = tree.add(parent, L, first)
        used += L + 1
        if used < budget:
            fork(sid)
    return tree, used


def agentic_trie(seed_start: int = 3000, budget: int = 32768, seg_lo: int = 64, seg_hi: int = 2048,
                 p_fork: float = 0.5, kid_lo: int = 2, kid_hi: int = 4, ratio_lo: float = 4.1,
                 ratio_hi: float = 4.3, Hq: int = 16, Hkv: int = 8, D: int = 128, dtype: str = "bf16",
                 row_len: Optional[int] = 32768, seed_base: int = 3000, max_scan: int = 2000) -> Workload:
    """Agentic multi-turn trie: the first seed from ``seed_start`` whose raw/row ratio is in range."""
    for seed in range(seed_start, seed_start + max_scan):
        tree, used = _agentic_tree(seed, budget, seg_lo, seg_hi, p_fork, kid_lo, kid_hi)
        seqs, _, _, _, _ = tree.to_sequences()
        raw = sum(len(s) for s in seqs)
        ratio = raw / used
        if ratio_lo <= ratio <= ratio_hi:
            w = _finish("agentic_trie", tree, Hq, Hkv, D, dtype, row_len, seed_base,
                        notes={"tree_seed": seed, "slots_budgeted": used, "ratio_budgeted": ratio})
            return w
    raise RuntimeError("no seed in the scanned range gives the requested ratio")


def independent(seed_base: int = 4000, n: int = 64, length: int = 512, Hq: int = 16, Hkv: int = 8,
                D: int = 128, dtype: str = "bf16", row_len: Optional[int] = 32768) -> Workload:
    """``n`` independent sequences with distinct first tokens: nothing is shared."""
    rng = np.random.Generator(np.random.PCG64(seed_base))
    tree = _SegmentTree(rng)
    firsts = tree.first_tokens(n)
    for f in firsts.tolist():
        tree.add(-1, length, f)
    return _finish("independent", tree, Hq, Hkv, D, dtype, row_len, seed_base)


def long_history(seed_base: int = 5000, prefix: int = 20000, n: int = 8, unique: int = 2000,
                 Hq: int = 32, Hkv: int = 8, D: int = 128, dtype: str = "bf16",
                 row_len: Optional[int] = 36864) -> Workload:
    """A long shared history followed by ``n`` rollouts of ``unique`` tokens each."""
    rng = np.random.Generator(np.random.PCG64(seed_base))
    tree = _SegmentTree(rng)
    root = tree.add(-1, prefix)
    tree.add_children(root, [unique] * n)
    return _finish("long_history", tree, Hq, Hkv, D, dtype, row_len, seed_base)


def shared_history(prefix: int, n: int = 8, unique: int = 2000, seed_base: int = 7000, Hq: int = 16,
                   Hkv: int = 8, D: int = 128, dtype: str = "bf16") -> Workload:
    """``n`` rollouts of ``unique`` tokens after a shared history of ``prefix`` tokens (none if 0).

    The packing ratio is n (prefix + unique) / (prefix + n unique), plus the join copies; rows
    are padded to a multiple of 64.  prefix 20000, n 8, unique 2000 is the agent-history
    example of [explainx.ai on TRL tree packing, "A back-of-envelope example"] (ratio 4.9).
    """
    rng = np.random.Generator(np.random.PCG64(seed_base + prefix))
    tree = _SegmentTree(rng)
    if prefix > 0:
        root = tree.add(-1, prefix)
        tree.add_children(root, [unique] * n)
    else:
        for f in tree.first_tokens(n).tolist():
            tree.add(-1, unique, f)
    return _finish(f"shared_history_p{prefix}", tree, Hq, Hkv, D, dtype, None, seed_base + prefix)


def sequence_packing_forest(sequences):
    """Parent array and last node of every sequence when nothing is shared: one chain per sequence.

    Node ids run through the sequences in order (sequence s holds ids o_s .. o_s + len_s - 1, its
    first token a root, each later token the child of the one before).  Laid out depth first,
    this is plain sequence packing: each token attends to the tokens before it in its own
    sequence and positions restart at 0 in every sequence.
    """
    lens = np.array([len(s) for s in sequences], dtype=np.int64)
    total = int(lens.sum())
    parent = np.arange(-1, total - 1, dtype=np.int64)
    starts = np.concatenate([[0], np.cumsum(lens)[:-1]]) if len(lens) else np.zeros(0, np.int64)
    parent[starts[lens > 0]] = -1
    seq_last = np.where(lens > 0, starts + lens - 1, -1)
    return parent.astype(np.int32), seq_last.astype(np.int32)


def from_sequences(sequences, *, Hq: int, Hkv: int, D: int, dtype: str, seed_base: int,
                   row_len: Optional[int] = None, backward: bool = True, theta: float = 10000.0,
                   name: str = "custom") -> Workload:
    """A workload from explicit token sequences (any overlap pattern, e.g. a tiny vocabulary).

    Feature rows are assigned per distinct prefix and gradient rows per
    distinct (prefix, next token or end), with plain dictionaries.
    """
    seqs = [np.asarray(s, dtype=np.int32) for s in sequences]
    pre: dict = {}
    nxt: dict = {}
    fids, dkeys = [], []
    for s in seqs:
        toks = s.tolist()
        f = np.empty(len(toks), dtype=np.int64)
        d = np.empty(len(toks), dtype=np.int64)
        for t in range(len(toks)):
            f[t] = pre.setdefault(tuple(toks[:t + 1]), len(pre))
            key = tuple(toks[:t + 2]) if t + 1 < len(toks) else (tuple(toks), "end")
            d[t] = nxt.setdefault(key, len(nxt))
        fids.append(f)
        dkeys.append(d)
    return Workload(name=name, sequences=seqs, fid=fids, dkey=dkeys, n_feat=max(len(pre), 1),
                    n_dkey=max(len(nxt), 1), Hq=Hq, Hkv=Hkv, D=D, dtype=dtype, row_len=row_len,
                    theta=theta, backward=backward, seed_base=seed_base)


def standard(c: int) -> Workload:
    """The five workloads at their full sizes (c = 1..5)."""
    if c == 1:
        return tiny_tree()
    if c == 2:
        return grpo_group()
    if c == 3:
        return agentic_trie()
    if c == 4:
        return independent()
    if c == 5:
        return long_history()
    raise ValueError(c)


# --------------------------------------------------------------------------
# per-token tensors
# --------------------------------------------------------------------------

def feature_tables(w: Workload, which=("q", "k", "v", "do")) -> dict:
    """N(0,1) tables: q [n_feat,Hq,D], k/v [n_feat,Hkv,D], do [n_dkey,Hq,D] (float32).

    Seeds are ``seed_base + 1..4`` for q, k, v, do; bf16 workloads round to bf16.
    """
    shapes = {"q": (w.n_feat, w.Hq, w.D), "k": (w.n_feat, w.Hkv, w.D),
              "v": (w.n_feat, w.Hkv, w.D), "do": (w.n_dkey, w.Hq, w.D)}
    offs = {"q": 1, "k": 2, "v": 3, "do": 4}
    out = {}
    for name in which:
        rng = np.random.Generator(np.random.PCG64(w.seed_base + offs[name]))
        x = rng.standard_normal(shapes[name], dtype=np.float32)
        if w.dtype == "bf16":
            x = round_bf16(x)
        out[name] = x
    return out


def curriculum_batch(n_groups: int, seed: int = 6000, n_system: int = 4, system_len: int = 4096,
                     prefix_lo: int = 2000, prefix_hi: int = 16000, group_lo: int = 4, group_hi: int = 13,
                     comp_lo: int = 4000, comp_hi: int = 28000):
    """A multi-task batch for the row planner: ``n_groups`` RL groups, each a task prefix under one
    of ``n_system`` shared system prompts, with U{group_lo..group_hi} trainable completions.

    Returns (sequences, trainable flags, group id per sequence).  Token ids are fresh random
    values, so sharing comes only from the stated structure.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    systems = [rng.integers(0, TOKEN_HIGH, size=system_len, dtype=np.int64).astype(np.int32)
               for _ in range(n_system)]
    for i, s in enumerate(systems):
        s[0] = i            # distinct first tokens: the system prompts do not share a prefix
    seqs, train, group = [], [], []
    for g in range(n_groups):
        sysp = systems[int(rng.integers(0, n_system))]
        prefix = rng.integers(0, TOKEN_HIGH, size=int(rng.integers(prefix_lo, prefix_hi + 1)),
                              dtype=np.int64).astype(np.int32)
        for _ in range(int(rng.integers(group_lo, group_hi + 1))):
            comp = rng.integers(0, TOKEN_HIGH, size=int(rng.integers(comp_lo, comp_hi + 1)),
                                dtype=np.int64).astype(np.int32)
            seqs.append(np.concatenate([sysp, prefix, comp]))
            t = np.zeros(len(seqs[-1]), dtype=bool)
            t[len(sysp) + len(prefix):] = True
            train.append(t)
            group.append(g)
    return seqs, train, np.asarray(group, dtype=np.int32)


def gdn_tables(w: Workload, Hk: int = 16, Hv: int = 32, dk: int = 128, dv: int = 128, conv_width: int = 4) -> dict:
    """Inputs of a gated-delta-rule mixing layer for a workload, per distinct prefix.

    x [n_feat, 2*Hk*dk + Hv*dv] ~ N(0, 1) (channels q | k | v; bf16 workloads round to bf16);
    conv weights [C, conv_width] ~ N(0, 1/conv_width); log-decay g [n_feat, Hv] = -c_h u with
    u ~ U(0, 1) and c_h log-spaced over the value heads from 1e-4 (memory of ~10^4 tokens) to 0.5;
    beta [n_feat, Hv] = sigmoid(N(0, 1)).  g and beta are float32.  Seeds ``seed_base + 11..14``.
    """
    C = 2 * Hk * dk + Hv * dv
    rng = lambda i: np.random.Generator(np.random.PCG64(w.seed_base + i))  # noqa: E731
    x = rng(11).standard_normal((w.n_feat, C), dtype=np.float32)
    if w.dtype == "bf16":
        x = round_bf16(x)
    conv_w = (rng(12).standard_normal((C, conv_width)) / np.sqrt(conv_width)).astype(np.float32)
    c = np.exp(np.linspace(np.log(1e-4), np.log(0.5), Hv))
    g = (-c[None, :] * rng(13).random((w.n_feat, Hv))).astype(np.float32)
    beta = (1.0 / (1.0 + np.exp(-rng(14).standard_normal((w.n_feat, Hv))))).astype(np.float32)
    return {"x": x, "conv_w": conv_w, "g": g, "beta": beta}
