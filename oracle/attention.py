"""Oracle steps 5-6: attention over a packed tree, by its plain definition.

A token of a packed row attends only to itself and its root-to-leaf
ancestors [ART "Token-mixing layers"; DAG "The mask"].  Unpacked, that is
ordinary causal attention on every root-to-leaf sequence, so the oracle
computes exactly that, sequence by sequence, and maps the results back
through token_index [TRL "How tree packing works"]:

* forward: per sequence s and query head h (KV head g = h // (Hq/Hkv)),
  S = scale * Q K^T with keys after the query masked, lse = log sum exp(S)
  (natural log), P = exp(S - lse), O = P V;
* backward: the exact gradient of L = sum over packed slots of
  <dout[slot], out[slot]>.  Each slot is counted once: it is owned by the
  first sequence (input order) whose path contains it; that sequence's row
  gets dout[slot], the other sequences through the slot get zero.  Per
  sequence: delta = rowsum(dO * O), dP = dO V^T, dS = P * (dP - delta),
  dQ = scale dS K, dK = scale dS^T Q, dV = P^T dO; dK, dV are summed over
  the query heads of each KV head and scattered back into packed slots.

Readings: scale 1/sqrt(D); lse in natural log; GQA groups are contiguous.
Rows are processed in chunks only to bound memory: each row is computed
exactly as the definition says, independently of the others.
"""

from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import numpy as np

from .layout import Layout, dfs_layout
from .precision import round_to
from .rope import rope
from .trie import Trie, build_trie

CHUNK = 1024


def causal_forward(Q, K, V, scale, rows=None):
    """Q [L,Hq,D], K/V [L,Hkv,D] -> (O [R,Hq,D], lse [Hq,R]) for query rows ``rows`` (default all)."""
    L, Hq, D = Q.shape
    G = Hq // K.shape[1]
    rows = np.arange(L) if rows is None else np.asarray(rows, dtype=np.int64)
    O = np.empty((len(rows), Hq, D))
    lse = np.empty((Hq, len(rows)))
    for c0 in range(0, len(rows), CHUNK):
        r = rows[c0:c0 + CHUNK]
        kmax = int(r.max()) + 1
        later = np.arange(kmax)[None, :] > r[:, None]
        for h in range(Hq):
            g = h // G
            S = scale * (Q[r, h] @ K[:kmax, g].T)
            S[later] = -np.inf
            m = S.max(axis=1)
            l = m + np.log(np.exp(S - m[:, None]).sum(axis=1))
            P = np.exp(S - l[:, None])
            O[c0:c0 + len(r), h] = P @ V[:kmax, g]
            lse[h, c0:c0 + len(r)] = l
    return O, lse


def causal_backward(Q, K, V, dO, scale, rows=None):
    """Gradient of sum(dO * O) for causal attention, from query rows ``rows`` (default all).

    Returns dQ [R,Hq,D] for those rows and dK, dV [L,Hkv,D] summed over
    them.  Rows left out must have dO == 0 for dK, dV to be complete.
    """
    L, Hq, D = Q.shape
    Hkv = K.shape[1]
    G = Hq // Hkv
    rows = np.arange(L) if rows is None else np.asarray(rows, dtype=np.int64)
    dQ = np.zeros((len(rows), Hq, D))
    dK = np.zeros((L, Hkv, D))
    dV = np.zeros((L, Hkv, D))
    for c0 in range(0, len(rows), CHUNK):
        r = rows[c0:c0 + CHUNK]
        kmax = int(r.max()) + 1
        later = np.arange(kmax)[None, :] > r[:, None]
        for h in range(Hq):
            g = h // G
            S = scale * (Q[r, h] @ K[:kmax, g].T)
            S[later] = -np.inf
            m = S.max(axis=1)
            l = m + np.log(np.exp(S - m[:, None]).sum(axis=1))
            P = np.exp(S - l[:, None])
            O = P @ V[:kmax, g]
            dOr = dO[r, h]
            delta = (dOr * O).sum(axis=1)
            dP = dOr @ V[:kmax, g].T
            dS = P * (dP - delta[:, None])
            dQ[c0:c0 + len(r), h] = scale * (dS @ K[:kmax, g])
            dK[:kmax, g] += scale * (dS.T @ Q[r, h])
            dV[:kmax, g] += P.T @ dOr
    return dQ, dK, dV


@dataclass
class TreeResult:
    trie: Trie
    layout: Layout
    owner: np.ndarray        # [n_nodes] sequence owning each slot
    out: np.ndarray          # [row_len, Hq, D] (NaN where not computed)
    lse: np.ndarray          # [Hq, row_len]
    dq: Optional[np.ndarray]
    dk: Optional[np.ndarray]
    dv: Optional[np.ndarray]
    max_shared_gap: float    # largest disagreement between sequences sharing a slot


def slot_owners(token_index, n_nodes):
    owner = np.full(n_nodes, -1, dtype=np.int64)
    for s, ti in enumerate(token_index):
        new = ti[owner[ti] < 0]
        owner[new] = s
    return owner


def tree_attention(sequences, fid, dkey, tables, *, theta: Optional[float], min_shared: int = 64,
                   row_len: Optional[int] = None, backward: bool = True, scale: Optional[float] = None,
                   q_slots=None, k_slots=None, storage: Optional[str] = None, kv_heads=None) -> TreeResult:
    """The whole oracle path: trie, layout, RoPE at depth, per-sequence attention, map back.

    ``tables`` holds q [n_feat,Hq,D], k/v [n_feat,Hkv,D] and do [n_dkey,Hq,D];
    token t of sequence s reads row fid[s][t] (q/k/v) and dkey[s][t] (do).
    By default every row of every sequence is computed.  ``q_slots`` /
    ``k_slots`` restrict the work to what out/lse/dq at ``q_slots`` and
    dk/dv at ``k_slots`` need (each of those outputs is still exact).
    ``theta`` None applies no rotary embedding.  ``storage`` ("f32" or "bf16") rounds the rotated q and k once to the
    dtype of the tensors that hold them; everything else stays fp64.  ``kv_heads`` (a list of KV heads)
    computes only those heads and the query heads that read them (whole GQA groups, so dk/dv of those
    heads are complete); the other heads' outputs are NaN.
    """
    trie = build_trie(sequences, min_shared=min_shared)
    n = trie.n_nodes
    layout = dfs_layout(trie.parent, trie.seq_last, n if row_len is None else row_len)
    ti = layout.token_index
    owner = slot_owners(ti, n)
    qt, kt, vt = tables["q"], tables["k"], tables["v"]
    Hq, D = qt.shape[1], qt.shape[2]
    Hkv = kt.shape[1]
    G = Hq // Hkv
    kvh = np.arange(Hkv) if kv_heads is None else np.asarray(sorted(set(int(g) for g in kv_heads)), dtype=np.int64)
    qh = (kvh[:, None] * G + np.arange(G)[None, :]).ravel()   # the query heads of those groups
    scale = 1.0 / np.sqrt(D) if scale is None else scale
    R = layout.row_len
    sampled = q_slots is not None or k_slots is not None
    want_q = np.zeros(R, dtype=bool)
    want_k = np.zeros(R, dtype=bool)
    if sampled:
        if q_slots is not None:
            want_q[np.asarray(q_slots, dtype=np.int64)] = True
        if k_slots is not None:
            want_k[np.asarray(k_slots, dtype=np.int64)] = True
    out = np.full((R, Hq, D), np.nan)
    lse = np.full((Hq, R), np.nan)
    dq = np.full((R, Hq, D), np.nan) if backward else None
    dk = np.zeros((R, Hkv, D)) if backward else None
    dv = np.zeros((R, Hkv, D)) if backward else None
    gap = 0.0
    for s, seq in enumerate(sequences):
        L = len(seq)
        if L == 0:
            continue
        slots = ti[s]
        pos = np.arange(L)
        if theta is None:                      # no rotary embedding
            Qs = np.asarray(qt[fid[s]][:, qh], dtype=np.float64)
            Ks = np.asarray(kt[fid[s]][:, kvh], dtype=np.float64)
        else:
            Qs = round_to(rope(qt[fid[s]][:, qh], pos, theta), storage)
            Ks = round_to(rope(kt[fid[s]][:, kvh], pos, theta), storage)
        Vs = np.asarray(vt[fid[s]][:, kvh], dtype=np.float64)
        owned = owner[slots] == s
        if sampled:
            fwd_rows = np.nonzero(owned & want_q[slots])[0]
        else:
            fwd_rows = pos
        if len(fwd_rows):
            O, l = causal_forward(Qs, Ks, Vs, scale, fwd_rows)
            dst = slots[fwd_rows]
            done = ~np.isnan(out[dst, qh[0], 0])
            if np.any(done):
                gap = max(gap, float(np.max(np.abs(out[dst[done]][:, qh] - O[done]))),
                          float(np.max(np.abs(lse[qh][:, dst[done]] - l[:, done]))))
            out[dst[:, None], qh[None, :]] = O
            lse[qh[:, None], dst[None, :]] = l
        if not backward:
            continue
        dOs = np.zeros((L, len(qh), D))
        dOs[owned] = tables["do"][dkey[s][owned]][:, qh]
        if sampled:
            kpos = np.nonzero(want_k[slots])[0]
            kmin = int(kpos.min()) if len(kpos) else L
            need = owned & (want_q[slots] | (pos >= kmin))
            bwd_rows = np.nonzero(need)[0]
        else:
            bwd_rows = pos
        if len(bwd_rows) == 0:
            continue
        dQ, dK, dV = causal_backward(Qs, Ks, Vs, dOs, scale, bwd_rows)
        own_rows = owned[bwd_rows]
        dq[slots[bwd_rows[own_rows]][:, None], qh[None, :]] = dQ[own_rows]
        dk_s = np.zeros((L, Hkv, D))
        dv_s = np.zeros((L, Hkv, D))
        dk_s[:, kvh] = dK
        dv_s[:, kvh] = dV
        np.add.at(dk, slots, dk_s)
        np.add.at(dv, slots, dv_s)
    if backward and kv_heads is not None:
        other = np.setdiff1d(np.arange(Hkv), kvh)
        dk[:, other] = np.nan
        dv[:, other] = np.nan
    if backward and sampled:
        keep = np.zeros(R, dtype=bool)
        keep[np.asarray(k_slots if k_slots is not None else [], dtype=np.int64)] = True
        dk[~keep] = np.nan
        dv[~keep] = np.nan
    if backward and not sampled:
        dq[n:] = np.nan
        dk[n:] = np.nan
        dv[n:] = np.nan
    return TreeResult(trie=trie, layout=layout, owner=owner, out=out, lse=lse, dq=dq, dk=dk, dv=dv,
                      max_shared_gap=gap)
