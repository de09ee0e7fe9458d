"""Oracle for gated-delta-rule token mixing (GDN) over a packed tree, by its plain definition.

Test infrastructure: only tests/, the smoke check and the bench's CPU
baseline use it; it shares no code with the library.

Over a packed tree a recurrent layer threads its state token by token along
every root-to-leaf path: the state forks where the path branches and starts
from zero at every root [ART "Token-mixing layers"].  Unpacked, that is the
layer run on each sequence by itself, which is what this oracle does; the
per-token results go back to packed slots through token_index, and tokens
that several sequences share must get the same value from each (checked).

The layer on one sequence (Gated DeltaNet: Yang, Kautz and Hatamizadeh,
"Gated Delta Networks: Improving Mamba2 with Delta Rule", 2024; the
mixing core with its short convolution, as [ART "Token-mixing layers"] runs
it in two calls, a causal convolution and the delta rule):

* input x_t has C = 2*Hk*dk + Hv*dv channels, ordered q | k | v;
* depthwise causal convolution of width W along the sequence with zeros
  before its first token, y_t[c] = sum_j w[c, W-1-j] x_{t-j}[c] (the last
  tap weighs the current token), then SiLU, y * sigmoid(y);
* q and k divided by their L2 norm per head (a zero vector stays zero),
  q then scaled by dk^-1/2;
* per value head h, key head h // (Hv/Hk), state S in R^{dv x dk}, S_0 = 0:
      S_t = alpha_t S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,
      alpha_t = exp(g_t),   o_t = S_t q_t.

``storage`` "bf16" models the one rounding of the kernel's stored q, k, v
(after normalisation and scaling) to bf16; everything else is fp64.
"""

from __future__ import annotations

from dataclasses import dataclass
from typing import Optional, Sequence

import numpy as np

from .layout import Layout, dfs_layout
from .precision import round_to
from .trie import Trie, build_trie


def conv_silu(x: np.ndarray, w: np.ndarray) -> np.ndarray:
    """x [T, C], w [C, W] -> SiLU(causal depthwise convolution) [T, C], zeros before token 0."""
    x = np.asarray(x, dtype=np.float64)
    T, C = x.shape
    W = w.shape[1]
    y = np.zeros((T, C))
    for j in range(W):               # token t - j, weighed by tap W-1-j
        if j >= T:
            break
        y[j:] += w[:, W - 1 - j] * x[:T - j]
    return y / (1.0 + np.exp(-y))


def l2_normalise(x: np.ndarray) -> np.ndarray:
    """Divide every vector along the last axis by its Euclidean norm (zero stays zero)."""
    n = np.sqrt((x * x).sum(axis=-1, keepdims=True))
    return np.divide(x, n, out=np.zeros_like(x), where=n > 0)


def delta_rule_step(S, q, k, v, alpha, beta):
    """One token, every head at once: S [H,dv,dk], q/k [H,dk], v [H,dv], alpha/beta [H].

    S (I - beta k k^T) is formed as S - beta (S k) k^T (the same matrix, no dk x dk product)."""
    Sk = np.einsum("hvk,hk->hv", S, k)
    S = alpha[:, None, None] * (S - beta[:, None, None] * Sk[:, :, None] * k[:, None, :]) \
        + beta[:, None, None] * v[:, :, None] * k[:, None, :]
    o = np.einsum("hvk,hk->hv", S, q)
    return S, o


def gated_delta_rule(q, k, v, g, beta, S0=None):
    """q, k [T,H,dk], v [T,H,dv], g, beta [T,H] (per value head) -> (o [T,H,dv], S_T [H,dv,dk])."""
    T, H, dk = q.shape
    dv = v.shape[2]
    S = np.zeros((H, dv, dk)) if S0 is None else np.array(S0, dtype=np.float64)
    o = np.empty((T, H, dv))
    alpha = np.exp(np.asarray(g, dtype=np.float64))
    beta = np.asarray(beta, dtype=np.float64)
    for t in range(T):
        S, o[t] = delta_rule_step(S, q[t], k[t], v[t], alpha[t], beta[t])
    return o, S


@dataclass
class GdnShape:
    Hk: int
    Hv: int
    dk: int
    dv: int

    @property
    def channels(self) -> int:
        return 2 * self.Hk * self.dk + self.Hv * self.dv


def mixing_inputs(x, conv_w, shape: GdnShape, storage: Optional[str] = None):
    """Convolution, SiLU, split, normalisation and scaling: x [T,C] -> q, k [T,Hv,dk], v [T,Hv,dv].

    q and k are returned per value head (key head h // (Hv/Hk) repeated)."""
    y = conv_silu(x, conv_w)
    T = y.shape[0]
    a = shape.Hk * shape.dk
    q = l2_normalise(y[:, :a].reshape(T, shape.Hk, shape.dk)) / np.sqrt(shape.dk)
    k = l2_normalise(y[:, a:2 * a].reshape(T, shape.Hk, shape.dk))
    v = y[:, 2 * a:].reshape(T, shape.Hv, shape.dv)
    q, k, v = round_to(q, storage), round_to(k, storage), round_to(v, storage)
    r = shape.Hv // shape.Hk
    return np.repeat(q, r, axis=1), np.repeat(k, r, axis=1), v


def gdn_sequence(x, conv_w, g, beta, shape: GdnShape, storage: Optional[str] = None, heads=None):
    """The layer on one sequence: x [T,C], g/beta [T,Hv] -> (o [T,Hv',dv], S_T) for value heads ``heads``."""
    q, k, v = mixing_inputs(x, conv_w, shape, storage)
    h = np.arange(shape.Hv) if heads is None else np.asarray(heads)
    return gated_delta_rule(q[:, h], k[:, h], v[:, h], np.asarray(g)[:, h], np.asarray(beta)[:, h])


@dataclass
class GdnTreeResult:
    trie: Trie
    layout: Layout
    heads: np.ndarray
    out: np.ndarray            # [row_len, len(heads), dv], NaN where not computed
    max_shared_gap: float      # largest disagreement between sequences sharing a slot


def tree_gdn(sequences, fid, tables, conv_w, shape: GdnShape, *, min_shared: int = 64,
             row_len: Optional[int] = None, storage: Optional[str] = None, heads=None,
             seqs: Optional[Sequence[int]] = None) -> GdnTreeResult:
    """Trie, layout, the layer on every sequence (or on ``seqs``), results mapped back to slots.

    ``tables`` holds x [n_feat, C], g [n_feat, Hv] and beta [n_feat, Hv]; token t of
    sequence s reads row fid[s][t] (a token's inputs depend only on its prefix)."""
    trie = build_trie(sequences, min_shared=min_shared)
    n = trie.n_nodes
    layout = dfs_layout(trie.parent, trie.seq_last, n if row_len is None else row_len)
    h = np.arange(shape.Hv) if heads is None else np.asarray(heads)
    out = np.full((layout.slot_node.shape[0], len(h), shape.dv), np.nan)
    gap = 0.0
    for s in (range(len(sequences)) if seqs is None else seqs):
        f = np.asarray(fid[s])
        if len(f) == 0:
            continue
        o, _ = gdn_sequence(tables["x"][f], conv_w, tables["g"][f], tables["beta"][f], shape, storage, h)
        slots = layout.token_index[s]
        prev = out[slots]
        seen = ~np.isnan(prev[:, 0, 0])
        if seen.any():
            gap = max(gap, float(np.max(np.abs(prev[seen] - o[seen]))))
        out[slots] = o
    return GdnTreeResult(trie=trie, layout=layout, heads=h, out=out, max_shared_gap=gap)
