"""Pins for the oracle's tree attention (CPU only)."""

import numpy as np
import pytest
import torch

from oracle.attention import causal_backward, causal_forward, tree_attention
from oracle.brute import ancestor_mask, dense_backward, dense_forward, finite_difference
from oracle.rope import rope


def _random_case(seed, n_seqs=6, max_len=14, vocab=3, Hq=4, Hkv=2, D=8):
    """Sequences over a tiny vocabulary (many forks) with prefix-consistent tensors."""
    rng = np.random.default_rng(seed)
    seqs = [rng.integers(0, vocab, size=int(rng.integers(1, max_len))).tolist() for _ in range(n_seqs)]
    # prefix ids / (prefix, next) ids computed directly from tuples (fine at this size)
    fids, dkeys, pre, nxt = [], [], {}, {}
    for s in seqs:
        f, d = [], []
        for t in range(len(s)):
            f.append(pre.setdefault(tuple(s[:t + 1]), len(pre)))
            key = tuple(s[:t + 2]) if t + 1 < len(s) else (tuple(s), "end")
            d.append(nxt.setdefault(key, len(nxt)))
        fids.append(np.asarray(f))
        dkeys.append(np.asarray(d))
    tables = {"q": rng.standard_normal((len(pre), Hq, D)), "k": rng.standard_normal((len(pre), Hkv, D)),
              "v": rng.standard_normal((len(pre), Hkv, D)), "do": rng.standard_normal((len(nxt), Hq, D))}
    return seqs, fids, dkeys, tables


def _packed_inputs(res, seqs, fids, dkeys, tables, theta):
    """Packed q/k/v/dout in the oracle's slot order, taken from any sequence through each slot."""
    lay = res.layout
    n = lay.n_nodes
    Hq, D = tables["q"].shape[1:]
    Hkv = tables["k"].shape[1]
    q = np.zeros((n, Hq, D)); k = np.zeros((n, Hkv, D)); v = np.zeros((n, Hkv, D)); do = np.zeros((n, Hq, D))
    for s in range(len(seqs)):
        ti = lay.token_index[s]
        q[ti] = tables["q"][fids[s]]
        k[ti] = tables["k"][fids[s]]
        v[ti] = tables["v"][fids[s]]
        do[ti] = tables["do"][dkeys[s]]
    pos = lay.pos_ids[:n]
    q = rope(q, pos, theta)
    k = rope(k, pos, theta)
    slot_parent = np.asarray([-1 if res.trie.parent[lay.slot_node[s]] < 0
                              else lay.node_slot[res.trie.parent[lay.slot_node[s]]] for s in range(n)])
    return q, k, v, do, slot_parent


@pytest.mark.parametrize("seed", range(12))
def test_tree_attention_matches_dense_brute_force(seed):
    seqs, fids, dkeys, tables = _random_case(seed)
    theta = 10.0
    res = tree_attention(seqs, fids, dkeys, tables, theta=theta, min_shared=1)
    n = res.layout.n_nodes
    assert res.max_shared_gap < 1e-12
    q, k, v, do, sp = _packed_inputs(res, seqs, fids, dkeys, tables, theta)
    M = ancestor_mask(sp)
    scale = 1 / np.sqrt(q.shape[-1])
    out, lse = dense_forward(q, k, v, M, scale)
    dq, dk, dv = dense_backward(q, k, v, M, do, scale)
    assert np.allclose(res.out[:n], out, atol=1e-12)
    assert np.allclose(res.lse[:, :n], lse, atol=1e-12)
    assert np.allclose(res.dq[:n], dq, atol=1e-11)
    assert np.allclose(res.dk[:n], dk, atol=1e-11)
    assert np.allclose(res.dv[:n], dv, atol=1e-11)


@pytest.mark.parametrize("seed", range(4))
def test_finite_differences(seed):
    seqs, fids, dkeys, tables = _random_case(100 + seed, n_seqs=3, max_len=6, Hq=2, Hkv=1, D=4)
    res = tree_attention(seqs, fids, dkeys, tables, theta=10.0, min_shared=1)
    n = res.layout.n_nodes
    assert n <= 12
    q, k, v, do, sp = _packed_inputs(res, seqs, fids, dkeys, tables, 10.0)
    M = ancestor_mask(sp)
    scale = 0.5

    def loss():
        o, _ = dense_forward(q, k, v, M, scale)
        return float(np.sum(o * do))

    res = tree_attention(seqs, fids, dkeys, tables, theta=10.0, min_shared=1, scale=scale)
    for name, x, g in (("q", q, res.dq), ("k", k, res.dk), ("v", v, res.dv)):
        fd = finite_difference(loss, x)
        assert np.allclose(g[:n], fd, atol=1e-7), name


def test_torch_autograd_dense():
    seqs, fids, dkeys, tables = _random_case(7, n_seqs=5, max_len=10)
    res = tree_attention(seqs, fids, dkeys, tables, theta=100.0, min_shared=1)
    n = res.layout.n_nodes
    q, k, v, do, sp = _packed_inputs(res, seqs, fids, dkeys, tables, 100.0)
    M = torch.from_numpy(ancestor_mask(sp))
    tq, tk, tv = (torch.from_numpy(x).requires_grad_(True) for x in (q, k, v))
    G = q.shape[1] // k.shape[1]
    kk = tk.repeat_interleave(G, dim=1)
    vv = tv.repeat_interleave(G, dim=1)
    o = torch.nn.functional.scaled_dot_product_attention(
        tq.transpose(0, 1), kk.transpose(0, 1), vv.transpose(0, 1), attn_mask=M).transpose(0, 1)
    (o * torch.from_numpy(do)).sum().backward()
    assert np.allclose(res.out[:n], o.detach().numpy(), atol=1e-12)
    assert np.allclose(res.dq[:n], tq.grad.numpy(), atol=1e-11)
    assert np.allclose(res.dk[:n], tk.grad.numpy(), atol=1e-11)
    assert np.allclose(res.dv[:n], tv.grad.numpy(), atol=1e-11)


def test_chain_is_causal_attention():
    rng = np.random.default_rng(5)
    L, H, D = 50, 2, 16
    Q, K, V = (rng.standard_normal((L, H, D)) for _ in range(3))
    O, lse = causal_forward(Q, K, V, 0.25)
    ref = torch.nn.functional.scaled_dot_product_attention(
        *(torch.from_numpy(x).transpose(0, 1) for x in (Q, K, V)), is_causal=True, scale=0.25)
    assert np.allclose(O, ref.transpose(0, 1).numpy(), atol=1e-12)
    S = 0.25 * np.einsum("qhd,khd->hqk", Q, K)
    S = np.where(np.tril(np.ones((L, L), dtype=bool))[None], S, -np.inf)
    assert np.allclose(lse, np.log(np.exp(S).sum(-1)), atol=1e-12)


def test_independent_sequences_block_diagonal():
    rng = np.random.default_rng(6)
    seqs = [[100 * i + j for j in range(9)] for i in range(4)]
    fids = [np.arange(9 * i, 9 * i + 9) for i in range(4)]
    dkeys = [np.arange(10 * i, 10 * i + 9) for i in range(4)]
    tables = {"q": rng.standard_normal((36, 2, 8)), "k": rng.standard_normal((36, 2, 8)),
              "v": rng.standard_normal((36, 2, 8)), "do": rng.standard_normal((40, 2, 8))}
    res = tree_attention(seqs, fids, dkeys, tables, theta=10000.0, min_shared=1)
    for i in range(4):
        Q = rope(tables["q"][fids[i]], np.arange(9), 1e4)
        K = rope(tables["k"][fids[i]], np.arange(9), 1e4)
        ref = torch.nn.functional.scaled_dot_product_attention(
            *(torch.from_numpy(x).transpose(0, 1) for x in (Q, K, tables["v"][fids[i]])), is_causal=True)
        assert np.allclose(res.out[res.layout.token_index[i]], ref.transpose(0, 1).numpy(), atol=1e-12)


def test_sequence_order_does_not_matter():
    seqs, fids, dkeys, tables = _random_case(9)
    a = tree_attention(seqs, fids, dkeys, tables, theta=10.0, min_shared=1)
    perm = [2, 0, 5, 1, 4, 3]
    b = tree_attention([seqs[i] for i in perm], [fids[i] for i in perm], [dkeys[i] for i in perm],
                       tables, theta=10.0, min_shared=1)
    for new, old in enumerate(perm):
        ta, tb = a.layout.token_index[old], b.layout.token_index[new]
        for x, y in ((a.out, b.out), (a.dq, b.dq), (a.dk, b.dk), (a.dv, b.dv)):
            assert np.allclose(x[ta], y[tb], atol=1e-12)
        assert np.allclose(a.lse[:, ta], b.lse[:, tb], atol=1e-12)


def test_sampled_mode_matches_full():
    seqs, fids, dkeys, tables = _random_case(11, n_seqs=6, max_len=20)
    full = tree_attention(seqs, fids, dkeys, tables, theta=10.0, min_shared=1)
    n = full.layout.n_nodes
    rng = np.random.default_rng(0)
    qs = rng.choice(n, size=min(6, n), replace=False)
    ks = rng.choice(n, size=min(6, n), replace=False)
    part = tree_attention(seqs, fids, dkeys, tables, theta=10.0, min_shared=1, q_slots=qs, k_slots=ks)
    assert np.allclose(part.out[qs], full.out[qs], atol=1e-13)
    assert np.allclose(part.lse[:, qs], full.lse[:, qs], atol=1e-13)
    assert np.allclose(part.dq[qs], full.dq[qs], atol=1e-12)
    assert np.allclose(part.dk[ks], full.dk[ks], atol=1e-12)
    assert np.allclose(part.dv[ks], full.dv[ks], atol=1e-12)


@pytest.mark.parametrize("Hq,Hkv,heads", [(4, 2, [1]), (6, 2, [0]), (8, 4, [0, 3])])
def test_kv_head_subset_matches_full(Hq, Hkv, heads):
    """Restricting the work to some KV heads (their whole query-head groups) leaves every output of those
    heads as in the full run, alone and together with sampled slots; the other heads are not computed."""
    seqs, fids, dkeys, tables = _random_case(17, n_seqs=6, max_len=20, Hq=Hq, Hkv=Hkv)
    full = tree_attention(seqs, fids, dkeys, tables, theta=10.0, min_shared=1)
    n = full.layout.n_nodes
    G = Hq // Hkv
    qh = [g * G + i for g in heads for i in range(G)]
    other_q = [h for h in range(Hq) if h not in qh]
    other_kv = [g for g in range(Hkv) if g not in heads]
    part = tree_attention(seqs, fids, dkeys, tables, theta=10.0, min_shared=1, kv_heads=heads)
    for a, b in ((part.out[:n, qh], full.out[:n, qh]), (part.lse[qh][:, :n], full.lse[qh][:, :n]),
                 (part.dq[:n, qh], full.dq[:n, qh]), (part.dk[:n, heads], full.dk[:n, heads]),
                 (part.dv[:n, heads], full.dv[:n, heads])):
        assert np.allclose(a, b, atol=1e-12, rtol=0)
    assert np.all(np.isnan(part.out[:, other_q])) and np.all(np.isnan(part.dq[:, other_q]))
    if other_kv:
        assert np.all(np.isnan(part.dk[:, other_kv])) and np.all(np.isnan(part.dv[:, other_kv]))
    rng = np.random.default_rng(1)
    ks = rng.choice(n, size=min(5, n), replace=False)
    both = tree_attention(seqs, fids, dkeys, tables, theta=10.0, min_shared=1, kv_heads=heads, k_slots=ks)
    assert np.allclose(both.dk[ks][:, heads], full.dk[ks][:, heads], atol=1e-12, rtol=0)
    assert np.allclose(both.dv[ks][:, heads], full.dv[ks][:, heads], atol=1e-12, rtol=0)


def test_gradient_sums_hold():
    """sum_j dV[j] = sum_i dout[i] per KV head; sum_j dK[j] = 0 (softmax rows sum to one)."""
    seqs, fids, dkeys, tables = _random_case(13)
    res = tree_attention(seqs, fids, dkeys, tables, theta=10.0, min_shared=1)
    n = res.layout.n_nodes
    q, k, v, do, sp = _packed_inputs(res, seqs, fids, dkeys, tables, 10.0)
    G = q.shape[1] // k.shape[1]
    dsum = do.reshape(n, k.shape[1], G, -1).sum(axis=(0, 2))
    assert np.allclose(res.dv[:n].sum(axis=0), dsum, atol=1e-10)
    assert np.allclose(res.dk[:n].sum(axis=0), 0.0, atol=1e-10)


def test_backward_rows_subset_is_exact_when_rest_is_zero():
    rng = np.random.default_rng(8)
    L, H, D = 30, 2, 4
    Q, K, V = (rng.standard_normal((L, H, D)) for _ in range(3))
    dO = rng.standard_normal((L, H, D))
    dO[:12] = 0
    dq_all, dk_all, dv_all = causal_backward(Q, K, V, dO, 0.5)
    dq, dk, dv = causal_backward(Q, K, V, dO, 0.5, rows=np.arange(12, L))
    assert np.allclose(dk, dk_all, atol=1e-13) and np.allclose(dv, dv_all, atol=1e-13)
    assert np.allclose(dq, dq_all[12:], atol=1e-13) and np.allclose(dq_all[:12], 0)
