"""Pins of the GDN oracle (CPU): library routines, closed forms, the delta rule as a gradient step,
an independently derived chunked form, and tree invariants."""

import numpy as np
import pytest
import torch

from oracle.gdn import (GdnShape, conv_silu, delta_rule_step, gated_delta_rule, gdn_sequence, l2_normalise,
                        mixing_inputs, tree_gdn)
from oracle.precision import round_to
from synth import from_sequences, gdn_tables, grpo_group

torch.set_default_dtype(torch.float64)


def _unit(rng, *shape):
    return l2_normalise(rng.standard_normal(shape))


# --------------------------------------------------------------------------
# convolution, SiLU and normalisation against torch
# --------------------------------------------------------------------------

@pytest.mark.parametrize("W,T", [(4, 1), (4, 3), (4, 17), (2, 9), (1, 5)])
def test_conv_silu_matches_torch_depthwise_conv1d(W, T):
    rng = np.random.default_rng(W * 100 + T)
    C = 6
    x = rng.standard_normal((T, C))
    w = rng.standard_normal((C, W))
    xt = torch.from_numpy(x).T[None]                       # [1, C, T]
    y = torch.nn.functional.conv1d(torch.nn.functional.pad(xt, (W - 1, 0)), torch.from_numpy(w)[:, None, :],
                                   groups=C)
    ref = torch.nn.functional.silu(y)[0].T.numpy()
    np.testing.assert_allclose(conv_silu(x, w), ref, rtol=1e-13, atol=1e-13)


def test_conv_impulse_response_is_the_taps_reversed():
    w = np.array([[1.0, 2.0, 3.0, 4.0]])
    x = np.zeros((6, 1))
    x[1, 0] = 1.0
    y = conv_silu(x, w)
    silu = lambda z: z / (1 + np.exp(-z))  # noqa: E731
    np.testing.assert_allclose(y[:, 0], [0, silu(4), silu(3), silu(2), silu(1), 0], rtol=1e-14, atol=0)


def test_l2_normalise_matches_torch_and_keeps_zero():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((5, 3, 8))
    x[2, 1] = 0
    ref = torch.nn.functional.normalize(torch.from_numpy(x), dim=-1, eps=1e-300).numpy()
    np.testing.assert_allclose(l2_normalise(x), ref, rtol=1e-14, atol=1e-300)
    assert np.all(l2_normalise(x)[2, 1] == 0)


# --------------------------------------------------------------------------
# the recurrence
# --------------------------------------------------------------------------

def test_step_is_decay_then_one_gradient_step_on_the_key_value_loss():
    """alpha S, then S <- S - beta * d/dS (1/2 |S k - v|^2), by autograd; o = S q."""
    rng = np.random.default_rng(2)
    H, dk, dv = 3, 5, 4
    S = rng.standard_normal((H, dv, dk))
    q, k, v = rng.standard_normal((H, dk)), _unit(rng, H, dk), rng.standard_normal((H, dv))
    alpha, beta = rng.random(H), rng.random(H)
    S_new, o = delta_rule_step(S, q, k, v, alpha, beta)
    for h in range(H):
        St = (alpha[h] * torch.from_numpy(S[h])).requires_grad_(True)
        loss = 0.5 * ((St @ torch.from_numpy(k[h]) - torch.from_numpy(v[h])) ** 2).sum()
        (grad,) = torch.autograd.grad(loss, St)
        ref = (St - beta[h] * grad).detach().numpy()
        np.testing.assert_allclose(S_new[h], ref, rtol=1e-13, atol=1e-13)
        np.testing.assert_allclose(o[h], ref @ q[h], rtol=1e-13, atol=1e-13)


def test_first_token_from_zero_state():
    rng = np.random.default_rng(3)
    T, H, dk, dv = 1, 2, 6, 3
    q, k, v = rng.standard_normal((T, H, dk)), _unit(rng, T, H, dk), rng.standard_normal((T, H, dv))
    g, beta = -rng.random((T, H)), rng.random((T, H))
    o, S = gated_delta_rule(q, k, v, g, beta)
    ref = beta[0][:, None] * (k[0] * q[0]).sum(-1)[:, None] * v[0]
    np.testing.assert_allclose(o[0], ref, rtol=1e-14, atol=1e-14)


def test_zero_decay_forgets_everything_before():
    rng = np.random.default_rng(4)
    T, H, dk, dv = 7, 2, 5, 3
    q, k, v = rng.standard_normal((T, H, dk)), _unit(rng, T, H, dk), rng.standard_normal((T, H, dv))
    g, beta = np.full((T, H), -np.inf), rng.random((T, H))
    o, _ = gated_delta_rule(q, k, v, g, beta)
    ref = beta[:, :, None] * (k * q).sum(-1)[:, :, None] * v
    np.testing.assert_allclose(o, ref, rtol=1e-14, atol=1e-14)


def test_no_writes_after_the_first_only_decay():
    rng = np.random.default_rng(5)
    T, H, dk, dv = 6, 2, 4, 3
    q, k, v = rng.standard_normal((T, H, dk)), _unit(rng, T, H, dk), rng.standard_normal((T, H, dv))
    g = -rng.random((T, H))
    beta = np.zeros((T, H))
    beta[0] = rng.random(H)
    o, _ = gated_delta_rule(q, k, v, g, beta)
    decay = np.exp(np.cumsum(g, axis=0) - g[0])     # prod of alpha_2 .. alpha_t (the write follows alpha_1)
    ref = decay[:, :, None] * beta[0][None, :, None] * (k[0][None] * q).sum(-1)[:, :, None] * v[0][None]
    np.testing.assert_allclose(o, ref, rtol=1e-13, atol=1e-14)


def test_orthonormal_keys_with_unit_gates_recall_exactly():
    """alpha = beta = 1 and orthonormal keys: the state maps every key written so far to its value."""
    rng = np.random.default_rng(6)
    dk = dv = 8
    T = dk
    Qm, _ = np.linalg.qr(rng.standard_normal((dk, dk)))
    k = Qm.T[:, None, :]                             # T orthonormal keys, one head
    v = rng.standard_normal((T, 1, dv))
    # query each step with an earlier key j (cycling): recall v_j exactly
    js = [t // 2 for t in range(T)]
    q = k[js]
    o, S = gated_delta_rule(q, k, v, np.zeros((T, 1)), np.ones((T, 1)))
    np.testing.assert_allclose(o[:, 0], v[js, 0], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(S[0] @ k[:, 0].T, v[:, 0].T, rtol=1e-12, atol=1e-12)


def test_rewriting_a_key_replaces_its_value():
    """beta = 1 writes the new value over the old one for the same key (the delta rule's correction)."""
    rng = np.random.default_rng(7)
    dk, dv = 5, 3
    k1 = _unit(rng, dk)
    k = np.stack([k1, k1])[:, None]
    v = rng.standard_normal((2, 1, dv))
    o, _ = gated_delta_rule(k.copy(), k, v, np.zeros((2, 1)), np.ones((2, 1)))
    np.testing.assert_allclose(o[1, 0], v[1, 0], rtol=1e-13, atol=1e-13)


def test_output_is_linear_in_values_and_initial_state():
    rng = np.random.default_rng(8)
    T, H, dk, dv = 9, 2, 4, 3
    q, k = rng.standard_normal((T, H, dk)), _unit(rng, T, H, dk)
    g, beta = -rng.random((T, H)), rng.random((T, H))
    v1, v2 = rng.standard_normal((T, H, dv)), rng.standard_normal((T, H, dv))
    S1, S2 = rng.standard_normal((H, dv, dk)), rng.standard_normal((H, dv, dk))
    o1, _ = gated_delta_rule(q, k, v1, g, beta, S1)
    o2, _ = gated_delta_rule(q, k, v2, g, beta, S2)
    o12, _ = gated_delta_rule(q, k, 2 * v1 - v2, g, beta, 2 * S1 - S2)
    np.testing.assert_allclose(o12, 2 * o1 - o2, rtol=1e-12, atol=1e-12)


def test_running_in_two_pieces_with_the_state_handed_over():
    rng = np.random.default_rng(9)
    T, H, dk, dv = 11, 2, 4, 3
    q, k, v = rng.standard_normal((T, H, dk)), _unit(rng, T, H, dk), rng.standard_normal((T, H, dv))
    g, beta = -rng.random((T, H)), rng.random((T, H))
    o, S = gated_delta_rule(q, k, v, g, beta)
    oa, Sa = gated_delta_rule(q[:4], k[:4], v[:4], g[:4], beta[:4])
    ob, Sb = gated_delta_rule(q[4:], k[4:], v[4:], g[4:], beta[4:], Sa)
    np.testing.assert_allclose(np.concatenate([oa, ob]), o, rtol=0, atol=0)
    np.testing.assert_allclose(Sb, S, rtol=0, atol=0)


def _chunked(q, k, v, g, beta, C, S0=None):
    """The chunked form, derived independently: within a chunk with log decays G_i = sum_{s<=i} g_s,
    A_ij = beta_i (k_i.k_j) e^{G_i - G_j} (j < i), T = (I + A)^-1, U = T diag(beta) V,
    W = T diag(beta e^G) K, D = U - W S0^T, o_i = e^{G_i} S0 q_i + sum_{j<=i} e^{G_i-G_j} (q_i.k_j) D_j,
    S_end = e^{G_L} S0 + sum_j e^{G_L - G_j} D_j k_j^T."""
    T_, H, dk = q.shape
    dv = v.shape[2]
    S = np.zeros((H, dv, dk)) if S0 is None else S0.copy()
    o = np.empty((T_, H, dv))
    for c0 in range(0, T_, C):
        sl = slice(c0, min(T_, c0 + C))
        L = sl.stop - sl.start
        for h in range(H):
            Q, K, V = q[sl, h], k[sl, h], v[sl, h]
            G = np.cumsum(g[sl, h])
            b = beta[sl, h]
            dec = np.exp(G[:, None] - G[None, :])
            A = np.tril(b[:, None] * (K @ K.T) * dec, -1)
            Tm = np.linalg.inv(np.eye(L) + A)
            U = Tm @ (b[:, None] * V)
            Wm = Tm @ ((b * np.exp(G))[:, None] * K)
            D = U - Wm @ S[h].T
            o[sl, h] = np.exp(G)[:, None] * (Q @ S[h].T) + (np.tril(Q @ K.T * dec)) @ D
            S[h] = np.exp(G[-1]) * S[h] + (np.exp(G[-1] - G)[:, None] * D).T @ K
    return o, S


@pytest.mark.parametrize("T,C", [(1, 4), (13, 4), (64, 64), (150, 64), (7, 64)])
def test_chunked_form_equals_the_recurrence(T, C):
    rng = np.random.default_rng(10 + T)
    H, dk, dv = 2, 8, 6
    q, k, v = rng.standard_normal((T, H, dk)), _unit(rng, T, H, dk), rng.standard_normal((T, H, dv))
    g, beta = -0.3 * rng.random((T, H)), rng.random((T, H))
    S0 = rng.standard_normal((H, dv, dk))
    o, S = gated_delta_rule(q, k, v, g, beta, S0)
    oc, Sc = _chunked(q, k, v, g, beta, C, S0)
    np.testing.assert_allclose(oc, o, rtol=1e-10, atol=1e-10)
    np.testing.assert_allclose(Sc, S, rtol=1e-10, atol=1e-10)


def test_padding_a_chunk_with_zero_gates_and_writes_changes_nothing():
    """g = 0, beta = 0, k = 0 after the last token: the state and the outputs are those of the short run."""
    rng = np.random.default_rng(11)
    T, H, dk, dv = 5, 2, 4, 3
    q, k, v = rng.standard_normal((T, H, dk)), _unit(rng, T, H, dk), rng.standard_normal((T, H, dv))
    g, beta = -rng.random((T, H)), rng.random((T, H))
    o, S = gated_delta_rule(q, k, v, g, beta)
    P = 3
    pad = lambda a: np.concatenate([a, np.zeros((P,) + a.shape[1:])])  # noqa: E731
    op, Sp = _chunked(pad(q), pad(k), pad(v), pad(g), pad(beta), 8)
    np.testing.assert_allclose(op[:T], o, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(Sp, S, rtol=1e-12, atol=1e-12)


# --------------------------------------------------------------------------
# the layer: channel order, head mapping, storage
# --------------------------------------------------------------------------

def _layer_inputs(seed, T, shape, W=4):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((T, shape.channels))
    w = rng.standard_normal((shape.channels, W)) / 2
    g = -rng.random((T, shape.Hv)) * 0.2
    beta = rng.random((T, shape.Hv))
    return x, w, g, beta


def test_value_head_reads_key_head_h_over_ratio():
    shape = GdnShape(Hk=2, Hv=4, dk=4, dv=3)
    x, w, g, beta = _layer_inputs(12, 10, shape)
    a = shape.Hk * shape.dk
    x[:, a + shape.dk:2 * a] = 0          # key head 1 silent: k = 0, nothing is ever written
    o, _ = gdn_sequence(x, w, g, beta, shape)
    assert np.all(o[:, 2:] == 0) and np.all(np.abs(o[:, :2]).max(axis=(0, 2)) > 0)


@pytest.mark.parametrize("part", ["q", "k", "v"])
def test_channel_order_q_k_v(part):
    shape = GdnShape(Hk=1, Hv=2, dk=4, dv=3)
    x, w, g, beta = _layer_inputs(13, 8, shape)
    a = shape.Hk * shape.dk
    cols = {"q": slice(0, a), "k": slice(a, 2 * a), "v": slice(2 * a, None)}[part]
    x[:, cols] = 0
    o, _ = gdn_sequence(x, w, g, beta, shape)
    assert np.all(o == 0)


def test_q_scaled_and_normalised_k_normalised_storage_rounded():
    shape = GdnShape(Hk=2, Hv=2, dk=16, dv=8)
    x, w, g, beta = _layer_inputs(14, 6, shape)
    q, k, v = mixing_inputs(x, w, shape)
    np.testing.assert_allclose(np.linalg.norm(q, axis=-1), 1 / 4, rtol=1e-14)
    np.testing.assert_allclose(np.linalg.norm(k, axis=-1), 1, rtol=1e-14)
    qb, kb, vb = mixing_inputs(x, w, shape, storage="bf16")
    for a, b in ((qb, q), (kb, k), (vb, v)):
        assert np.array_equal(a, round_to(a, "bf16"))
        assert np.max(np.abs(a - b) - 2.0 ** -8 * np.abs(b)) <= 1e-18   # half an ulp of 8 bits


# --------------------------------------------------------------------------
# over a tree
# --------------------------------------------------------------------------

def _tree_case(seed, shape):
    rng = np.random.default_rng(seed)
    seqs = []
    for _ in range(6):
        L = int(rng.integers(1, 90))
        seqs.append(np.repeat(rng.integers(0, 2, size=L // 12 + 1), 12)[:L].astype(np.int32))
    seqs.append(seqs[0].copy())
    w = from_sequences(seqs, Hq=1, Hkv=1, D=8, dtype="f32", seed_base=300 + seed)
    t = gdn_tables(w, Hk=shape.Hk, Hv=shape.Hv, dk=shape.dk, dv=shape.dv)
    return w, t


@pytest.mark.parametrize("seed", range(4))
def test_shared_slots_get_one_value_and_sequences_are_independent(seed):
    shape = GdnShape(Hk=1, Hv=2, dk=8, dv=4)
    w, t = _tree_case(seed, shape)
    r = tree_gdn(w.sequences, w.fid, t, t["conv_w"], shape, min_shared=2)
    assert r.max_shared_gap == 0.0
    assert not np.isnan(r.out[:r.trie.n_nodes]).any()
    # every sequence alone gives the values the tree holds at its slots
    for s in range(len(w.sequences)):
        f = w.fid[s]
        if len(f) == 0:
            continue
        o, _ = gdn_sequence(t["x"][f], t["conv_w"], t["g"][f], t["beta"][f], shape)
        np.testing.assert_array_equal(r.out[r.layout.token_index[s]], o)


def test_grpo_group_outputs_of_the_prompt_do_not_depend_on_the_completions():
    w = grpo_group(prompt=96, n=3, completion=40, Hq=1, Hkv=1, D=8, row_len=None)
    shape = GdnShape(Hk=1, Hv=2, dk=8, dv=4)
    t = gdn_tables(w, Hk=1, Hv=2, dk=8, dv=4)
    r = tree_gdn(w.sequences, w.fid, t, t["conv_w"], shape, seqs=[0])
    f = w.fid[0][:96]
    o, _ = gdn_sequence(t["x"][f], t["conv_w"], t["g"][f], t["beta"][f], shape)
    np.testing.assert_array_equal(r.out[r.layout.token_index[0][:96]], o)
