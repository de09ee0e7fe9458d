"""Oracle step 7: dense brute force on small packed trees, fp64.

The ancestor mask is built by walking parent pointers, not from any
interval: M[i, j] = 1 iff j is i or an ancestor of i [DAG "The mask": a
token attends to itself and the nodes on its own path; ART "Token-mixing
layers"].  Attention is then a dense masked softmax over the whole row, its
gradient the closed form of softmax attention, and the finite-difference
check perturbs one input element at a time.
"""

from __future__ import annotations

import numpy as np


def ancestor_mask(slot_parent) -> np.ndarray:
    """slot_parent[i] = slot of i's parent (-1 for a root) -> dense bool mask [n, n]."""
    slot_parent = np.asarray(slot_parent, dtype=np.int64)
    n = len(slot_parent)
    M = np.zeros((n, n), dtype=bool)
    for i in range(n):
        j = i
        steps = 0
        while j >= 0:
            M[i, j] = True
            j = int(slot_parent[j])
            steps += 1
            if steps > n:
                raise ValueError("cycle in parent pointers")
    return M


def dense_forward(q, k, v, mask, scale):
    """q [n,Hq,D], k/v [n,Hkv,D], mask [n,n] -> out [n,Hq,D], lse [Hq,n]."""
    n, Hq, D = q.shape
    G = Hq // k.shape[1]
    out = np.zeros((n, Hq, D))
    lse = np.zeros((Hq, n))
    for h in range(Hq):
        g = h // G
        S = scale * (q[:, h] @ k[:, g].T)
        S = np.where(mask, S, -np.inf)
        m = S.max(axis=1)
        l = m + np.log(np.exp(S - m[:, None]).sum(axis=1))
        P = np.exp(S - l[:, None])
        out[:, h] = P @ v[:, g]
        lse[h] = l
    return out, lse


def dense_backward(q, k, v, mask, dout, scale):
    """Closed-form gradient of sum(dout * out) for dense masked softmax attention."""
    n, Hq, D = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    dq = np.zeros_like(q, dtype=np.float64)
    dk = np.zeros((n, Hkv, D))
    dv = np.zeros((n, Hkv, D))
    for h in range(Hq):
        g = h // G
        S = scale * (q[:, h] @ k[:, g].T)
        S = np.where(mask, S, -np.inf)
        m = S.max(axis=1)
        P = np.exp(S - m[:, None])
        P /= P.sum(axis=1, keepdims=True)
        # Jacobian of row softmax: dS = P * (dP - sum_j P dP)
        dP = dout[:, h] @ v[:, g].T
        dS = P * (dP - (P * dP).sum(axis=1, keepdims=True))
        dq[:, h] = scale * dS @ k[:, g]
        dk[:, g] += scale * dS.T @ q[:, h]
        dv[:, g] += P.T @ dout[:, h]
    return dq, dk, dv


def finite_difference(fn, x, eps=1e-6):
    """Central differences of the scalar fn() with respect to every element of x (modified in place)."""
    g = np.zeros_like(x, dtype=np.float64)
    flat = x.reshape(-1)
    gf = g.reshape(-1)
    for idx in range(flat.size):
        keep = flat[idx]
        flat[idx] = keep + eps
        up = fn()
        flat[idx] = keep - eps
        down = fn()
        flat[idx] = keep
        gf[idx] = (up - down) / (2 * eps)
    return g
