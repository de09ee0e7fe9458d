"""Test harness: run one workload through the library and through the oracle, then compare.

The two sides share only the workload (sequences, per-token table rows,
tables).  The library side builds its own trie and layout with the C ABI and
fills its packed tensors by inverting its own token_index; the oracle side
builds everything with ``oracle``.  Results are compared token by token:
token t of sequence s sits in library slot lib_ti[s][t] and oracle slot
ora_ti[s][t].
"""

from __future__ import annotations

import sys
import time
from dataclasses import dataclass
from typing import Optional

import numpy as np

import prefix_tree_packed_dfs_amd as lib
from oracle.attention import tree_attention


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@dataclass
class LibResult:
    layout: lib.PackedLayout
    n: int
    R: int
    out: np.ndarray
    lse: np.ndarray
    dq: Optional[np.ndarray]
    dk: Optional[np.ndarray]
    dv: Optional[np.ndarray]
    q_rot: np.ndarray       # rotated q and k as the kernels read them
    k_rot: np.ndarray


def slot_rows(w, layout, n):
    """Feature row and gradient row of every slot, from the library's token_index.

    Every token mapped to one slot must name the same rows (same prefix, same
    next token); a trie that merged two different tokens would fail here.
    """
    ti = np.concatenate([layout.sequence_slots(s) for s in range(len(w.sequences))]).astype(np.int64)
    f = np.concatenate(w.fid)
    d = np.concatenate(w.dkey)
    fid_slot = np.full(layout.slot_node.shape[0], -1, dtype=np.int64)
    dkey_slot = np.full(layout.slot_node.shape[0], -1, dtype=np.int64)
    fid_slot[ti] = f
    dkey_slot[ti] = d
    assert np.array_equal(fid_slot[ti], f), "one slot holds tokens with different prefixes"
    assert np.array_equal(dkey_slot[ti], d), "one slot holds tokens with different targets"
    assert np.all(fid_slot[:n] >= 0), "a real slot is reached by no sequence"
    return fid_slot, dkey_slot


def bwd_workspace(w, lay, R, mode: Optional[str], device="cuda"):
    """Backward workspace by mode: None (the binding's default, the largest), "exact" (what this row's
    dK/dV plan uses), "fixed" (no partial-sum slots: no key tile is cut into chunks)."""
    import torch
    if mode is None:
        return None
    dt = lib.TREE_BF16 if w.dtype == "bf16" else lib.TREE_F32
    se = lay.subtree_end.astype(np.int32) if mode == "exact" else np.arange(R, dtype=np.int32)
    nbytes = lib.tree_attn_bwd_workspace_bytes_for(dt, se, w.Hq, w.Hkv, w.D)
    return torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device)


def run_library(w, tables, *, rope: bool = True, backward: Optional[bool] = None, device="cuda",
                min_shared: int = 64, ws_mode: Optional[str] = None) -> LibResult:
    import torch
    backward = w.backward if backward is None else backward
    tdt = {"f32": torch.float32, "bf16": torch.bfloat16}[w.dtype]
    parent, seq_last = lib.tree_build_trie(w.sequences, min_shared=min_shared)
    n = len(parent)
    R = w.row_length(n)
    lay = lib.tree_pack_layout(parent, seq_last, R)
    fid_slot, dkey_slot = slot_rows(w, lay, n)

    def packed(table, rows, H):
        x = np.zeros((R, H, w.D), dtype=np.float32)
        x[:n] = table[rows[:n]]
        return torch.from_numpy(x).to(tdt).view(1, R, H, w.D).to(device)

    q = packed(tables["q"], fid_slot, w.Hq)
    k = packed(tables["k"], fid_slot, w.Hkv)
    v = packed(tables["v"], fid_slot, w.Hkv)
    se = torch.from_numpy(lay.subtree_end.astype(np.int32)).view(1, R).to(device)
    pos = torch.from_numpy(lay.pos_ids.astype(np.int32)).view(1, R).to(device)
    if rope:
        lib.tree_rope(q, pos, w.theta)
        lib.tree_rope(k, pos, w.theta)
    out, lse = lib.tree_attn_fwd(q, k, v, se)
    dq = dk = dv = None
    if backward:
        do = packed(tables["do"], dkey_slot, w.Hq)
        dq, dk, dv = lib.tree_attn_bwd(q, k, v, se, out, lse, do, ws=bwd_workspace(w, lay, R, ws_mode, device))
    torch.cuda.synchronize()

    def host(t):
        return None if t is None else t[0].to(torch.float64).cpu().numpy()

    return LibResult(layout=lay, n=n, R=R, out=host(out), lse=host(lse), dq=host(dq), dk=host(dk), dv=host(dv),
                     q_rot=host(q), k_rot=host(k))


def run_oracle(w, tables, *, rope: bool = True, backward: Optional[bool] = None, q_slots=None, k_slots=None,
               R=None, kv_heads=None):
    backward = w.backward if backward is None else backward
    theta = w.theta if rope else None
    return tree_attention(w.sequences, w.fid, w.dkey, tables, theta=theta, row_len=R, backward=backward,
                          q_slots=q_slots, k_slots=k_slots, storage=w.dtype, kv_heads=kv_heads)


def slot_map(w, lres, ores):
    """Library slot -> oracle slot, checked to be one consistent bijection on real slots."""
    m = np.full(lres.R, -1, dtype=np.int64)
    for s in range(len(w.sequences)):
        a = lres.layout.sequence_slots(s).astype(np.int64)
        b = ores.layout.token_index[s]
        assert len(a) == len(b)
        prev = m[a]
        assert np.all((prev < 0) | (prev == b)), "slot correspondence is not a function"
        m[a] = b
    real = m[:lres.n]
    assert np.all(real >= 0) and len(np.unique(real)) == lres.n, "slot correspondence is not a bijection"
    return m


@dataclass
class Cmp:
    name: str
    max_abs: float
    max_ref: float
    rel: float
    cos: float
    count: int
    beyond_half_ulp: float   # max over elements of |a-b| - 2^-8 |b| (bf16 storage rounding taken out)
    vs_rounded: float = 0.0  # max|a - bf16(b)|: against the oracle rounded to the library's storage (bf16 only)

    def __str__(self):
        return (f"{self.name:8s} max|d|={self.max_abs:.3e} max|ref|={self.max_ref:.3e} rel={self.rel:.3e} "
                f"cos={self.cos:.8f} beyond-half-ulp={self.beyond_half_ulp:.3e} "
                f"vs-bf16(ref)={self.vs_rounded:.3e} n={self.count}")


def cmp(name, a, b, storage: Optional[str] = None) -> Cmp:
    a = np.asarray(a, dtype=np.float64).ravel()
    b = np.asarray(b, dtype=np.float64).ravel()
    assert np.all(np.isfinite(a)), f"{name}: non-finite library values"
    assert np.all(np.isfinite(b)), f"{name}: oracle values missing"
    d = float(np.max(np.abs(a - b))) if a.size else 0.0
    ref = float(np.max(np.abs(b))) if b.size else 0.0
    den = float(np.linalg.norm(a) * np.linalg.norm(b))
    cos = float(a @ b / den) if den > 0 else 1.0
    beyond = float(np.max(np.abs(a - b) - 2.0**-8 * np.abs(b))) if a.size else 0.0
    vr = 0.0
    if storage == "bf16" and a.size:
        from oracle.precision import round_to
        vr = float(np.max(np.abs(a - round_to(b, "bf16"))))
    return Cmp(name, d, ref, d / ref if ref > 0 else d, cos, a.size, beyond, vr)


TOL = {
    # fp32: max|a-b| <= 1e-5 * max|b| per tensor
    "f32": {"rel": 1e-5},
    # bf16: 2e-2 absolute on out/dq/dk/dv on top of the half-ulp rounding of the bf16 output
    # (|a-b| <= 2e-2 + 2^-8 |b| per element), 1e-3 absolute on the fp32 lse, and a relative
    # max-norm bar of 2e-2 on every tensor.  The half-ulp allowance came with the bf16
    # matrix-core forward: a bf16 tensor cannot hold values above 5.12 to within 2e-2.  Every
    # comparison also logs the strict max|a-b| and max|a - bf16(b)| (the oracle rounded to the
    # library's storage dtype).
    "bf16": {"abs": 2e-2, "abs_lse": 1e-3, "rel": 2e-2},
}


def compare(w, lres, ores, *, lib_slots=None, key_slots=None, deep_depth=1024):
    """Compare on library slots (default all real); returns the list of Cmp rows."""
    m = slot_map(w, lres, ores)
    ls = np.arange(lres.n) if lib_slots is None else np.asarray(lib_slots, dtype=np.int64)
    ks = ls if key_slots is None else np.asarray(key_slots, dtype=np.int64)
    os_, ok = m[ls], m[ks]
    st = w.dtype
    rows = [cmp("out", lres.out[ls], ores.out[os_], st), cmp("lse", lres.lse[:, ls], ores.lse[:, os_])]
    if lres.dq is not None and ores.dq is not None:
        rows += [cmp("dq", lres.dq[ls], ores.dq[os_], st), cmp("dk", lres.dk[ks], ores.dk[ok], st),
                 cmp("dv", lres.dv[ks], ores.dv[ok], st)]
    deep = ls[lres.layout.pos_ids[ls] >= deep_depth]
    if len(deep):
        rows.append(cmp("out@deep", lres.out[deep], ores.out[m[deep]], st))
        if lres.dq is not None and ores.dq is not None:
            rows.append(cmp("dq@deep", lres.dq[deep], ores.dq[m[deep]], st))
    return rows


def assert_within(w, rows):
    tol = TOL[w.dtype]
    for r in rows:
        log("   ", r)
    for r in rows:
        if r.name.endswith("@deep"):
            assert r.cos > 0.999, f"{r.name}: cosine {r.cos}"
            continue
        if w.dtype == "f32":
            assert r.max_abs <= tol["rel"] * r.max_ref, f"{r.name}: {r}"
        else:
            if r.name == "lse":
                assert r.max_abs <= tol["abs_lse"], f"{r.name}: {r}"
            else:
                assert r.beyond_half_ulp <= tol["abs"], f"{r.name}: {r}"
            assert r.rel <= tol["rel"], f"{r.name}: {r}"


def timed(label, fn, *a, **k):
    t0 = time.time()
    r = fn(*a, **k)
    log(f"  [{label}] {time.time() - t0:.1f}s")
    return r
