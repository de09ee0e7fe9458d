"""GPU: tree packing against sequence packing, both through the C ABI.

Sequence packing lays every sequence out as its own chain (nothing shared);
the same kernels run over both layouts.  A token of sequence s attends to the
same keys either way, so per token:

* out and lse agree, and with the upstream gradient given to every copy of a
  token, so does dq;
* with the upstream gradient given to one copy only (the first sequence
  through the slot; the other copies get zero), the loss of the chain row
  equals the loss of the tree row as a function of the tree's tokens, so
  the tree's dk and dv are the sums of the copies' dk and dv, the tree's dq
  is the owning copy's dq, and every other copy's dq is exactly zero.

This is the gradient-sharing property that lets a trie forward a shared token
once [ART "Does it actually help?"; TRL tree packing "How tree packing works"].
Comparisons run on the device; every case prints its name first.
"""

import numpy as np
import pytest

from synth import (agentic_trie, feature_tables, from_sequences, grpo_group, long_history, sequence_packing_forest,
                   shared_history)

from .pipeline import assert_within, cmp, log, timed

pytestmark = pytest.mark.gpu

HALF_ULP = 2.0 ** -8     # bf16 storage rounding, relative
BF16_ABS = 2e-2          # the bf16 bar on out / dq / dk / dv
LSE_ABS = 1e-3
F32_REL = 1e-5


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import prefix_tree_packed_dfs_amd  # noqa: F401  (fails loudly if the library is not built)
    yield


def _pad64(n):
    return max(64, (n + 63) // 64 * 64)


class _Row:
    """One packed row of a workload (tree or chains) with its inputs gathered on the device."""

    def __init__(self, w, dev_tables, parent, seq_last):
        import torch

        import prefix_tree_packed_dfs_amd as lib
        self.n = n = len(parent)
        self.R = R = _pad64(n)
        self.lay = lib.tree_pack_layout(parent, seq_last, R)
        ti = np.concatenate([self.lay.sequence_slots(s) for s in range(len(w.sequences))]).astype(np.int64)
        self.ti = ti
        fid = np.full(R, -1, np.int64)
        dkey = np.full(R, -1, np.int64)
        fid[ti] = np.concatenate(w.fid)
        dkey[ti] = np.concatenate(w.dkey)
        assert np.array_equal(fid[ti], np.concatenate(w.fid)) and np.array_equal(dkey[ti], np.concatenate(w.dkey))
        dev = dev_tables["q"].device
        tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
        real = torch.from_numpy(np.arange(n)).to(dev)
        f = torch.from_numpy(fid[:n]).to(dev)
        d = torch.from_numpy(dkey[:n]).to(dev)

        def packed(table, rows, H):
            x = torch.zeros((R, H, w.D), device=dev, dtype=torch.float32)
            x[real] = table[rows]
            return x.to(tdt).view(1, R, H, w.D)

        self.q = packed(dev_tables["q"], f, w.Hq)
        self.k = packed(dev_tables["k"], f, w.Hkv)
        self.v = packed(dev_tables["v"], f, w.Hkv)
        self.do = packed(dev_tables["do"], d, w.Hq)
        self.se = torch.from_numpy(self.lay.subtree_end.astype(np.int32)).view(1, R).to(dev)
        pos = torch.from_numpy(self.lay.pos_ids.astype(np.int32)).view(1, R).to(dev)
        lib.tree_rope(self.q, pos, w.theta)
        lib.tree_rope(self.k, pos, w.theta)

    def forward(self):
        import prefix_tree_packed_dfs_amd as lib
        self.out, self.lse = lib.tree_attn_fwd(self.q, self.k, self.v, self.se)

    def backward(self, do):
        import prefix_tree_packed_dfs_amd as lib
        return lib.tree_attn_bwd(self.q, self.k, self.v, self.se, self.out, self.lse, do)


def _excess(a, b, dtype):
    """bf16: max of |a-b| - 2^-8 |b| (storage rounding taken out); f32: max|a-b| / max|b|."""
    a = a.float()
    b = b.float()
    if dtype == "bf16":
        return float(((a - b).abs() - HALF_ULP * b.abs()).max()) if a.numel() else 0.0
    den = float(b.abs().max()) if b.numel() else 0.0
    return float((a - b).abs().max()) / den if den > 0 else float((a - b).abs().max())


def _check(name, a, b, dtype):
    e = _excess(a, b, dtype)
    log(f"    {name:14s} excess={e:.3e}")
    assert e <= (BF16_ABS if dtype == "bf16" else F32_REL), f"{name}: {e}"


def _compare_layouts(w, label):
    import torch

    import prefix_tree_packed_dfs_amd as lib
    log(f"case {label}: dtype={w.dtype} Hq={w.Hq} Hkv={w.Hkv} D={w.D} seqs={len(w.sequences)} raw={w.raw_tokens} "
        f"seed={w.seed_base}")
    dev = torch.device("cuda", 0)
    tables = {k: torch.from_numpy(v).to(dev) for k, v in feature_tables(w).items()}
    tree = _Row(w, tables, *lib.tree_build_trie(w.sequences, min_shared=64))
    chains = _Row(w, tables, *sequence_packing_forest(w.sequences))
    assert chains.n == w.raw_tokens
    log(f"    forwarded {tree.n} of {w.raw_tokens} raw tokens (ratio {w.raw_tokens / max(tree.n, 1):.3f})")
    tree.forward()
    chains.forward()
    dq_t, dk_t, dv_t = tree.backward(tree.do)
    dq_all, _, _ = chains.backward(chains.do)

    ts = torch.from_numpy(tree.ti).to(dev)       # tree slot of raw token r
    cs = torch.from_numpy(chains.ti).to(dev)     # chain slot of raw token r
    first = np.zeros(len(tree.ti), bool)
    first[np.unique(tree.ti, return_index=True)[1]] = True
    fr = torch.from_numpy(first).to(dev)
    keep = torch.zeros(chains.R, device=dev, dtype=torch.bool)
    keep[cs[fr]] = True
    do_first = torch.where(keep.view(1, -1, 1, 1), chains.do, torch.zeros_like(chains.do))
    dq_1, dk_1, dv_1 = chains.backward(do_first)
    torch.cuda.synchronize()

    dt = w.dtype
    _check("out", chains.out[0, cs], tree.out[0, ts], dt)
    lse_d = float((chains.lse[0][:, cs] - tree.lse[0][:, ts]).abs().max())
    log(f"    {'lse':14s} max|d|={lse_d:.3e}")
    assert lse_d <= (LSE_ABS if dt == "bf16" else F32_REL * float(tree.lse[0][:, ts].abs().max()))
    _check("dq every copy", dq_all[0, cs], dq_t[0, ts], dt)
    _check("dq owner", dq_1[0, cs[fr]], dq_t[0, ts[fr]], dt)
    others = dq_1[0, cs[~fr]]
    log(f"    {'dq non-owner':14s} max|x|={float(others.float().abs().max()) if others.numel() else 0.0:.3e}")
    assert others.numel() == 0 or int((others != 0).sum()) == 0, "a copy without upstream gradient got dq != 0"
    for name, g_t, g_1 in (("dk", dk_t, dk_1), ("dv", dv_t, dv_1)):
        s = torch.zeros((tree.R,) + tuple(g_t.shape[2:]), device=dev, dtype=torch.float64)
        a = torch.zeros_like(s)
        s.index_add_(0, ts, g_1[0, cs].double())
        a.index_add_(0, ts, g_1[0, cs].double().abs())
        ref = g_t[0, :tree.n].double()
        d = (ref - s[:tree.n]).abs()
        if dt == "bf16":
            # one bf16 rounding per copy and one on the tree side
            e = float((d - HALF_ULP * (ref.abs() + a[:tree.n])).max())
            bar = BF16_ABS
        else:
            e = float(d.max()) / max(float(a[:tree.n].max()), 1e-30)
            bar = F32_REL
        log(f"    {name + ' = sum copies':14s} excess={e:.3e}")
        assert e <= bar, f"{name}: {e}"


def _random_workload(seed, dtype, Hq, Hkv, D, n_seqs=7, max_len=400, vocab=2, run=48):
    """Runs of a small alphabet: many forks, sequences ending at forks, duplicated sequences."""
    rng = np.random.default_rng(seed)
    seqs = []
    for _ in range(n_seqs):
        L = int(rng.integers(1, max_len))
        s = np.repeat(rng.integers(0, vocab, size=L // run + 1), run)[:L]
        seqs.append(s.astype(np.int32))
    seqs.append(seqs[0].copy())
    return from_sequences(seqs, Hq=Hq, Hkv=Hkv, D=D, dtype=dtype, seed_base=20_000 + seed)


@pytest.mark.parametrize("seed", range(4))
def test_random_trees_bf16(seed):
    _compare_layouts(_random_workload(seed, "bf16", 8, 2, 128), f"seqpack random bf16 seed {seed}")


@pytest.mark.parametrize("seed", range(2))
def test_random_trees_f32(seed):
    _compare_layouts(_random_workload(100 + seed, "f32", 4, 2, 64), f"seqpack random f32 seed {seed}")


def test_shared_history_ragged():
    _compare_layouts(shared_history(700, n=5, unique=333), "seqpack shared history 700 + 5 x 333")


def test_grpo_group_full():
    _compare_layouts(grpo_group(), "seqpack grpo_group (16 x (2048 + 1024))")


def test_agentic_trie_full():
    _compare_layouts(agentic_trie(), "seqpack agentic_trie (32K-slot trie)")


def test_long_history_full():
    _compare_layouts(long_history(), "seqpack long_history (20000 + 8 x 2000)")


def _chains_vs_oracle(w, label):
    """The sequence-packed row (one chain per sequence, plain varlen causal attention) through the C ABI
    against the oracle run on each sequence alone, token by token: out, lse, and with the upstream
    gradient on every token, dq, dk and dv of every copy.  The oracle shares no code with the layout or
    the kernels, so this checks the baseline side of the tree-vs-sequence-packing comparison directly."""
    import torch

    from oracle.attention import tree_attention
    log(f"case {label}: dtype={w.dtype} Hq={w.Hq} Hkv={w.Hkv} D={w.D} seqs={len(w.sequences)} raw={w.raw_tokens} "
        f"seed={w.seed_base}")
    dev = torch.device("cuda", 0)
    tables_np = feature_tables(w)
    tables = {k: torch.from_numpy(v).to(dev) for k, v in tables_np.items()}
    chains = _Row(w, tables, *sequence_packing_forest(w.sequences))
    assert chains.n == w.raw_tokens
    chains.forward()
    dq, dk, dv = chains.backward(chains.do)
    torch.cuda.synchronize()

    def host(t):
        return t[0].double().cpu().numpy()

    lib_t = {"out": host(chains.out), "lse": chains.lse[0].double().cpu().numpy(), "dq": host(dq), "dk": host(dk),
             "dv": host(dv)}
    got = {k: [] for k in lib_t}
    want = {k: [] for k in lib_t}

    def oracle_all():
        for s in range(len(w.sequences)):
            o = tree_attention([w.sequences[s]], [w.fid[s]], [w.dkey[s]], tables_np, theta=w.theta, storage=w.dtype)
            cs = chains.lay.sequence_slots(s).astype(np.int64)
            os_ = o.layout.token_index[0]
            for k in ("out", "dq", "dk", "dv"):
                got[k].append(lib_t[k][cs])
                want[k].append(getattr(o, k)[os_])
            got["lse"].append(lib_t["lse"][:, cs])
            want["lse"].append(o.lse[:, os_])

    timed("oracle, per sequence", oracle_all)
    rows = []
    for k in ("out", "lse", "dq", "dk", "dv"):
        ax = 1 if k == "lse" else 0
        rows.append(cmp(k, np.concatenate(got[k], axis=ax), np.concatenate(want[k], axis=ax),
                        w.dtype if k != "lse" else None))
    assert_within(w, rows)


def test_sequence_packing_vs_oracle_ragged():
    _chains_vs_oracle(shared_history(700, n=5, unique=333), "seqpack vs oracle: shared history 700 + 5 x 333")


def test_sequence_packing_vs_oracle_grpo_group_full():
    _chains_vs_oracle(grpo_group(), "seqpack vs oracle: grpo_group (16 x (2048 + 1024), 49,152-slot row)")
