"""GPU parity of gated-delta-rule mixing over packed trees: the C ABI against the oracle, and the tree
layout against sequence packing (every sequence its own chain) through the same kernels.

Every case prints its name, seed and shape before touching the GPU.
"""

import numpy as np
import pytest

from oracle.gdn import GdnShape, tree_gdn
from synth import from_sequences, gdn_tables, grpo_group, long_history, sequence_packing_forest

from .pipeline import log

pytestmark = pytest.mark.gpu

# bf16 output after bf16 operands with fp32 accumulation and an fp32 state: per value head,
# |a - b| <= REL * max|b| + 2^-8 |b| (the output's own storage rounding taken out), and cosine >= COS
REL = 2e-2
COS = 0.9999


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import prefix_tree_packed_dfs_amd  # noqa: F401  (fails loudly if the library is not built)
    yield


def _run(w, t, Hk, Hv, layout="tree", min_shared=64):
    import torch

    import prefix_tree_packed_dfs_amd as lib
    if layout == "tree":
        parent, seq_last = lib.tree_build_trie(w.sequences, min_shared=min_shared)
    else:
        parent, seq_last = sequence_packing_forest(w.sequences)
    n = len(parent)
    lay = lib.tree_pack_layout(parent, seq_last, n)
    ti = np.concatenate([lay.sequence_slots(s) for s in range(len(w.sequences))]).astype(np.int64)
    fid = np.full(n, -1, np.int64)
    fid[ti] = np.concatenate(w.fid)
    assert np.array_equal(fid[ti], np.concatenate(w.fid)) and np.all(fid >= 0)
    plan = lib.tree_gdn_plan(lay.subtree_end, n)
    dev = torch.device("cuda", 0)
    x = torch.from_numpy(t["x"][fid]).to(dev).to(torch.bfloat16)
    g = torch.from_numpy(t["g"][fid]).to(dev)
    beta = torch.from_numpy(t["beta"][fid]).to(dev)
    conv_w = torch.from_numpy(t["conv_w"]).to(dev)
    log(f"    {layout}: {n} slots, {plan.n_segments} chains, {plan.n_chunks} chunks, {plan.n_depths} depths")
    out = lib.tree_gdn_fwd(x, conv_w, g, beta, plan, Hk, Hv)
    torch.cuda.synchronize()
    return lay, out


def _token_slots(w, lay):
    return np.concatenate([lay.sequence_slots(s) for s in range(len(w.sequences))]).astype(np.int64)


def _check(name, a, b):
    """a (library) and b (reference) [tokens, heads, dv]; bar per head."""
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert np.all(np.isfinite(a)), f"{name}: non-finite library values"
    for h in range(b.shape[1]):
        ref = float(np.abs(b[:, h]).max())
        d = np.abs(a[:, h] - b[:, h])
        excess = float((d - 2.0 ** -8 * np.abs(b[:, h])).max())
        cos = float((a[:, h] * b[:, h]).sum() / max(np.linalg.norm(a[:, h]) * np.linalg.norm(b[:, h]), 1e-300))
        log(f"    {name} head {h}: max|d|={d.max():.3e} max|ref|={ref:.3e} excess/ref={excess / max(ref, 1e-30):.3e} "
            f"cos={cos:.8f}")
        assert excess <= REL * ref, f"{name} head {h}: {excess} > {REL} * {ref}"
        assert cos >= COS, f"{name} head {h}: cosine {cos}"


def _vs_oracle(w, Hk, Hv, label, *, W=4, min_shared=64, heads=None, seqs=None):
    import torch
    log(f"case {label}: Hk={Hk} Hv={Hv} seqs={len(w.sequences)} raw={w.raw_tokens} seed={w.seed_base} W={W} "
        f"min_shared={min_shared}")
    t = gdn_tables(w, Hk=Hk, Hv=Hv, conv_width=W)
    lay, out = _run(w, t, Hk, Hv, min_shared=min_shared)
    shape = GdnShape(Hk=Hk, Hv=Hv, dk=128, dv=128)
    r = tree_gdn(w.sequences, w.fid, t, t["conv_w"], shape, min_shared=min_shared, storage="bf16", heads=heads,
                 seqs=seqs)
    assert r.max_shared_gap == 0.0
    ss = range(len(w.sequences)) if seqs is None else seqs
    a_slots = np.concatenate([lay.sequence_slots(s) for s in ss]).astype(np.int64)
    b_slots = np.concatenate([r.layout.token_index[s] for s in ss]).astype(np.int64)
    got = out[torch.from_numpy(a_slots).to(out.device)].float().cpu().numpy()[:, r.heads]
    _check("out", got, r.out[b_slots])


def _small_alphabet(seed, n_seqs=7, max_len=300, run=24):
    rng = np.random.default_rng(seed)
    seqs = []
    for _ in range(n_seqs):
        L = int(rng.integers(1, max_len))
        seqs.append(np.repeat(rng.integers(0, 2, size=L // run + 1), run)[:L].astype(np.int32))
    seqs.append(seqs[0].copy())
    return seqs


@pytest.mark.parametrize("seed", range(4))
def test_random_tries(seed):
    w = from_sequences(_small_alphabet(seed), Hq=1, Hkv=1, D=8, dtype="bf16", seed_base=40_000 + seed)
    _vs_oracle(w, 1, 2, f"gdn random trie seed {seed}", min_shared=2 + seed)


def test_deep_trie_many_depths():
    """Forks every 20 tokens: chains of 20, a dozen depths, several chains per depth."""
    w = from_sequences(_small_alphabet(11, n_seqs=12, max_len=400, run=20), Hq=1, Hkv=1, D=8, dtype="bf16",
                       seed_base=40_100)
    _vs_oracle(w, 2, 4, "gdn deep trie", min_shared=1)


@pytest.mark.parametrize("W", [1, 2, 3, 4])
def test_conv_widths_on_a_group(W):
    w = grpo_group(seed_base=40_200, prompt=300, n=4, completion=150, Hq=1, Hkv=1, D=8, row_len=None)
    _vs_oracle(w, 2, 4, f"gdn grpo group width {W}", W=W)


def test_chains_of_64_and_65_and_one_token():
    seqs = [np.arange(64, dtype=np.int32), np.arange(1000, 1065, dtype=np.int32), np.array([7], np.int32),
            np.arange(2000, 2001 + 700, dtype=np.int32)]
    w = from_sequences(seqs, Hq=1, Hkv=1, D=8, dtype="bf16", seed_base=40_300)
    _vs_oracle(w, 1, 2, "gdn chains 64, 65, 1, 701")


def test_one_token_row():
    w = from_sequences([np.array([3], np.int32)], Hq=1, Hkv=1, D=8, dtype="bf16", seed_base=40_400)
    _vs_oracle(w, 1, 1, "gdn one token")


def test_tree_equals_sequence_packing_on_random_tries():
    for seed in range(3):
        w = from_sequences(_small_alphabet(50 + seed), Hq=1, Hkv=1, D=8, dtype="bf16", seed_base=40_500 + seed)
        log(f"case gdn tree vs sequence packing seed {seed}: raw={w.raw_tokens}")
        t = gdn_tables(w, Hk=1, Hv=2)
        lt, ot = _run(w, t, 1, 2, min_shared=2)
        lc, oc = _run(w, t, 1, 2, layout="chains")
        a = ot.float().cpu().numpy()[_token_slots(w, lt)]
        b = oc.float().cpu().numpy()[_token_slots(w, lc)]
        _check("tree vs chains", a, b)


def test_full_grpo_group_sampled_vs_oracle():
    """16 x (2,048 + 1,024) tokens, 16 key / 32 value heads: two sequences, three heads against the oracle."""
    w = grpo_group()
    _vs_oracle(w, 16, 32, "gdn grpo_group full size", heads=[0, 17, 31], seqs=[0, 9])


def test_full_long_history_tree_equals_sequence_packing():
    """20,000 shared tokens + 8 x 2,000: the tree row (36,007 slots) against 176,000 sequence-packed slots."""
    import torch
    w = long_history(Hq=1, Hkv=1, D=8)
    log(f"case gdn long_history tree vs sequence packing: raw={w.raw_tokens}")
    t = gdn_tables(w, Hk=4, Hv=8)
    lt, ot = _run(w, t, 4, 8)
    lc, oc = _run(w, t, 4, 8, layout="chains")
    dev = ot.device
    a = ot[torch.from_numpy(_token_slots(w, lt)).to(dev)].float().cpu().numpy()
    b = oc[torch.from_numpy(_token_slots(w, lc)).to(dev)].float().cpu().numpy()
    _check("tree vs chains", a, b)
