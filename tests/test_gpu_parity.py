"""GPU parity: the HIP path through the C ABI against the oracle.

Every case prints its name, seed and shape before touching the GPU.
"""

import numpy as np
import pytest

from synth import (agentic_trie, feature_tables, from_sequences, grpo_group, independent, long_history,
                   standard, tiny_tree)

from .pipeline import assert_within, cmp, compare, log, run_library, run_oracle, timed

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import prefix_tree_packed_dfs_amd  # noqa: F401  (fails loudly if the library is not built)
    yield


def _random_workload(seed, dtype, Hq, Hkv, D, n_seqs=6, max_len=300, vocab=2, fork_every=40):
    """Sequences over a small alphabet of long runs: many forks, short and long shared runs."""
    rng = np.random.default_rng(seed)
    seqs = []
    for _ in range(n_seqs):
        L = int(rng.integers(1, max_len))
        # runs of a repeated symbol: agreement over long stretches, then forks
        s = np.repeat(rng.integers(0, vocab, size=L // fork_every + 1), fork_every)[:L]
        seqs.append(s.astype(np.int32))
    return from_sequences(seqs, Hq=Hq, Hkv=Hkv, D=D, dtype=dtype, seed_base=10_000 + seed)


def _run_full(w, rope=True, label="", ws_mode=None):
    log(f"case {label or w.name}: dtype={w.dtype} Hq={w.Hq} Hkv={w.Hkv} D={w.D} seqs={len(w.sequences)} "
        f"raw={w.raw_tokens} seed={w.seed_base} bwd workspace={ws_mode or 'largest'}")
    tables = feature_tables(w)
    lres = timed("library", run_library, w, tables, rope=rope, ws_mode=ws_mode)
    ores = timed("oracle", run_oracle, w, tables, rope=rope, R=lres.R)
    rows = compare(w, lres, ores)
    assert_within(w, rows)
    return lres, ores


# ---------------------------------------------------------------------------
# rotary embedding alone
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("dtype,D", [("f32", 64), ("f32", 128), ("bf16", 64), ("bf16", 128)])
def test_rope_matches_oracle(dtype, D):
    import torch

    import prefix_tree_packed_dfs_amd as lib
    from oracle.precision import round_to
    from oracle.rope import rope

    log(f"case rope dtype={dtype} D={D}")
    rng = np.random.default_rng(D)
    N, H = 1000, 3
    x = rng.standard_normal((N, H, D)).astype(np.float32)
    pos = rng.integers(0, 40000, size=N).astype(np.int32)
    pos[:5] = [0, 1, 2, 36863, 32767]
    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    xt = torch.from_numpy(x).to(tdt)
    x_in = xt.to(torch.float64).numpy()
    dev = xt.view(1, N, H, D).cuda()
    lib.tree_rope(dev, torch.from_numpy(pos).view(1, N).cuda(), 10000.0)
    got = dev[0].to(torch.float64).cpu().numpy()
    want = round_to(rope(x_in, pos, 10000.0), dtype)
    ulp = np.abs(want) * (2.0**-23 if dtype == "f32" else 2.0**-7) + 1e-30
    diff = np.abs(got - want)
    log(f"    exact {np.mean(diff == 0):.6f}, max diff/ulp {np.max(diff / ulp):.3f}")
    assert np.all(diff <= ulp * 1.0001)
    assert np.mean(diff == 0) > 0.999
    assert np.array_equal(got[pos == 0], x_in[pos == 0])


@pytest.mark.gpu
@pytest.mark.parametrize("dtype,D,Hq,Hkv", [("bf16", 128, 16, 8), ("bf16", 64, 3, 1), ("f32", 128, 4, 2),
                                            ("bf16", 128, 0, 2), ("bf16", 128, 2, 0)])
def test_rope_qk_equals_rope_on_each(dtype, D, Hq, Hkv):
    """tree_rope_qk is tree_rope(q) then tree_rope(k), bit for bit (tree_rope is pinned to the oracle above)."""
    import torch

    import prefix_tree_packed_dfs_amd as lib

    log(f"case rope_qk dtype={dtype} D={D} Hq={Hq} Hkv={Hkv}")
    rng = np.random.default_rng(D + 7 * Hq + Hkv)
    N = 1500
    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    q = torch.from_numpy(rng.standard_normal((1, N, Hq, D)).astype(np.float32)).to(tdt).cuda()
    k = torch.from_numpy(rng.standard_normal((1, N, Hkv, D)).astype(np.float32)).to(tdt).cuda()
    pos = rng.integers(0, 40000, size=N).astype(np.int32)
    pos[:4] = [0, 1, 36863, 0]
    pos_d = torch.from_numpy(pos).view(1, N).cuda()
    q1, k1 = q.clone(), k.clone()
    lib.tree_rope(q1, pos_d, 10000.0)
    lib.tree_rope(k1, pos_d, 10000.0)
    lib.tree_rope_qk(q, k, pos_d, 10000.0)
    torch.cuda.synchronize()
    assert torch.equal(q, q1)
    assert torch.equal(k, k1)


@pytest.mark.gpu
def test_rope_qk_rejects_aliased_q_and_k():
    import torch

    import prefix_tree_packed_dfs_amd as lib

    x = torch.zeros((1, 8, 2, 64), dtype=torch.bfloat16, device="cuda")
    pos = torch.zeros((1, 8), dtype=torch.int32, device="cuda")
    with pytest.raises(lib.TreeAttnError):
        lib.tree_rope_qk(x, x, pos, 10000.0)


# ---------------------------------------------------------------------------
# small trees, every element compared
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("seed", range(6))
def test_random_trees_f32(seed):
    w = _random_workload(seed, "f32", Hq=2, Hkv=2, D=64)
    _run_full(w, label=f"random_tree_f32[{seed}]")


@pytest.mark.parametrize("seed", range(6))
def test_random_trees_bf16_gqa(seed):
    w = _random_workload(100 + seed, "bf16", Hq=4, Hkv=2, D=128)
    _run_full(w, label=f"random_tree_bf16[{seed}]")


@pytest.mark.parametrize("rope", [False, True])
def test_random_tree_bf16_no_rope_and_rope(rope):
    w = _random_workload(500, "bf16", Hq=8, Hkv=2, D=128, n_seqs=9, max_len=700)
    _run_full(w, rope=rope, label=f"random_tree_bf16_rope={rope}")


@pytest.mark.parametrize("Hq,Hkv,D", [(2, 2, 64), (4, 1, 64), (8, 1, 128), (16, 2, 128), (32, 2, 64), (3, 3, 128),
                                     (6, 2, 64), (6, 2, 128)])
def test_random_tree_bf16_head_shapes(Hq, Hkv, D):
    """Every GQA grouping the matrix-core kernels specialise (1, 4, 8 heads per KV head, and 16 as two
    workgroups of 8), head dim 64, and a ratio they do not cover (3 KV heads of 1), which runs on the
    vector path."""
    w = _random_workload(700 + Hq * 10 + D, "bf16", Hq=Hq, Hkv=Hkv, D=D, n_seqs=7, max_len=400)
    _run_full(w, label=f"random_tree_bf16_Hq{Hq}_Hkv{Hkv}_D{D}")


def test_degenerate_rows():
    # a single token; a single chain shorter than a tile; a row that is all padding but one slot
    for seqs in ([[5]], [list(range(37))], [[1, 2], [1, 3]]):
        w = from_sequences(seqs, Hq=2, Hkv=1, D=128, dtype="bf16", seed_base=77, row_len=130)
        _run_full(w, label=f"degenerate{[len(s) for s in seqs]}")


# ---------------------------------------------------------------------------
# the five workloads, shrunk: same structure and head shapes, several tiles and ragged tails
# ---------------------------------------------------------------------------

SHRUNK = {
    "tiny_tree": lambda: tiny_tree(),
    "grpo_group": lambda: grpo_group(prompt=300, n=5, completion=150, row_len=None),
    "agentic_trie": lambda: agentic_trie(budget=3000, seg_lo=64, seg_hi=400, ratio_lo=1.5, ratio_hi=9.0,
                                         row_len=3072),
    "independent": lambda: independent(n=7, length=200, row_len=1408),
    "long_history": lambda: long_history(prefix=1000, n=4, unique=300, row_len=None),
}


@pytest.mark.parametrize("name", list(SHRUNK))
def test_shrunk_workloads(name):
    _run_full(SHRUNK[name](), label=f"shrunk_{name}")


# ---------------------------------------------------------------------------
# full sizes
# ---------------------------------------------------------------------------

def test_full_c1_tiny_fp32():
    _run_full(standard(1), label="full_tiny_tree")


def test_full_c2_grpo():
    _run_full(standard(2), label="full_grpo_group")


def test_full_c4_independent():
    _run_full(standard(4), label="full_independent")


def _run_sampled(w, label, n_q=256, tail=256):
    from oracle.layout import dfs_layout
    from oracle.trie import build_trie

    log(f"case {label}: dtype={w.dtype} Hq={w.Hq} Hkv={w.Hkv} D={w.D} seqs={len(w.sequences)} "
        f"raw={w.raw_tokens} (sampled)")
    tables = feature_tables(w)
    lres = timed("library", run_library, w, tables)
    trie = build_trie(w.sequences)
    olay = dfs_layout(trie.parent, trie.seq_last, lres.R)
    rng = np.random.default_rng(w.seed_base)
    qs_lib, qs_ora, ks_lib, ks_ora = [], [], [], []
    for _ in range(n_q):                     # uniformly random tokens: out, lse, dq
        s = int(rng.integers(len(w.sequences)))
        t = int(rng.integers(len(w.sequences[s])))
        qs_lib.append(lres.layout.sequence_slots(s)[t])
        qs_ora.append(olay.token_index[s][t])
    for s in range(len(w.sequences)):        # keys near the end of every sequence: dk, dv
        L = len(w.sequences[s])
        for t in rng.choice(np.arange(max(0, L - tail), L), size=min(16, L), replace=False):
            ks_lib.append(lres.layout.sequence_slots(s)[t])
            ks_ora.append(olay.token_index[s][t])
    ores = timed("oracle", run_oracle, w, tables, R=lres.R, q_slots=np.unique(qs_ora), k_slots=np.unique(ks_ora))
    rows = compare(w, lres, ores, lib_slots=np.unique(qs_lib), key_slots=np.unique(ks_lib))
    assert_within(w, rows)
    # properties that hold at any size, over every slot
    n = lres.n
    G = w.Hq // w.Hkv
    do_sum = _dout_sum(w, tables, lres)
    assert np.allclose(lres.dv[:n].sum(axis=0), do_sum, atol=0.05 * np.abs(do_sum).max() + 0.5)
    assert np.abs(lres.dk[:n].sum(axis=0)).max() < 0.05 * np.sqrt(n * G)
    assert np.all(np.isfinite(lres.out[:n])) and np.all(np.isfinite(lres.dq[:n]))
    return lres, tables


def _check_shared_keys(w, lres, tables, label, per_group=16, kv_head=0):
    """dk, dv at keys many queries see, against the oracle restricted to one KV head (its whole
    query-head group, so each output is exact): random keys of the segment every sequence shares
    (the root), the deepest 512 of them (the end of a shared history), and keys of segments shared by
    some sequences but not all (inner segments).  These keys carry most of the dK/dV work, and on long
    rows their key tiles are the ones the dK/dV plan cuts into chunks whose partial sums are added by
    the reduce pass."""
    from oracle.layout import dfs_layout
    from oracle.trie import build_trie

    n_seqs = len(w.sequences)
    counts = np.zeros(lres.R, np.int64)
    for s in range(n_seqs):
        counts[lres.layout.sequence_slots(s)] += 1
    real = np.arange(lres.n)
    root = real[counts[:lres.n] == n_seqs]
    inner = real[(counts[:lres.n] >= 2) & (counts[:lres.n] < n_seqs)]
    rng = np.random.default_rng(w.seed_base + 7)
    picks = []
    if len(root):
        picks += list(rng.choice(root, min(per_group, len(root)), replace=False))
        deep = root[np.argsort(lres.layout.pos_ids[root], kind="stable")[-512:]]
        picks += list(rng.choice(deep, min(per_group, len(deep)), replace=False))
    if len(inner):
        picks += list(rng.choice(inner, min(per_group, len(inner)), replace=False))
    picks = np.unique(np.asarray(picks, np.int64))
    assert len(picks), "no shared keys"
    # library slot -> oracle slot through the sequences' paths
    trie = build_trie(w.sequences)
    olay = dfs_layout(trie.parent, trie.seq_last, lres.R)
    m = np.full(lres.R, -1, np.int64)
    for s in range(n_seqs):
        m[lres.layout.sequence_slots(s)] = olay.token_index[s]
    depths = lres.layout.pos_ids[picks]
    log(f"  shared keys {label}: {len(picks)} keys (root {len(root)}, inner {len(inner)} slots), depths "
        f"{int(depths.min())}..{int(depths.max())}, KV head {kv_head}")
    ores = timed("oracle, one KV head", run_oracle, w, tables, R=lres.R, k_slots=m[picks], kv_heads=[kv_head])
    rows = [cmp("dk@shared", lres.dk[picks, kv_head], ores.dk[m[picks], kv_head], w.dtype),
            cmp("dv@shared", lres.dv[picks, kv_head], ores.dv[m[picks], kv_head], w.dtype)]
    assert_within(w, rows)


def _dout_sum(w, tables, lres):
    """Sum over packed slots of dout, per KV head group: equals sum_j dV[j] (softmax rows sum to one)."""
    from .pipeline import slot_rows
    _, dkey_slot = slot_rows(w, lres.layout, lres.n)
    do = tables["do"][dkey_slot[:lres.n]].astype(np.float64)
    return do.reshape(lres.n, w.Hkv, w.Hq // w.Hkv, w.D).sum(axis=(0, 2))


def test_long_chain_beyond_one_tile_list_sampled():
    """One 70,000-token sequence: the query blocks near its end see more than 1,024 key tiles, so the
    visible-tile list is built in several passes, and every key tile's query range is split for dK/dV."""
    w = from_sequences([np.arange(70_000, dtype=np.int32)], Hq=2, Hkv=1, D=64, dtype="bf16", seed_base=15_000,
                       row_len=70_016)
    _run_sampled(w, "long_chain_70000")


def test_full_c3_agentic_sampled():
    w = standard(3)
    lres, tables = _run_sampled(w, "full_agentic_trie")
    _check_shared_keys(w, lres, tables, "full_agentic_trie")


def test_full_c5_long_history_sampled():
    w = standard(5)
    lres, tables = _run_sampled(w, "full_long_history")
    _check_shared_keys(w, lres, tables, "full_long_history")


def _split_prompt(tail=300, prompt=4000, n=4):
    rng = np.random.default_rng(31)
    base = np.arange(prompt, dtype=np.int32)
    seqs = [np.concatenate([base, 10_000 + 1000 * i + rng.permutation(tail).astype(np.int32)]) for i in range(n)]
    return from_sequences(seqs, Hq=32, Hkv=8, D=128, dtype="bf16", seed_base=16_000, name="split_prompt")


@pytest.mark.parametrize("ws_mode", [None, "fixed"])
def test_split_prompt_tiles_gqa4_every_element(ws_mode):
    """A 4,000-token prompt and four 300-token tails at 32 query / 8 KV heads, every element against
    the oracle.  Four query heads per KV head make the dK/dV plan's chunk 80 query blocks, so the
    prompt's key tiles (whose keys every tail sees) are cut into chunks that write partial sums and the
    reduce pass adds them; with the fixed-only workspace nothing is cut and each tile is one unit."""
    import prefix_tree_packed_dfs_amd as lib
    w = _split_prompt()
    parent, seq_last = lib.tree_build_trie(w.sequences, min_shared=64)
    R = w.row_length(len(parent))
    se = lib.tree_pack_layout(parent, seq_last, R).subtree_end
    slots = (lib.tree_attn_bwd_workspace_bytes_for(lib.TREE_BF16, se, w.Hq, w.Hkv, w.D)
             - lib.tree_attn_bwd_workspace_bytes_for(lib.TREE_BF16, np.arange(R, dtype=np.int32), w.Hq, w.Hkv, w.D)
             ) // (2 * 256 * 128 * 4)
    log(f"  split_prompt: {len(parent)} slots, the plan takes {slots} partial-sum slots")
    assert slots > 0
    _run_full(w, label=f"split_prompt_gqa4[{ws_mode or 'largest'}]", ws_mode=ws_mode)


def test_backward_workspace_exact_size_gives_the_same_results():
    """grpo_group at full size: the backward with the exact workspace of its plan is bitwise the
    backward with the largest workspace (the same plan); with the fixed part only, nothing is cut into
    chunks and the results differ by the order of summation only."""
    import torch

    import prefix_tree_packed_dfs_amd as lib
    from .pipeline import bwd_workspace
    w = standard(2)
    log(f"case workspace sizes: {w.name} Hq={w.Hq} Hkv={w.Hkv} D={w.D}")
    parent, seq_last = lib.tree_build_trie(w.sequences, min_shared=64)
    R = w.row_length(len(parent))
    lay = lib.tree_pack_layout(parent, seq_last, R)
    se = torch.from_numpy(lay.subtree_end.astype(np.int32)).view(1, R).cuda()
    g = torch.Generator().manual_seed(9)
    mk = lambda H: torch.randn(1, R, H, w.D, generator=g).to(torch.bfloat16).cuda()  # noqa: E731
    q, k, v, do = mk(w.Hq), mk(w.Hkv), mk(w.Hkv), mk(w.Hq)
    out, lse = lib.tree_attn_fwd(q, k, v, se)
    res = {}
    for mode in (None, "exact", "fixed"):
        ws = bwd_workspace(w, lay, R, mode)
        res[mode] = lib.tree_attn_bwd(q, k, v, se, out, lse, do, ws=ws)
        torch.cuda.synchronize()
        log(f"    {mode or 'largest'}: {ws.numel() if ws is not None else 'default'} bytes")
    for a, b in zip(res[None], res["exact"]):
        assert torch.equal(a, b)
    for a, b in zip(res[None], res["fixed"]):
        a, b = a.float(), b.float()
        e = float(((a - b).abs() - 2.0 ** -7 * b.abs()).max())
        log(f"    fixed-only vs largest: max|d| {float((a - b).abs().max()):.3e}, beyond one ulp {e:.3e}")
        assert e <= 1e-2


@pytest.mark.gpu
def test_backward_reads_no_workspace_it_did_not_write():
    """grpo_group at full size (its padding rows after the last real keys included): the backward
    with its workspace filled with zeros and with 0xFF bytes (NaN as fp32) before the call gives
    bitwise the same dq, dk, dv, so every workspace word a kernel reads was written in the call."""
    import torch

    import prefix_tree_packed_dfs_amd as lib
    w = standard(2)
    log(f"case workspace contents: {w.name} Hq={w.Hq} Hkv={w.Hkv} D={w.D}")
    parent, seq_last = lib.tree_build_trie(w.sequences, min_shared=64)
    n = len(parent)
    R = w.row_length(n)
    assert R - n >= 256, "the row needs padding past a 256-key tile"
    lay = lib.tree_pack_layout(parent, seq_last, R)
    se = torch.from_numpy(lay.subtree_end.astype(np.int32)).view(1, R).cuda()
    g = torch.Generator().manual_seed(13)
    mk = lambda H: torch.randn(1, R, H, w.D, generator=g).to(torch.bfloat16).cuda()  # noqa: E731
    q, k, v, do = mk(w.Hq), mk(w.Hkv), mk(w.Hkv), mk(w.Hq)
    out, lse = lib.tree_attn_fwd(q, k, v, se)
    nbytes = lib.tree_attn_bwd_workspace_bytes_for(lib.TREE_BF16, lay.subtree_end.astype(np.int32), w.Hq,
                                                   w.Hkv, w.D)
    res = []
    for fill in (0x00, 0xFF):
        ws = torch.full((nbytes,), fill, dtype=torch.uint8, device="cuda")
        res.append(lib.tree_attn_bwd(q, k, v, se, out, lse, do, ws=ws))
        torch.cuda.synchronize()
    for name, a, b in zip(("dq", "dk", "dv"), res[0], res[1]):
        assert torch.isfinite(a.float()).all(), name
        assert torch.equal(a, b), name


def test_outputs_stay_inside_their_buffers():
    """Guard bands of sentinel values before and after out, lse, dq, dk, dv and both workspaces
    (grpo_group at full size, each buffer a view into a larger one): after the forward and the
    backward every sentinel is still there, and every output element was written."""
    import torch

    import prefix_tree_packed_dfs_amd as lib
    w = standard(2)
    log(f"case guard bands: {w.name}")
    parent, seq_last = lib.tree_build_trie(w.sequences, min_shared=64)
    R = w.row_length(len(parent))
    lay = lib.tree_pack_layout(parent, seq_last, R)
    se = torch.from_numpy(lay.subtree_end.astype(np.int32)).view(1, R).cuda()
    g = torch.Generator().manual_seed(10)
    mk = lambda H: torch.randn(1, R, H, w.D, generator=g).to(torch.bfloat16).cuda()  # noqa: E731
    q, k, v, do = mk(w.Hq), mk(w.Hkv), mk(w.Hkv), mk(w.Hq)
    GUARD = 4096
    bands = []

    def guarded(shape, dtype, sentinel):
        numel = int(np.prod(shape))
        full = torch.full((GUARD + numel + GUARD,), sentinel, dtype=dtype, device="cuda")
        bands.append((full, numel, sentinel))
        return full[GUARD:GUARD + numel].view(shape)

    NAN16 = float("nan")
    out = guarded((1, R, w.Hq, w.D), torch.bfloat16, NAN16)
    lse = guarded((1, w.Hq, R), torch.float32, float("nan"))
    dq = guarded((1, R, w.Hq, w.D), torch.bfloat16, NAN16)
    dk = guarded((1, R, w.Hkv, w.D), torch.bfloat16, NAN16)
    dv = guarded((1, R, w.Hkv, w.D), torch.bfloat16, NAN16)
    wsf = guarded((lib.tree_attn_workspace_bytes(lib.TREE_BF16, 1, R, w.Hq, w.Hkv, w.D, False),), torch.uint8, 0xA5)
    wsb = guarded((lib.tree_attn_bwd_workspace_bytes_for(lib.TREE_BF16, lay.subtree_end, w.Hq, w.Hkv, w.D),),
                  torch.uint8, 0x5A)
    lib.tree_attn_fwd(q, k, v, se, out=out, lse=lse, ws=wsf)
    lib.tree_attn_bwd(q, k, v, se, out, lse, do, dq=dq, dk=dk, dv=dv, ws=wsb)
    torch.cuda.synchronize()
    for full, numel, sentinel in bands:
        for part in (full[:GUARD], full[GUARD + numel:]):
            if isinstance(sentinel, float) and np.isnan(sentinel):
                assert bool(torch.isnan(part.float()).all()), "a guard band was written"
            else:
                assert bool((part == sentinel).all()), "a guard band was written"
    for t in (out, lse, dq, dk, dv):
        assert not bool(torch.isnan(t.float()).any()), "an output element was not written"
    log(f"    {len(bands)} buffers: guard bands intact, every output element written")


# ---------------------------------------------------------------------------
# batch of rows, determinism
# ---------------------------------------------------------------------------

def test_batch_rows_are_independent_and_deterministic():
    import torch

    import prefix_tree_packed_dfs_amd as lib
    log("case batch_of_two_rows")
    R = 1024
    rows = []
    for seed in (1, 2):
        w = _random_workload(900 + seed, "bf16", Hq=4, Hkv=2, D=128, n_seqs=5, max_len=500)
        parent, seq_last = lib.tree_build_trie(w.sequences)
        lay = lib.tree_pack_layout(parent, seq_last, R)
        rows.append(lay.subtree_end)
    g = torch.Generator().manual_seed(3)
    q = torch.randn(2, R, 4, 128, generator=g).to(torch.bfloat16).cuda()
    k = torch.randn(2, R, 2, 128, generator=g).to(torch.bfloat16).cuda()
    v = torch.randn(2, R, 2, 128, generator=g).to(torch.bfloat16).cuda()
    do = torch.randn(2, R, 4, 128, generator=g).to(torch.bfloat16).cuda()
    se = torch.from_numpy(np.stack(rows).astype(np.int32)).cuda()
    out, lse = lib.tree_attn_fwd(q, k, v, se)
    grads = lib.tree_attn_bwd(q, k, v, se, out, lse, do)
    out2, lse2 = lib.tree_attn_fwd(q, k, v, se)
    assert torch.equal(out, out2) and torch.equal(lse, lse2)
    for b in range(2):
        o1, l1 = lib.tree_attn_fwd(q[b:b + 1].contiguous(), k[b:b + 1].contiguous(), v[b:b + 1].contiguous(),
                                   se[b:b + 1].contiguous())
        assert torch.equal(o1[0], out[b]) and torch.equal(l1[0], lse[b])
        g1 = lib.tree_attn_bwd(q[b:b + 1].contiguous(), k[b:b + 1].contiguous(), v[b:b + 1].contiguous(),
                               se[b:b + 1].contiguous(), o1, l1, do[b:b + 1].contiguous())
        for x, y in zip(g1, grads):
            assert torch.allclose(x[0].float(), y[b].float(), atol=1e-2, rtol=0)


def test_batch_rows_of_very_different_lengths():
    """Two rows of 2,048 slots in one call: one holds a 120-token tree and is padding past it, the other
    is nearly full.  The kernels give work items to query blocks up to the last tile of any row with a
    non-isolated slot, so the short row's padding blocks are items (that return at once) in the batch
    call and no items in its own call: both calls must give the same results, and the short row must
    match the oracle."""
    import torch

    import prefix_tree_packed_dfs_amd as lib
    log("case batch_of_a_short_and_a_full_row")
    R = 2048
    short = _random_workload(931, "bf16", Hq=8, Hkv=4, D=128, n_seqs=3, max_len=120)
    full = _random_workload(932, "bf16", Hq=8, Hkv=4, D=128, n_seqs=9, max_len=700, fork_every=64)
    rows = []
    for w in (short, full):
        parent, seq_last = lib.tree_build_trie(w.sequences)
        assert len(parent) <= R
        rows.append(lib.tree_pack_layout(parent, seq_last, R).subtree_end)
    log(f"  real slots per row: {[int((se != np.arange(R)).sum()) for se in rows]}")
    g = torch.Generator().manual_seed(5)
    q = torch.randn(2, R, 8, 128, generator=g).to(torch.bfloat16).cuda()
    k = torch.randn(2, R, 4, 128, generator=g).to(torch.bfloat16).cuda()
    v = torch.randn(2, R, 4, 128, generator=g).to(torch.bfloat16).cuda()
    do = torch.randn(2, R, 8, 128, generator=g).to(torch.bfloat16).cuda()
    se = torch.from_numpy(np.stack(rows).astype(np.int32)).cuda()
    out, lse = lib.tree_attn_fwd(q, k, v, se)
    grads = lib.tree_attn_bwd(q, k, v, se, out, lse, do)
    for b in range(2):
        one = [t[b:b + 1].contiguous() for t in (q, k, v, se)]
        o1, l1 = lib.tree_attn_fwd(*one)
        assert torch.equal(o1[0], out[b]) and torch.equal(l1[0], lse[b])
        g1 = lib.tree_attn_bwd(*one, o1, l1, do[b:b + 1].contiguous())
        for x, y in zip(g1, grads):
            assert torch.isfinite(y[b].float()).all()
            assert torch.allclose(x[0].float(), y[b].float(), atol=1e-2, rtol=0)
    short.row_len = R  # against the oracle in its 2,048-slot row, padding included
    _run_full(short, label="short_row_alone")


# ---------------------------------------------------------------------------
# isolated slots (each sees only itself): one-token sequences and padding
# ---------------------------------------------------------------------------

def _trees_around_singles(seed, n_single):
    """Two random tries with n_single one-token sequences between them in the DFS order (roots are
    ordered by first token): long runs of isolated slots, so whole query blocks and key tiles of the
    kernels hold nothing else, next to blocks that mix them with tree tokens."""
    rng = np.random.default_rng(seed)
    seqs = []
    for lo in (0, 50_000):
        for _ in range(4):
            L = int(rng.integers(60, 400))
            s = np.repeat(rng.integers(0, 2, size=L // 40 + 1), 40)[:L].astype(np.int32) + lo
            seqs.append(s)
    singles = [np.array([1000 + i], np.int32) for i in range(n_single)]
    return seqs[:4] + singles + seqs[4:]


@pytest.mark.parametrize("Hq,Hkv,D", [(2, 2, 64), (4, 2, 128), (16, 2, 128)])
def test_isolated_tokens_between_trees(Hq, Hkv, D):
    w = from_sequences(_trees_around_singles(Hq + D, 700), Hq=Hq, Hkv=Hkv, D=D, dtype="bf16",
                       seed_base=12_000 + Hq + D, row_len=4608)
    _run_full(w, label=f"isolated_tokens_Hq{Hq}_Hkv{Hkv}_D{D}")


def test_padding_slots_attend_to_themselves():
    """grpo_group at full size (18,447 tokens in a 32,768-slot row) with random values in the padding
    slots too: a padding slot is isolated (subtree_end[j] = j), so its softmax has one term --
    out = v, lse = scale q.k, dq = dk = 0 and dv = the sum of its group's dout rows -- and the
    real slots' results do not depend on what the padding holds."""
    import torch

    import prefix_tree_packed_dfs_amd as lib
    w = standard(2)
    log(f"case padding_slots: {w.name} Hq={w.Hq} Hkv={w.Hkv} D={w.D}")
    parent, seq_last = lib.tree_build_trie(w.sequences, min_shared=64)
    n = len(parent)
    R = w.row_length(n)
    lay = lib.tree_pack_layout(parent, seq_last, R)
    se = torch.from_numpy(lay.subtree_end.astype(np.int32)).view(1, R).cuda()
    g = torch.Generator().manual_seed(5)
    mk = lambda H: torch.randn(1, R, H, w.D, generator=g).to(torch.bfloat16)  # noqa: E731
    q, k, v, do = mk(w.Hq), mk(w.Hkv), mk(w.Hkv), mk(w.Hq)
    res = []
    for zero_pad in (False, True):
        t = [x.clone() for x in (q, k, v, do)]
        if zero_pad:
            for x in t:
                x[:, n:] = 0
        t = [x.cuda() for x in t]
        out, lse = lib.tree_attn_fwd(t[0], t[1], t[2], se)
        dq, dk, dv = lib.tree_attn_bwd(t[0], t[1], t[2], se, out, lse, t[3])
        torch.cuda.synchronize()
        res.append([x.cpu() for x in (out, lse, dq, dk, dv)])
    (out, lse, dq, dk, dv), (out0, lse0, dq0, dk0, dv0) = res
    # real slots: identical whatever the padding holds
    assert torch.equal(out[:, :n], out0[:, :n]) and torch.equal(lse[:, :, :n], lse0[:, :, :n])
    assert torch.equal(dq[:, :n], dq0[:, :n])
    assert torch.equal(dk[:, :n], dk0[:, :n]) and torch.equal(dv[:, :n], dv0[:, :n])
    # padding slots: the one-key closed form
    G = w.Hq // w.Hkv
    qp = q[0, n:].double().numpy()
    kp = k[0, n:].double().numpy()
    vp = v[0, n:].double().numpy()
    dop = do[0, n:].double().numpy()
    kq = np.repeat(kp, G, axis=1)
    want_lse = (qp * kq).sum(-1).T * w.D ** -0.5                       # [Hq, pads]
    got_lse = lse[0, :, n:].double().numpy()
    assert np.abs(got_lse - want_lse).max() <= 1e-5 * (1 + np.abs(want_lse).max())
    assert torch.equal(out[0, n:], torch.repeat_interleave(v[0, n:], G, dim=1))
    # exactly zero where the kernels see a whole block of isolated slots; in the block that mixes
    # padding with the last packed tokens, zero up to the rounding of dP - delta (fp32)
    dq_pad, dk_pad = dq[0, n:].abs().max().item(), dk[0, n:].abs().max().item()
    assert dq_pad <= 1e-3 and dk_pad <= 1e-3, (dq_pad, dk_pad)
    blk = (n + 255) // 256 * 256
    assert not dq[0, blk:].any() and not dk[0, blk:].any()
    want_dv = dop.reshape(R - n, w.Hkv, G, w.D).sum(axis=2)
    got_dv = dv[0, n:].double().numpy()
    assert np.all(np.abs(got_dv - want_dv) <= 2.0 ** -8 * np.abs(want_dv) + 1e-6)
    log(f"    {R - n} padding slots: out = v, lse err {np.abs(got_lse - want_lse).max():.2e}, "
        f"max |dq| {dq_pad:.1e}, max |dk| {dk_pad:.1e}, dv err {np.abs(got_dv - want_dv).max():.2e}")
