"""Host-side logic of bench.py (no GPU): the algorithmic byte count, the tile classes it reports, the
row counts, the source-hash guard on counter-based traffic and the one-GPU refusal.

The tile classes are checked against a brute force over every (query, key) pair of the interval mask
[ART "Token-mixing layers"]: query i sees key j iff j <= i <= subtree_end[j]."""
import os
import subprocess
import sys
from types import SimpleNamespace

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import prefix_tree_packed_dfs_amd as lib  # noqa: E402
from synth import standard  # noqa: E402


def _layout(w):
    parent, seq_last = lib.tree_build_trie(w.sequences, min_shared=64)
    n = len(parent)
    R = w.row_length(n)
    return lib.tree_pack_layout(parent, seq_last, R), n, R


def test_algorithmic_bytes_match_the_stated_grpo_group_figures():
    # The measurement plan states 228 MB (forward) and 457 MB (backward) for the 32K-row GRPO group:
    # q, k, v in and out written (+ lse) forward; q, k, v, out, dout, lse in, delta out and back,
    # dq, dk, dv written backward.
    w = standard(2)
    _, n, _ = _layout(w)
    fwd, bwd = bench.algorithmic_bytes(w, n)
    assert n == 18447
    assert round(fwd / 1e6) == 228
    assert round(bwd / 1e6) == 457


def test_algorithmic_bytes_scale_with_element_size_and_heads():
    # fp32 doubles every tensor term and leaves the fp32 lse / delta terms alone
    w = SimpleNamespace(Hq=4, Hkv=2, D=64, dtype="bf16")
    f2, b2 = bench.algorithmic_bytes(w, 10)
    w.dtype = "f32"
    f4, b4 = bench.algorithmic_bytes(w, 10)
    assert f4 - 4 * 10 * w.Hq == 2 * (f2 - 4 * 10 * w.Hq)
    assert b4 - 12 * 10 * w.Hq == 2 * (b2 - 12 * 10 * w.Hq)


def _brute_classes(se, R, BM, KT):
    """Per query block (skipping blocks of isolated slots only) and key tile up to the block's last
    one: skipped = no visible pair, full = every pair visible, partial = the rest."""
    T = (R + KT - 1) // KT
    idx = np.arange(R)
    # a tile is isolated when each of its slots sees and is seen by itself only
    iso = []
    for t in range(T):
        j = idx[t * KT:(t + 1) * KT]
        reach_before = se[:t * KT].max() if t else -1
        iso.append(bool(np.all(se[j] == j)) and reach_before < t * KT)
    full = partial = skipped = blocks = 0
    for qb in range((R + BM - 1) // BM):
        i0, i1 = qb * BM, min(qb * BM + BM, R) - 1
        if all(iso[i0 // KT:i1 // KT + 1]):
            continue
        blocks += 1
        qi = np.arange(i0, i1 + 1)[None, :]
        for t in range(i1 // KT + 1):
            kj = idx[t * KT:min(t * KT + KT, R)][:, None]
            vis = (kj <= qi) & (qi <= se[kj])
            if not vis.any():
                skipped += 1
            elif vis.all():
                full += 1
            else:
                partial += 1
    return blocks, full, partial, skipped


@pytest.mark.parametrize("seed", range(6))
def test_tile_classes_equal_a_brute_force_over_the_mask(seed):
    rng = np.random.default_rng(seed)
    # small-alphabet sequences fork at many depths; the row is padded past the packed slots
    seqs = [rng.integers(0, 3, size=int(rng.integers(20, 300)), dtype=np.int32) for _ in range(12)]
    parent, seq_last = lib.tree_build_trie(seqs, min_shared=8)
    n = len(parent)
    R = ((n + 200) + 63) // 64 * 64
    lay = lib.tree_pack_layout(parent, seq_last, R)
    se = lay.subtree_end.astype(np.int64)
    w = SimpleNamespace(Hq=16, Hkv=8)  # two query heads per KV head: 128-position blocks
    got = bench.tile_classes(w, se, R)
    blocks, full, partial, skipped = _brute_classes(se, R, got["block_rows"], got["key_tile"])
    assert got["block_rows"] == 128 and got["key_tile"] == 64
    assert (got["query_blocks"], got["full"], got["partial"], got["skipped"]) == (blocks, full, partial, skipped)


def test_tile_classes_where_subtrees_end_on_a_block_start():
    # Independent chains whose last slots fall exactly on the first query of a 128-position block
    # (slots 128, 384 and 640): the tiles holding those chains are visible to that block through
    # its first query alone.
    lengths = [129, 127, 128, 1, 200, 56, 191]
    parent, seq_last, start = [], [], 0
    for L in lengths:
        parent += [-1] + list(range(start, start + L - 1))
        seq_last.append(start + L - 1)
        start += L
    R = (start + 63) // 64 * 64
    lay = lib.tree_pack_layout(np.array(parent, np.int32), np.array(seq_last, np.int32), R)
    se = lay.subtree_end.astype(np.int64)
    assert {128, 384, 640} <= set(se.tolist())
    w = SimpleNamespace(Hq=16, Hkv=8)
    got = bench.tile_classes(w, se, R)
    assert (got["query_blocks"], got["full"], got["partial"], got["skipped"]) == _brute_classes(se, R, 128, 64)


def test_tile_classes_of_independent_sequences():
    # 64 sequences of 512 tokens, 128-position blocks: the block at offset 128 m of its sequence sees
    # the 2 m 64-key tiles of its sequence before it in full and its own two tiles in part (the
    # causal diagonal); every other tile of the row up to the block is skipped.
    w = standard(4)
    lay, n, R = _layout(w)
    got = bench.tile_classes(w, lay.subtree_end.astype(np.int64), R)
    assert got["query_blocks"] == 256
    assert got["full"] == 64 * sum(2 * m for m in range(4))
    assert got["partial"] == 64 * 4 * 2
    total = sum((qb * 128 + 127) // 64 + 1 for qb in range(256))
    assert got["full"] + got["partial"] + got["skipped"] == total


def test_row_counts_follow_the_workload_recipes():
    w = standard(2)  # 16 completions under one 2,048-token prompt
    lay, n, R = _layout(w)
    c = bench.row_counts(w, lay, n, R)
    assert c["fork_frac"] == 1.0
    assert c["row_fill"] == round(18447 / 32768, 4)
    assert c["packing_ratio"] == round(49152 / 18447, 4)
    w = standard(4)  # 64 independent sequences fill the row, nothing shared
    lay, n, R = _layout(w)
    c = bench.row_counts(w, lay, n, R)
    assert (c["fork_frac"], c["row_fill"], c["packing_ratio"]) == (0.0, 1.0, 1.0)


def test_counter_traffic_is_reported_only_for_the_sources_it_was_taken_on(tmp_path, monkeypatch):
    (tmp_path / "profiles").mkdir()
    (tmp_path / "profiles" / "grpo_group_traffic.md").write_text(
        "# HBM traffic\n\n- source_hash: `abc123`\n- bwd_traffic_bytes_per_call: `1500000000`\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "source_hash", lambda: "abc123")
    assert bench.measured_traffic("grpo_group") == 1.5e9
    monkeypatch.setattr(bench, "source_hash", lambda: "other")
    assert bench.measured_traffic("grpo_group") is None
    assert bench.measured_traffic("agentic_trie") is None  # no file


def test_source_hash_covers_the_attention_kernel_sources():
    h = bench.source_hash()
    assert len(h) == 16 and int(h, 16) >= 0
    assert h == bench.source_hash()  # deterministic


def test_more_than_one_gpu_is_refused_before_any_device_work():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
