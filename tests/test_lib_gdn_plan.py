"""The GDN work plan on the CPU: chains, chunks and depth buckets against a direct derivation."""

import numpy as np
import pytest

import prefix_tree_packed_dfs_amd as lib
from oracle.layout import dfs_layout
from oracle.trie import build_trie
from synth import agentic_trie, grpo_group, sequence_packing_forest

from .test_lib_host import _random_forest


def _expected(parent_nodes, seq_last, n):
    """Parent slot, chains (start, length, parent chain, depth) in slot order, from the node tree."""
    lay = dfs_layout(parent_nodes, seq_last, n)
    node_slot = np.empty(n, np.int64)
    node_slot[lay.slot_node[:n]] = np.arange(n)
    pslot = np.array([-1 if parent_nodes[lay.slot_node[t]] < 0 else node_slot[parent_nodes[lay.slot_node[t]]]
                      for t in range(n)], dtype=np.int64)
    kids = np.bincount(pslot[pslot >= 0], minlength=n)
    chains, chain_of = [], np.empty(n, np.int64)
    for t in range(n):
        p = pslot[t]
        if p < 0 or p != t - 1 or kids[p] > 1:
            pc = -1 if p < 0 else chain_of[p]
            chains.append([t, 0, pc, 0 if pc < 0 else chains[pc][3] + 1])
        chain_of[t] = len(chains) - 1
        chains[-1][1] += 1
    return lay, pslot, chains


def _check_plan(parent_nodes, seq_last):
    n = len(parent_nodes)
    lay, pslot, chains = _expected(np.asarray(parent_nodes), np.asarray(seq_last), n)
    plan = lib.tree_gdn_plan(lay.subtree_end, n)
    assert np.array_equal(plan.parent_slot, pslot)
    # depth-major, slot order inside a depth
    order = sorted(range(len(chains)), key=lambda c: (chains[c][3], chains[c][0]))
    parents = {chains[c][2] for c in range(len(chains)) if chains[c][2] >= 0}
    slot = {}
    for c in order:
        if c in parents:
            slot[c] = len(slot)
    assert plan.n_segments == len(chains) and plan.n_states == len(slot)
    covered = np.zeros(n, np.int64)
    next_chunk = 0
    for r, c in enumerate(order):
        start, length, pc, depth = chains[c]
        first, count, par, own = plan.segments[r].tolist()
        assert (par, own) == ((-1 if pc < 0 else slot[pc]), slot.get(c, -1))
        assert first == next_chunk and count == (length + 63) // 64
        for j in range(count):
            s0, L = plan.chunks[first + j].tolist()
            assert s0 == start + 64 * j and L == min(64, length - 64 * j) and 1 <= L <= 64
            covered[s0:s0 + L] += 1
        next_chunk += count
    assert next_chunk == plan.n_chunks and np.all(covered == 1)
    depths = [chains[c][3] for c in order]
    assert plan.depth_offsets[0] == 0 and plan.depth_offsets[-1] == len(chains)
    for d in range(plan.n_depths):
        a, b = plan.depth_offsets[d], plan.depth_offsets[d + 1]
        assert b > a and all(x == d for x in depths[a:b])
    return plan


@pytest.mark.parametrize("seed", range(30))
def test_plan_on_random_forests(seed):
    rng = np.random.default_rng(700 + seed)
    n = int(rng.integers(1, 400))
    parent = _random_forest(rng, n)
    # a few long chains so that chains span several chunks
    if seed % 3 == 0:
        parent = np.concatenate([parent, np.arange(n - 1, n + 149, dtype=np.int32)])
    _check_plan(parent, np.zeros(0, np.int32))


@pytest.mark.parametrize("seed", range(10))
def test_plan_on_tries(seed):
    rng = np.random.default_rng(800 + seed)
    seqs = [np.repeat(rng.integers(0, 2, size=int(rng.integers(1, 30))), int(rng.integers(1, 40))).astype(np.int32)
            for _ in range(int(rng.integers(1, 9)))]
    for ms in (1, 64):
        t = build_trie(seqs, min_shared=ms)
        _check_plan(t.parent, t.seq_last)


def test_plan_of_workloads_and_of_sequence_packing():
    for w in (grpo_group(), agentic_trie()):
        t = build_trie(w.sequences)
        plan = _check_plan(t.parent, t.seq_last)
        assert plan.n_depths >= 2
        p, s = sequence_packing_forest(w.sequences)
        plan = _check_plan(p, s)
        assert plan.n_depths == 1 and plan.n_segments == len(w.sequences)
    w = grpo_group()
    plan = lib.tree_gdn_plan(lib.tree_pack_layout(*lib.tree_build_trie(w.sequences), 18447).subtree_end, 18447)
    # the 2,047-token prompt chain (its last token is copied into every branch), then 16 x 1,025
    assert plan.segments[0, 1] == 32 and plan.chunks[31, 1] == 2047 - 31 * 64
    assert list(plan.segments[1:, 1]) == [17] * 16 and plan.n_chunks == 32 + 16 * 17


def test_plan_errors_and_size_query():
    import ctypes as C
    with pytest.raises(lib.TreeAttnError) as e:
        lib.tree_gdn_plan(np.array([2, 3, 2, 3], np.int32), 4)          # crossing intervals
    assert e.value.status == 2
    se = np.array([2, 1, 2], np.int32)
    i32 = C.POINTER(C.c_int32)
    ns, nc, nd, nst = C.c_int64(0), C.c_int64(0), C.c_int64(0), C.c_int64(0)
    L = lib.lib
    assert L.tree_gdn_plan(3, se.ctypes.data_as(i32), None, None, 0, C.byref(ns), None, 0, C.byref(nc), None, 0,
                           C.byref(nd), C.byref(nst)) == 0
    assert (ns.value, nc.value, nd.value, nst.value) == (3, 3, 2, 1)    # root, then two single-token children
    par = np.zeros(3, np.int32)
    seg = np.zeros((1, 4), np.int32)
    ch = np.zeros((3, 2), np.int32)
    off = np.zeros(3, np.int32)
    st = L.tree_gdn_plan(3, se.ctypes.data_as(i32), par.ctypes.data_as(i32), seg.ctypes.data_as(i32), 1, C.byref(ns),
                         ch.ctypes.data_as(i32), 3, C.byref(nc), off.ctypes.data_as(i32), 2, C.byref(nd),
                         C.byref(nst))
    assert st == 3 and ns.value == 3
    plan = lib.tree_gdn_plan(np.zeros(0, np.int32), 0)
    assert plan.n_segments == 0 and plan.n_depths == 0


def test_fwd_rejects_bad_arguments_before_any_launch():
    L = lib.lib
    args = lambda dt, W, n, Hk, Hv, dk: (dt, None, None, W, None, None, None, None, 1, None, 1, None, 1, 0, n,  # noqa
                                         Hk, Hv, dk, 128, None, None, 0, None)
    assert L.tree_gdn_fwd(*args(0, 4, 8, 1, 2, 128)) == 4        # fp32 unsupported
    assert L.tree_gdn_fwd(*args(1, 4, 8, 1, 2, 64)) == 4         # head dim
    assert L.tree_gdn_fwd(*args(1, 4, 8, 2, 3, 128)) == 1        # Hv not a multiple of Hk
    assert L.tree_gdn_fwd(*args(1, 5, 8, 1, 2, 128)) == 4        # conv width
    assert L.tree_gdn_fwd(*args(1, 4, 8, 1, 2, 128)) == 1        # null pointers
    assert L.tree_gdn_fwd(1, None, None, 4, None, None, None, None, 0, None, 0, None, 0, 0, 0, 1, 2, 128, 128,
                          None, None, 0, None) == 0              # empty row: no-op
    assert L.tree_gdn_workspace_bytes(8, 2, 3, 1, 2, 128, 128) > 0
    assert L.tree_gdn_workspace_bytes(8, 2, 3, 1, 2, 64, 128) == 0
