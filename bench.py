#!/usr/bin/env python3
"""Benchmark one step of the prefix-tree-packed attention hot path on one MI355X.

A step is one pass of the whole path over one packed row:
  tree_pack_layout (host, into pinned buffers) -> async copy of pos_ids and
  subtree_end -> tree_rope_qk(q, k) -> tree_attn_fwd -> tree_attn_bwd.
Inputs (q, k, v, dout) are resident in HBM before timing starts.

Throughput is algorithmic: ancestor pairs per head = sum over real slots of
(depth + 1); forward FLOPs = 4 * D * Hq * pairs, backward = 2.5 x forward.
Prints one JSON line.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload grpo_group]
"""

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

WORKLOADS = {
    "tiny_tree": 1,
    "grpo_group": 2,
    "agentic_trie": 3,
    "independent": 4,
    "long_history": 5,
}
PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0      # MI355X HBM3E
COPY_BYTES = 1 << 30         # size of the plain copy used to calibrate the HBM byte counters


def source_hash() -> str:
    """Hash of the attention kernel sources: counter-based traffic is only reported for the kernels it
    was taken on."""
    import hashlib
    d = os.path.join(ROOT, "prefix_tree_packed_dfs_amd", "csrc")
    h = hashlib.sha256()
    for f in sorted(os.listdir(d)):
        if f.startswith("attn_") or f == "mfma_common.h":
            h.update(f.encode())
            h.update(open(os.path.join(d, f), "rb").read())
    return h.hexdigest()[:16]


def measured_traffic(workload: str):
    """HBM bytes per backward call from profiles/<workload>_traffic.md, if taken on these sources."""
    path = os.path.join(ROOT, "profiles", f"{workload}_traffic.md")
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        if line.startswith("- ") and ":" in line:
            k, v = line[2:].split(":", 1)
            vals[k.strip()] = v.strip().strip("`")
    if vals.get("source_hash") != source_hash():
        return None
    try:
        return float(vals["bwd_traffic_bytes_per_call"])
    except (KeyError, ValueError):
        return None


def describe(w, n, R, pairs):
    return {
        "workload": w.name,
        "sequences": len(w.sequences),
        "row_len": R,
        "forwarded_tokens": n,
        "raw_tokens": w.raw_tokens,
        "packing_ratio": round(w.raw_tokens / n, 4),
        "ancestor_pairs_per_head": int(pairs),
        "Hq": w.Hq,
        "Hkv": w.Hkv,
        "head_dim": w.D,
        "batch_rows": 1,
    }


def row_counts(w, lay, n, R):
    """[TRL "How to evaluate it on your own workload"]: packing ratio, fork fraction (share of sequences
    whose path shares a slot with another sequence) and row fill (forwarded / row slots), from the
    library's layout."""
    import numpy as np
    users = np.zeros(R, np.int64)
    paths = [lay.sequence_slots(s) for s in range(len(w.sequences))]
    for p in paths:
        users[np.unique(p)] += 1
    forked = sum(1 for p in paths if len(p) and bool((users[p] > 1).any()))
    return {"packing_ratio": round(w.raw_tokens / n, 4), "fork_frac": round(forked / max(len(paths), 1), 4),
            "row_fill": round(n / R, 4)}


def tile_classes(w, se, R):
    """The forward's tile classes per KV head: every (query block, 64-key tile) pair of a block's visible
    range, as the kernels classify them from per-tile min / max subtree_end (skipped: no key of the tile
    sees the block; full: every key sees every query; partial: the interval test runs per element).
    Query blocks are the kernels' items (256 rows = BM positions x HB query heads sharing a KV head);
    blocks of isolated slots only (padding) are left to the isolated-slot units and not counted."""
    import numpy as np
    G = w.Hq // w.Hkv
    HB = 8 if G >= 8 else G
    BM, KT = 256 // HB, 64
    T = (R + KT - 1) // KT
    pad = np.concatenate([se, np.full(T * KT - R, -1, np.int64)])
    idx = np.arange(T * KT)
    tmax = pad.reshape(T, KT).max(axis=1)
    tmin = np.where(idx < R, pad, np.iinfo(np.int64).max).reshape(T, KT).min(axis=1)
    self_only = np.all(((pad == idx) | (idx >= R)).reshape(T, KT), axis=1)
    before = np.concatenate([[-1], np.maximum.accumulate(tmax)[:-1]])
    iso = self_only & (before < np.arange(T) * KT)
    full = partial = skipped = blocks = 0
    for qb in range((R + BM - 1) // BM):
        i0, i1 = qb * BM, min(qb * BM + BM, R) - 1
        t_last = i1 // KT
        if iso[i0 // KT:t_last + 1].all():
            continue
        blocks += 1
        t = np.arange(t_last + 1)
        vis = tmax[:t_last + 1] >= i0
        f = vis & (t * KT + KT - 1 <= i0) & (tmin[:t_last + 1] >= i1)
        full += int(f.sum())
        partial += int((vis & ~f).sum())
        skipped += int((~vis).sum())
    chunks = G // HB
    return {"query_blocks": blocks * chunks, "full": full * chunks, "partial": partial * chunks,
            "skipped": skipped * chunks, "block_rows": BM, "key_tile": KT}


def algorithmic_bytes(w, n):
    """What the path must move per call (bf16 / fp32 elements, fp32 lse and delta): forward reads q, k, v
    and writes out, lse; backward reads q, k, v, out, dout and lse (4 bytes a row), writes and reads delta
    (8), and writes dq, dk, dv."""
    e = 2 if w.dtype == "bf16" else 4
    fwd = n * ((w.Hq + 2 * w.Hkv) * w.D * e + w.Hq * w.D * e + 4 * w.Hq)
    bwd = n * (2 * (w.Hq + 2 * w.Hkv) * w.D * e + 2 * w.Hq * w.D * e + 12 * w.Hq)
    return fwd, bwd


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w, total_flops, target_s):
    """Time the oracle (fwd + bwd, fp64, CPU) on the first sequences of the workload."""
    import numpy as np
    from threadpoolctl import threadpool_info

    from oracle.attention import tree_attention
    from synth import feature_tables

    tables = feature_tables(w)
    # grow the sample until one fwd + bwd run takes at least target_s / 2 (10 s by default; the
    # growth runs and the forward-only run bring the leg to about 1.5 x target_s)
    k = 1
    raw_all = w.raw_tokens
    while True:
        seqs = w.sequences[:k]
        t0 = time.perf_counter()
        tree_attention(seqs, w.fid[:k], w.dkey[:k], tables, theta=w.theta, backward=True, storage=w.dtype)
        dt = time.perf_counter() - t0
        if dt >= target_s / 2 or k == len(w.sequences):
            break
        k = min(len(w.sequences), max(k + 1, int(k * (target_s / 2) / max(dt, 1e-3)) + 1))
    raw_k = sum(len(s) for s in seqs)
    t0 = time.perf_counter()
    tree_attention(seqs, w.fid[:k], w.dkey[:k], tables, theta=w.theta, backward=False, storage=w.dtype)
    dt_fwd = time.perf_counter() - t0
    # the oracle's cost is per unpacked sequence: extrapolate by raw-token work share
    work = lambda ss: sum(len(s) * (len(s) + 1) / 2 for s in ss)  # noqa: E731
    frac = work(seqs) / work(w.sequences)
    full_s = dt / frac
    threads = sum(i.get("num_threads", 0) for i in threadpool_info() if i.get("user_api") == "blas") or 1
    _ = np
    return {
        "value": round(total_flops / full_s / 1e12, 6),
        "unit": "TFLOP/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": f"oracle fwd+bwd on the first {k} of {len(w.sequences)} sequences ({raw_k} of {raw_all} raw "
                  f"tokens, {frac:.3f} of the oracle's per-sequence work) took {dt:.2f} s (forward alone "
                  f"{dt_fwd:.2f} s); whole-row time extrapolated to {full_s:.1f} s",
        "seconds_sample": round(dt, 3),
        "seconds_sample_fwd": round(dt_fwd, 3),
        "raw_tok_s_sample": round(raw_k / dt, 1),
        "raw_tok_s_sample_fwd": round(raw_k / dt_fwd, 1),
        "cpu_model": cpu_model(),
        "host_cpus": os.cpu_count(),
    }


def bench_planner(args):
    """Host row planner on multi-task batches of 12 .. 768 groups, rows of 131,072 tokens.

    Times tree_build_trie (trainable mode) and tree_place_leaves (global best-fit decreasing, and
    in order), as [ART "Does it actually help?"] tables the tree walk against the bin-packing pass,
    and tree_plan_rows (rows grown in order under a 131,072-token budget, fork threshold 1024,
    [TRL "How tree packing works"]) with its row fill and fork fraction; the oracle runs beside
    it on the smallest batch.  Prints one JSON line."""
    import numpy as np

    import prefix_tree_packed_dfs_amd as lib
    from synth import curriculum_batch

    import ctypes as C

    row = 131072
    out = []
    i32, i64, u8 = C.POINTER(C.c_int32), C.POINTER(C.c_int64), C.POINTER(C.c_uint8)
    for n_groups in (12, 48, 192, 768):
        seqs, train, grp = curriculum_batch(n_groups)
        # flattened CSR inputs, built outside the timed region (argument marshalling only)
        offsets = np.zeros(len(seqs) + 1, dtype=np.int64)
        np.cumsum([len(x) for x in seqs], out=offsets[1:])
        tokens = np.concatenate(seqs)
        flags = np.concatenate(train).view(np.uint8)
        total = int(offsets[-1])
        parent = np.empty(total, dtype=np.int32)
        seq_last = np.empty(len(seqs), dtype=np.int32)
        n_nodes = C.c_int64(0)
        t0 = time.perf_counter()
        st = lib.lib.tree_build_trie(len(seqs), offsets.ctypes.data_as(i64), tokens.ctypes.data_as(i32),
                                     flags.ctypes.data_as(u8), 64, parent.ctypes.data_as(i32), total,
                                     C.byref(n_nodes), seq_last.ctypes.data_as(i32))
        t1 = time.perf_counter()
        assert st == 0
        parent = parent[:n_nodes.value]
        _, tok_g = lib.tree_place_leaves(parent, seq_last, grp, row, "global")
        t2 = time.perf_counter()
        _, tok_i = lib.tree_place_leaves(parent, seq_last, grp, row, "in_order")
        t3 = time.perf_counter()
        # TRL's planner on the same samples: rows grown in order under a forwarded-token budget
        t4 = time.perf_counter()
        row_of, row_tok, forked = lib.tree_plan_rows(seqs, row, 1024)
        t5 = time.perf_counter()
        out.append({"groups": n_groups, "completions": len(seqs), "raw_tokens": int(sum(len(x) for x in seqs)),
                    "trie_nodes": int(len(parent)), "trie_ms": round((t1 - t0) * 1e3, 2),
                    "place_global_ms": round((t2 - t1) * 1e3, 2), "rows_global": int(len(tok_g)),
                    "place_in_order_ms": round((t3 - t2) * 1e3, 2), "rows_in_order": int(len(tok_i)),
                    "plan_rows_ms": round((t5 - t4) * 1e3, 2), "rows_plan": int(len(row_tok)),
                    "plan_row_fill": round(float(row_tok.sum()) / (len(row_tok) * row), 4),
                    "plan_fork_frac": round(float(forked.mean()), 4)})
    oracle = None
    if not args.no_cpu_baseline:
        from oracle.pack import place_leaves, segments
        from oracle.trie import build_trie
        seqs, train, grp = curriculum_batch(12)
        t0 = time.perf_counter()
        tr = build_trie(seqs, trainable=train)
        t1 = time.perf_counter()
        pl = place_leaves(segments(tr.parent, tr.seq_last), grp, row, "global")
        t2 = time.perf_counter()
        oracle = {"groups": 12, "trie_s": round(t1 - t0, 3), "place_global_s": round(t2 - t1, 3),
                  "rows_global": int(len(pl.bin_tokens)), "kind": "oracle", "threads": 1}
    print(json.dumps({"metric": "row planner: trie walk + best-fit-decreasing placement", "unit": "ms",
                      "row_len": row, "data": "synthetic (synth.curriculum_batch)", "sizes": out,
                      "cpu_baseline": oracle}), flush=True)


def bench_sweep(args):
    """Tree packing against sequence packing over packing ratios 1.0 .. 4.9, same kernels.

    Sequence packing lays each sequence out as its own chain (a forest of chains: plain
    varlen causal attention); tree packing lays out the trie.  Each layout gets the same
    per-token q/k/v/dout (gathered from one set of tree-slot tensors) and runs rope(q),
    rope(k), tree_attn_fwd, tree_attn_bwd on device; layouts are on the host beforehand.
    Each layout is timed twice, alternating with the other, and reports its faster run.
    Peak memory is the device memory the layout's step allocates: its q/k/v/dout,
    out/lse, dq/dk/dv and workspaces (the backward's sized to the layout's dK/dV plan).  [TRL tree packing, "Claimed vs. verified"] reports
    the same comparison (speedup and peak memory against packing ratio) for FlashAttention 3
    on another GPU.  Prints one JSON line."""
    import numpy as np
    import torch

    import prefix_tree_packed_dfs_amd as lib
    from synth import grpo_group, agentic_trie, independent, long_history, sequence_packing_forest, shared_history

    torch.cuda.set_device(0)
    dev = torch.device("cuda", 0)
    points = [shared_history(p) for p in (0, 1000, 2000, 4000, 8000, 20000)]
    points += [independent(), grpo_group(), agentic_trie(), long_history()]
    steps, warmup = args.steps, args.warmup

    def pad64(n):
        return max(64, (n + 63) // 64 * 64)

    def layout(w, parent, seq_last):
        R = pad64(len(parent))
        lay = lib.tree_pack_layout(parent, seq_last, R)
        ti = np.concatenate([lay.sequence_slots(s) for s in range(len(w.sequences))]).astype(np.int64)
        pairs = int((lay.pos_ids[:len(parent)].astype(np.int64) + 1).sum())
        return lay, R, ti, pairs, len(parent)

    def run(w, lay, R, src, gather, pairs):
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        base = torch.cuda.memory_allocated()
        torch.cuda.reset_peak_memory_stats()
        q, k, v, do = (t[:, gather].contiguous() for t in src)
        pos = torch.from_numpy(lay.pos_ids.astype(np.int32)).view(1, R).to(dev)
        se = torch.from_numpy(lay.subtree_end.astype(np.int32)).view(1, R).to(dev)
        dt = lib.TREE_BF16
        out = torch.empty_like(q)
        lse = torch.empty((1, w.Hq, R), device=dev, dtype=torch.float32)
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        wsf = torch.empty(max(lib.tree_attn_workspace_bytes(dt, 1, R, w.Hq, w.Hkv, w.D, False), 1), device=dev,
                          dtype=torch.uint8)
        # the backward workspace this layout's dK/dV plan uses (fixed part + its partial-sum slots)
        wsb = torch.empty(max(lib.tree_attn_bwd_workspace_bytes_for(dt, lay.subtree_end, w.Hq, w.Hkv, w.D), 1),
                          device=dev, dtype=torch.uint8)
        scale = w.D ** -0.5

        def step(ev=None):
            if ev:
                ev[0].record()
            lib.tree_rope_qk(q, k, pos, w.theta)
            lib.tree_attn_fwd(q, k, v, se, scale, out=out, lse=lse, ws=wsf)
            if ev:
                ev[1].record()
            lib.tree_attn_bwd(q, k, v, se, out, lse, do, scale, dq=dq, dk=dk, dv=dv, ws=wsb)
            if ev:
                ev[2].record()

        for _ in range(warmup):
            step()
        torch.cuda.synchronize()
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
        for i in range(steps):
            step(evs[i])
        torch.cuda.synchronize()
        peak = torch.cuda.max_memory_allocated() - base
        ms = float(np.mean([e[0].elapsed_time(e[2]) for e in evs]))
        fwd = float(np.mean([e[0].elapsed_time(e[1]) for e in evs]))
        bwd = float(np.mean([e[1].elapsed_time(e[2]) for e in evs]))
        ws_bytes = int(wsf.numel() + wsb.numel())
        del q, k, v, do, out, lse, dq, dk, dv, wsf, wsb, pos, se
        flops = 3.5 * 4.0 * w.D * w.Hq * pairs
        return {"row_len": R, "ancestor_pairs_per_head": pairs, "ms_per_step": round(ms, 4),
                "rope_fwd_ms": round(fwd, 4), "bwd_ms": round(bwd, 4), "peak_bytes": int(peak),
                "workspace_bytes": ws_bytes,
                "tflops": round(flops / (ms * 1e-3) / 1e12, 2),
                "raw_tok_s": round(w.raw_tokens / (ms * 1e-3), 1)}

    rows = []
    for w in points:
        print(f"# {w.name}: {len(w.sequences)} sequences, {w.raw_tokens} raw tokens", file=sys.stderr, flush=True)
        tlay, tR, tti, tpairs, n = layout(w, *lib.tree_build_trie(w.sequences, min_shared=64))
        clay, cR, cti, cpairs, _ = layout(w, *sequence_packing_forest(w.sequences))
        g = torch.Generator(device=dev).manual_seed(7)
        src = [torch.randn((1, tR, h, w.D), generator=g, device=dev).to(torch.bfloat16)
               for h in (w.Hq, w.Hkv, w.Hkv, w.Hq)]
        # chain slot c holds the token whose tree slot is gather[c]; padding slots read tree slot 0
        gather = np.zeros(cR, np.int64)
        gather[cti] = tti
        tidx, cidx = torch.arange(tR, device=dev), torch.from_numpy(gather).to(dev)
        if not rows:  # bring the clocks up before the first timed run
            run(w, tlay, tR, src, tidx, tpairs)
        # two alternating runs per layout; each layout reports its faster run
        t_runs, c_runs = [], []
        for _ in range(2):
            t_runs.append(run(w, tlay, tR, src, tidx, tpairs))
            c_runs.append(run(w, clay, cR, src, cidx, cpairs))
        tree = min(t_runs, key=lambda r: r["ms_per_step"])
        seqp = min(c_runs, key=lambda r: r["ms_per_step"])
        del src
        rows.append({
            "workload": w.name, "sequences": len(w.sequences), "raw_tokens": w.raw_tokens,
            "forwarded_tokens": n, "packing_ratio": round(w.raw_tokens / n, 4),
            "Hq": w.Hq, "Hkv": w.Hkv, "head_dim": w.D,
            "tree": tree, "sequence_packing": seqp,
            "speedup": round(seqp["ms_per_step"] / tree["ms_per_step"], 3),
            "memory_ratio": round(seqp["peak_bytes"] / tree["peak_bytes"], 3),
            "pair_ratio": round(cpairs / tpairs, 3),
        })
        print(f"#   ratio {rows[-1]['packing_ratio']}: tree {tree['ms_per_step']} ms, sequence packing "
              f"{seqp['ms_per_step']} ms, speedup {rows[-1]['speedup']}, memory "
              f"{seqp['peak_bytes'] / 2**30:.2f} -> {tree['peak_bytes'] / 2**30:.2f} GiB", file=sys.stderr, flush=True)
    print(json.dumps({"metric": "tree packing vs sequence packing: fwd+bwd attention step time and peak memory",
                      "unit": "x (sequence-packing time / tree time)", "steps": steps, "warmup": warmup,
                      "dtype": "bf16", "data": "synthetic", "points": rows}), flush=True)


def bench_gdn(args):
    """Gated-delta-rule mixing (tree_gdn_fwd) on the packed row and on sequence packing.

    Layer shape: 16 key heads, 32 value heads, head dims 128, convolution width 4.  Inputs
    (x, g, beta) are resident in HBM and the plan's device tables are uploaded before timing;
    a step is one tree_gdn_fwd call.  The oracle (fp64, per sequence) is timed on the first
    sequence for two value heads and scaled to the row by raw tokens and heads.  Prints one
    JSON line."""
    import numpy as np
    import torch

    import prefix_tree_packed_dfs_amd as lib
    from synth import agentic_trie, grpo_group, long_history, sequence_packing_forest

    torch.cuda.set_device(0)
    dev = torch.device("cuda", 0)
    Hk, Hv, W = 16, 32, 4
    C = (2 * Hk + Hv) * 128
    names = args.gdn_workloads.split(",")
    makers = {"grpo_group": grpo_group, "agentic_trie": agentic_trie, "long_history": long_history}
    g0 = torch.Generator(device=dev).manual_seed(11)
    conv_w = (torch.randn((C, W), generator=g0, device=dev) / 2.0).contiguous()
    rows = []
    for name in names:
        w = makers[name]()
        res = {"workload": name, "sequences": len(w.sequences), "raw_tokens": w.raw_tokens}
        for layout in ("tree", "sequence_packing"):
            if layout == "tree":
                parent, seq_last = lib.tree_build_trie(w.sequences, min_shared=64)
            else:
                parent, seq_last = sequence_packing_forest(w.sequences)
            n = len(parent)
            lay = lib.tree_pack_layout(parent, seq_last, n)
            plan = lib.tree_gdn_plan(lay.subtree_end, n)
            tables = plan.device_tables(dev)
            x = torch.randn((n, C), generator=g0, device=dev).to(torch.bfloat16)
            g = -0.1 * torch.rand((n, Hv), generator=g0, device=dev)
            beta = torch.rand((n, Hv), generator=g0, device=dev)
            out = torch.empty((n, Hv, 128), dtype=torch.bfloat16, device=dev)
            ws = torch.empty(lib.tree_gdn_workspace_bytes(n, plan.n_states, plan.n_chunks, Hk, Hv), dtype=torch.uint8,
                             device=dev)
            for _ in range(args.warmup):
                lib.tree_gdn_fwd(x, conv_w, g, beta, plan, Hk, Hv, out=out, ws=ws, tables=tables)
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(args.steps):
                lib.tree_gdn_fwd(x, conv_w, g, beta, plan, Hk, Hv, out=out, ws=ws, tables=tables)
            e1.record()
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1) / args.steps
            res[layout] = {"slots": n, "chains": plan.n_segments, "chunks": plan.n_chunks, "depths": plan.n_depths,
                           "ms_per_call": round(ms, 4), "slots_per_s": round(n / (ms * 1e-3), 1),
                           "raw_tok_s": round(w.raw_tokens / (ms * 1e-3), 1),
                           "workspace_bytes": int(ws.numel())}
            print(f"# gdn {name} {layout}: {n} slots, {plan.n_segments} chains, {plan.n_depths} depths, "
                  f"{ms:.3f} ms", file=sys.stderr, flush=True)
            del x, g, beta, out, ws, tables
        res["packing_ratio"] = round(w.raw_tokens / res["tree"]["slots"], 4)
        res["speedup"] = round(res["sequence_packing"]["ms_per_call"] / res["tree"]["ms_per_call"], 3)
        rows.append(res)
    rec = {"metric": "gated-delta-rule mixing over packed rows: raw tokens/s, tree vs sequence packing",
           "unit": "tokens/s", "value": rows[0]["tree"]["raw_tok_s"], "steps": args.steps, "warmup": args.warmup,
           "dtype": "bf16", "data": "synthetic",
           "config": {"workload": rows[0]["workload"], "Hk": Hk, "Hv": Hv, "dk": 128, "dv": 128, "conv_width": W},
           "points": rows}
    if not args.no_cpu_baseline:
        from oracle.gdn import GdnShape, tree_gdn
        from synth import gdn_tables
        w = makers[names[0]]()
        t = gdn_tables(w, Hk=Hk, Hv=Hv, conv_width=W)
        heads = [0, Hv - 1]
        t0 = time.perf_counter()
        tree_gdn(w.sequences, w.fid, t, t["conv_w"], GdnShape(Hk, Hv, 128, 128), storage="bf16", heads=heads, seqs=[0])
        dt = time.perf_counter() - t0
        frac = len(w.sequences[0]) / w.raw_tokens * len(heads) / Hv
        rec["cpu_baseline"] = {"value": round(w.raw_tokens / (dt / frac), 1), "unit": "tokens/s", "cores": 1,
                               "kind": "oracle",
                               "sample": f"oracle GDN on sequence 0 ({len(w.sequences[0])} of {w.raw_tokens} raw "
                                         f"tokens), value heads {heads} of {Hv}: {dt:.2f} s, scaled by "
                                         f"{1 / frac:.0f}x"}
    print(json.dumps(rec), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="grpo_group", choices=list(WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=20.0)
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain device copy of 1 GiB (for calibrating HBM byte counters)")
    ap.add_argument("--planner", action="store_true",
                    help="only time the host row planner (trie walk + leaf placement) on curriculum batches")
    ap.add_argument("--sweep", action="store_true",
                    help="only run the tree-vs-sequence-packing sweep over packing ratios 1.0 .. 4.9")
    ap.add_argument("--gdn", action="store_true",
                    help="only time gated-delta-rule mixing (tree and sequence packing) on the bf16 workloads")
    ap.add_argument("--gdn-workloads", default="grpo_group,agentic_trie,long_history")
    args = ap.parse_args()
    if args.gdn:
        if args.gpus != 1:
            print("bench.py runs on one GPU only", file=sys.stderr)
            sys.exit(2)
        bench_gdn(args)
        return
    if args.sweep:
        if args.gpus != 1:
            print("bench.py runs on one GPU only", file=sys.stderr)
            sys.exit(2)
        bench_sweep(args)
        return
    if args.planner:
        bench_planner(args)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: this build has no multi-GPU path (asked for --gpus {args.gpus})",
              file=sys.stderr)
        sys.exit(2)

    import ctypes as C

    import numpy as np
    import torch

    import prefix_tree_packed_dfs_amd as lib
    from synth import standard

    torch.cuda.set_device(0)
    dev = torch.device("cuda", 0)
    if args.calibrate_copy:
        src = torch.ones(COPY_BYTES // 2, dtype=torch.bfloat16, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": COPY_BYTES, "copies": 3}), flush=True)
        return
    w = standard(WORKLOADS[args.workload])
    if not w.backward:
        w.backward = True  # time the full path on every workload
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    dt_code = lib.TREE_BF16 if w.dtype == "bf16" else lib.TREE_F32

    # planner output (the trie) is the input of the path
    parent, seq_last = lib.tree_build_trie(w.sequences, min_shared=64)
    n = len(parent)
    R = w.row_length(n)
    lay = lib.tree_pack_layout(parent, seq_last, R)
    pairs = int((lay.pos_ids[:n].astype(np.int64) + 1).sum())
    fwd_flops = 4.0 * w.D * w.Hq * pairs
    bwd_flops = 2.5 * fwd_flops
    total_flops = fwd_flops + bwd_flops

    g = torch.Generator(device=dev).manual_seed(2024)
    q = torch.randn((1, R, w.Hq, w.D), generator=g, device=dev).to(tdt)
    k = torch.randn((1, R, w.Hkv, w.D), generator=g, device=dev).to(tdt)
    v = torch.randn((1, R, w.Hkv, w.D), generator=g, device=dev).to(tdt)
    do = torch.randn((1, R, w.Hq, w.D), generator=g, device=dev).to(tdt)
    out = torch.empty_like(q)
    lse = torch.empty((1, w.Hq, R), device=dev, dtype=torch.float32)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    pos_d = torch.empty((1, R), device=dev, dtype=torch.int32)
    se_d = torch.empty((1, R), device=dev, dtype=torch.int32)
    wsf = torch.empty(max(lib.tree_attn_workspace_bytes(dt_code, 1, R, w.Hq, w.Hkv, w.D, False), 1),
                      device=dev, dtype=torch.uint8)
    # the backward workspace this row's dK/dV plan uses (fixed part + its partial-sum slots)
    wsb = torch.empty(max(lib.tree_attn_bwd_workspace_bytes_for(dt_code, lay.subtree_end, w.Hq, w.Hkv, w.D), 1),
                      device=dev, dtype=torch.uint8)

    # pinned, double-buffered host layout buffers
    parent_h = np.ascontiguousarray(parent, dtype=np.int32)
    seq_last_h = np.ascontiguousarray(seq_last, dtype=np.int32)
    ti_cap = int(lay.seq_offsets[-1])
    bufs = []
    for _ in range(2):
        pos_p = torch.empty(R, dtype=torch.int32, pin_memory=True)
        se_p = torch.empty(R, dtype=torch.int32, pin_memory=True)
        bufs.append({"pos": pos_p, "se": se_p, "slot": np.empty(R, np.int32),
                     "off": np.empty(len(seq_last_h) + 1, np.int64), "ti": np.empty(max(ti_cap, 1), np.int32),
                     "ev": torch.cuda.Event()})
    i32 = C.POINTER(C.c_int32)
    i64 = C.POINTER(C.c_int64)
    stream = torch.cuda.current_stream()
    scale = w.D ** -0.5
    host_ms = []

    def ptr(a, t):
        return a.ctypes.data_as(t)

    def step(i, timing=None):
        bf = bufs[i % 2]
        bf["ev"].synchronize()  # the copy that last read these pinned buffers is done
        t0 = time.perf_counter()
        st = lib.lib.tree_pack_layout(n, ptr(parent_h, i32), len(seq_last_h), ptr(seq_last_h, i32), R,
                                      ptr(bf["slot"], i32), C.cast(bf["pos"].data_ptr(), i32),
                                      C.cast(bf["se"].data_ptr(), i32), ptr(bf["off"], i64), ptr(bf["ti"], i32),
                                      ti_cap)
        host_ms.append(1e3 * (time.perf_counter() - t0))
        assert st == 0
        pos_d.view(-1).copy_(bf["pos"], non_blocking=True)
        se_d.view(-1).copy_(bf["se"], non_blocking=True)
        bf["ev"].record(stream)
        if timing:
            timing[0].record(stream)
        lib.tree_rope_qk(q, k, pos_d, w.theta)
        if timing:
            timing[1].record(stream)
        lib.tree_attn_fwd(q, k, v, se_d, scale, out=out, lse=lse, ws=wsf)
        if timing:
            timing[2].record(stream)
        lib.tree_attn_bwd(q, k, v, se_d, out, lse, do, scale, dq=dq, dk=dk, dv=dv, ws=wsb)
        if timing:
            timing[3].record(stream)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    host_ms.clear()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i, events[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = 1e3 * wall / args.steps
    rope_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in events]))
    fwd_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in events]))
    bwd_ms = float(np.mean([e[2].elapsed_time(e[3]) for e in events]))

    # one cold step at a time: a 1 GiB write between steps evicts the 256 MB
    # last-level cache, so the step reads its inputs from HBM
    flush = torch.empty(1 << 28, dtype=torch.float32, device=dev)
    cold = []
    for i in range(3):
        flush.fill_(float(i))
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
        step(args.warmup + args.steps + i, ev)
        torch.cuda.synchronize()
        cold.append(ev[0].elapsed_time(ev[3]))
    del flush
    # the matrix-core rate this GPU sustains on a plain chain of bf16 products
    sink = torch.zeros(256, dtype=torch.float32, device=dev)
    blocks = 8 * torch.cuda.get_device_properties(dev).multi_processor_count
    lib.tree_mfma_peak(blocks, 256, sink)
    torch.cuda.synchronize()
    p0, p1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    p0.record()
    peak_flops = lib.tree_mfma_peak(blocks, 20000, sink)
    p1.record()
    torch.cuda.synchronize()
    measured_peak = peak_flops / (p0.elapsed_time(p1) * 1e-3) / 1e12

    value = total_flops / (ms_step * 1e-3) / 1e12
    bwd_tf = bwd_flops / (bwd_ms * 1e-3) / 1e12
    fwd_bytes, bwd_bytes = algorithmic_bytes(w, n)
    fwd_gbs = fwd_bytes / (fwd_ms * 1e-3) / 1e9
    bwd_gbs = bwd_bytes / (bwd_ms * 1e-3) / 1e9
    traffic = measured_traffic(w.name)
    # matrix-core bound unless the row's algorithmic flop per byte is below the machine balance
    # (2.5 PFLOP/s / 8 TB/s), as for independent short sequences
    hbm_bound = (fwd_flops + bwd_flops) / (fwd_bytes + bwd_bytes) < PEAK_BF16_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9)
    if hbm_bound:
        roofline = {"kernel": "tree_attn_bwd (every kernel of the call)", "bound": "hbm",
                    "achieved": round(bwd_gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                    "frac": round(bwd_gbs / PEAK_HBM_GBS, 4)}
    else:
        roofline = {"kernel": "tree_attn_bwd (every kernel of the call)", "bound": "mfma",
                    "achieved": round(bwd_tf, 3), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                    "frac": round(bwd_tf / PEAK_BF16_TFLOPS, 4)}
    roofline["traffic"] = traffic
    roofline["traffic_source"] = (f"profiles/{w.name}_traffic.md: rocprofv3 FETCH_SIZE and WRITE_SIZE of every "
                                  "backward kernel, scaled by a plain copy, taken on these kernel sources "
                                  "(not measured in this run)") if traffic is not None else None
    roofline["algorithmic_bytes"] = int(bwd_bytes)
    rec = {
        "metric": "tree-attn fwd+bwd ancestor-pair TFLOP/s & forwarded tok/s, 32K row, 1 GPU",
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": describe(w, n, R, pairs),
        "forwarded_tok_s": round(n / (ms_step * 1e-3), 1),
        "raw_tok_s": round(w.raw_tokens / (ms_step * 1e-3), 1),
        "breakdown_ms": {"rope_q_k": round(rope_ms, 4), "fwd": round(fwd_ms, 4), "bwd": round(bwd_ms, 4),
                         "host_layout": round(float(np.mean(host_ms)), 4)},
        "tflops_fwd": round(fwd_flops / (fwd_ms * 1e-3) / 1e12, 3),
        "tflops_bwd": round(bwd_tf, 3),
        "frac_of_bf16_peak_step": round(value / PEAK_BF16_TFLOPS, 4),
        "measured_mfma_peak_tflops": round(measured_peak, 1),
        "frac_of_measured_peak_step": round(value / measured_peak, 4),
        "cold_ms_per_step": round(float(np.median(cold)), 4),
        "counts": row_counts(w, lay, n, R),
        "tiles_per_kv_head": tile_classes(w, lay.subtree_end.astype(np.int64), R),
        "hbm_gbs": {"fwd": round(fwd_gbs, 1), "bwd": round(bwd_gbs, 1),
                    "algorithmic_bytes_fwd": int(fwd_bytes), "algorithmic_bytes_bwd": int(bwd_bytes)},
        "bwd_workspace_bytes": int(wsb.numel()),
        "roofline": roofline,
        "source_hash": source_hash(),
    }
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(w, total_flops, args.cpu_seconds)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
