"""ctypes binding of libtreeattn.so: argument marshalling only.

Every function here has the name of the C entry point it calls and does no
arithmetic of its own: it checks shapes and dtypes, allocates outputs when
the caller passes none (torch for device memory, NumPy for host memory) and
forwards raw pointers plus the current HIP stream.  If the shared library is
missing, importing this module raises: there is no fallback.
"""

from __future__ import annotations

import ctypes as C
import os
from dataclasses import dataclass

import numpy as np

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libtreeattn.so")

TREE_F32 = 0
TREE_BF16 = 1


class TreeAttnError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{message} [{status}]")
        self.status = status


def _load():
    # torch ships its own HIP runtime with the same soname as ROCm's
    # (libamdhip64.so.7).  Loading torch first makes this library bind to that
    # one runtime, so torch's streams and allocations are valid here.
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    if not os.path.exists(_LIB_PATH):
        raise ImportError(f"{_LIB_PATH} is not built; run `python -m prefix_tree_packed_dfs_amd.build`")
    return C.CDLL(_LIB_PATH)


lib = _load()

_i32p = C.POINTER(C.c_int32)
_i64p = C.POINTER(C.c_int64)
_vp = C.c_void_p

lib.tree_abi_version.restype = C.c_int
lib.tree_status_string.restype = C.c_char_p
lib.tree_status_string.argtypes = [C.c_int]
lib.tree_last_error.restype = C.c_char_p
lib.tree_build_trie.restype = C.c_int
lib.tree_build_trie.argtypes = [C.c_int32, _i64p, _i32p, C.POINTER(C.c_uint8), C.c_int32, _i32p, C.c_int64,
                                _i64p, _i32p]
lib.tree_place_leaves.restype = C.c_int
lib.tree_place_leaves.argtypes = [C.c_int32, _i32p, C.c_int32, _i32p, _i32p, C.c_int32, C.c_int32, _i32p,
                                  _i32p, C.c_int32, _i32p]
lib.tree_plan_rows.restype = C.c_int
lib.tree_plan_rows.argtypes = [C.c_int32, _i64p, _i32p, C.c_int32, C.c_int64, _i32p, _i64p, C.c_int32, _i32p,
                               C.POINTER(C.c_uint8)]
lib.tree_pack_layout.restype = C.c_int
lib.tree_pack_layout.argtypes = [C.c_int32, _i32p, C.c_int32, _i32p, C.c_int32, _i32p, _i32p, _i32p, _i64p,
                                 _i32p, C.c_int64]
lib.tree_validate_subtree_end.restype = C.c_int
lib.tree_validate_subtree_end.argtypes = [_i32p, C.c_int64]
lib.tree_rope.restype = C.c_int
lib.tree_rope.argtypes = [C.c_int, _vp, C.c_int64, C.c_int64, C.c_int64, C.c_int64, _vp, C.c_float, _vp]
lib.tree_rope_qk.restype = C.c_int
lib.tree_rope_qk.argtypes = [C.c_int, _vp, _vp, C.c_int64, C.c_int64, C.c_int64, C.c_int64, C.c_int64, _vp, C.c_float,
                             _vp]
lib.tree_attn_workspace_bytes.restype = C.c_size_t
lib.tree_attn_workspace_bytes.argtypes = [C.c_int, C.c_int64, C.c_int64, C.c_int64, C.c_int64, C.c_int64,
                                          C.c_int]
lib.tree_attn_bwd_workspace_bytes_for.restype = C.c_size_t
lib.tree_attn_bwd_workspace_bytes_for.argtypes = [C.c_int, _i32p, C.c_int64, C.c_int64, C.c_int64, C.c_int64,
                                                  C.c_int64]
lib.tree_attn_fwd.restype = C.c_int
lib.tree_attn_fwd.argtypes = [C.c_int, _vp, _vp, _vp, _vp, C.c_int64, C.c_int64, C.c_int64, C.c_int64,
                              C.c_int64, C.c_float, _vp, _vp, _vp, C.c_size_t, _vp]
lib.tree_attn_fwd_noalloc.restype = C.c_int
lib.tree_attn_fwd_noalloc.argtypes = [C.c_int, _vp, _vp, _vp, _vp, C.c_int64, C.c_int64, C.c_int64, C.c_int64,
                                      C.c_int64, C.c_float, _vp, _vp, _vp]
lib.tree_attn_bwd.restype = C.c_int
lib.tree_attn_bwd.argtypes = [C.c_int, _vp, _vp, _vp, _vp, _vp, _vp, _vp, C.c_int64, C.c_int64, C.c_int64,
                              C.c_int64, C.c_int64, C.c_float, _vp, _vp, _vp, _vp, C.c_size_t, _vp]

lib.tree_gdn_plan.restype = C.c_int
lib.tree_gdn_plan.argtypes = [C.c_int64, _i32p, _i32p, _i32p, C.c_int64, _i64p, _i32p, C.c_int64, _i64p, _i32p,
                              C.c_int64, _i64p, _i64p]
lib.tree_gdn_workspace_bytes.restype = C.c_size_t
lib.tree_gdn_workspace_bytes.argtypes = [C.c_int64] * 7
lib.tree_gdn_fwd.restype = C.c_int
lib.tree_gdn_fwd.argtypes = [C.c_int, _vp, _vp, C.c_int64, _vp, _vp, _vp, _vp, C.c_int64, _vp, C.c_int64, _i32p,
                             C.c_int64, C.c_int64, C.c_int64, C.c_int64, C.c_int64, C.c_int64, C.c_int64, _vp, _vp,
                             C.c_size_t, _vp]

lib.tree_mfma_peak.restype = C.c_int
lib.tree_mfma_peak.argtypes = [C.c_int64, C.c_int64, _vp, C.POINTER(C.c_double), _vp]

EXPORTED = ("tree_abi_version", "tree_status_string", "tree_last_error", "tree_build_trie",
            "tree_place_leaves", "tree_plan_rows", "tree_pack_layout", "tree_validate_subtree_end", "tree_rope", "tree_rope_qk",
            "tree_attn_workspace_bytes", "tree_attn_bwd_workspace_bytes_for",
            "tree_attn_fwd", "tree_attn_fwd_noalloc", "tree_attn_bwd", "tree_gdn_plan", "tree_gdn_workspace_bytes", "tree_gdn_fwd",
            "tree_mfma_peak")


def _check(status: int):
    if status != 0:
        name = lib.tree_status_string(status).decode()
        msg = lib.tree_last_error().decode()
        raise TreeAttnError(status, f"{name}: {msg}")


def _ptr(a: np.ndarray, ctype):
    return a.ctypes.data_as(C.POINTER(ctype))


# ---------------------------------------------------------------------------
# host entry points
# ---------------------------------------------------------------------------

def tree_build_trie(sequences, min_shared: int = 64, trainable=None):
    """Token sequences -> (parent int32 [n_nodes], seq_last int32 [n_seqs]).

    ``trainable``: optional per-sequence boolean flags per token (trainable mode)."""
    seqs = [np.ascontiguousarray(s, dtype=np.int32) for s in sequences]
    lens = np.asarray([len(s) for s in seqs], dtype=np.int64)
    offsets = np.zeros(len(seqs) + 1, dtype=np.int64)
    np.cumsum(lens, out=offsets[1:])
    tokens = np.concatenate(seqs) if seqs and offsets[-1] > 0 else np.zeros(1, dtype=np.int32)
    total = int(offsets[-1])
    train = None
    if trainable is not None:
        if len(trainable) != len(seqs) or any(len(t) != len(s) for t, s in zip(trainable, seqs)):
            raise ValueError("trainable flags must match the sequences")
        flat = [np.asarray(t, dtype=np.uint8) for t in trainable]
        train = np.concatenate(flat) if total > 0 else np.zeros(1, dtype=np.uint8)
    parent = np.empty(max(total, 1), dtype=np.int32)
    seq_last = np.empty(max(len(seqs), 1), dtype=np.int32)
    n_nodes = C.c_int64(0)
    _check(lib.tree_build_trie(len(seqs), _ptr(offsets, C.c_int64), _ptr(tokens, C.c_int32),
                               None if train is None else _ptr(train, C.c_uint8), int(min_shared),
                               _ptr(parent, C.c_int32), total, C.byref(n_nodes), _ptr(seq_last, C.c_int32)))
    return parent[:n_nodes.value].copy(), seq_last[:len(seqs)].copy()


PLACE_MODES = {"global": 0, "in_order": 1}


def tree_place_leaves(parent, seq_last, group, seq_len: int, mode: str = "global"):
    """Sequences of a trie -> (row of each sequence int32 [n_seqs], tokens per row int32 [n_rows])."""
    parent = np.ascontiguousarray(parent, dtype=np.int32)
    seq_last = np.ascontiguousarray(seq_last, dtype=np.int32)
    n = len(seq_last)
    grp = None if group is None else np.ascontiguousarray(group, dtype=np.int32)
    if grp is not None and len(grp) != n:
        raise ValueError("one group id per sequence")
    bin_of = np.empty(max(n, 1), dtype=np.int32)
    cap = max(n, 1)
    tokens = np.empty(cap, dtype=np.int32)
    n_bins = C.c_int32(0)
    _check(lib.tree_place_leaves(len(parent), _ptr(parent, C.c_int32), n, _ptr(seq_last, C.c_int32),
                                 None if grp is None else _ptr(grp, C.c_int32), int(seq_len), PLACE_MODES[mode],
                                 _ptr(bin_of, C.c_int32), _ptr(tokens, C.c_int32), cap, C.byref(n_bins)))
    return bin_of[:n].copy(), tokens[:n_bins.value].copy()


def tree_plan_rows(sequences, token_budget: int, fork_threshold_tokens: int = 1024):
    """Samples -> (row of each sample int32 [n_seqs], forwarded tokens per row int64 [n_rows],
    forked flags uint8 [n_seqs]), rows grown in input order under the forwarded-token budget."""
    seqs = [np.ascontiguousarray(s, dtype=np.int32) for s in sequences]
    n = len(seqs)
    offsets = np.zeros(n + 1, dtype=np.int64)
    np.cumsum([len(s) for s in seqs], out=offsets[1:])
    tokens = np.concatenate(seqs) if n and offsets[-1] else np.zeros(1, np.int32)
    row_of = np.empty(max(n, 1), dtype=np.int32)
    row_tok = np.empty(max(n, 1), dtype=np.int64)
    forked = np.zeros(max(n, 1), dtype=np.uint8)
    n_rows = C.c_int32(0)
    _check(lib.tree_plan_rows(n, _ptr(offsets, C.c_int64), _ptr(tokens, C.c_int32), int(fork_threshold_tokens),
                              int(token_budget), _ptr(row_of, C.c_int32), _ptr(row_tok, C.c_int64), max(n, 1),
                              C.byref(n_rows), _ptr(forked, C.c_uint8)))
    return row_of[:n].copy(), row_tok[:n_rows.value].copy(), forked[:n].copy()


@dataclass
class PackedLayout:
    slot_node: np.ndarray      # [row_len] int32
    pos_ids: np.ndarray        # [row_len] int32
    subtree_end: np.ndarray    # [row_len] int32
    seq_offsets: np.ndarray    # [n_seqs+1] int64
    token_index: np.ndarray    # [seq_offsets[-1]] int32

    def sequence_slots(self, s: int) -> np.ndarray:
        return self.token_index[self.seq_offsets[s]:self.seq_offsets[s + 1]]


def tree_pack_layout(parent, seq_last, row_len: int) -> PackedLayout:
    parent = np.ascontiguousarray(parent, dtype=np.int32)
    seq_last = np.ascontiguousarray(seq_last, dtype=np.int32)
    n, ns = len(parent), len(seq_last)
    slot_node = np.empty(max(row_len, 1), dtype=np.int32)
    pos_ids = np.empty(max(row_len, 1), dtype=np.int32)
    se = np.empty(max(row_len, 1), dtype=np.int32)
    offs = np.empty(ns + 1, dtype=np.int64)
    pp = _ptr(parent if n else np.zeros(1, np.int32), C.c_int32)
    sp = _ptr(seq_last if ns else np.zeros(1, np.int32), C.c_int32)
    _check(lib.tree_pack_layout(n, pp, ns, sp, int(row_len), _ptr(slot_node, C.c_int32), _ptr(pos_ids, C.c_int32),
                                _ptr(se, C.c_int32), _ptr(offs, C.c_int64), None, 0))
    ti = np.empty(max(int(offs[-1]), 1), dtype=np.int32)
    _check(lib.tree_pack_layout(n, pp, ns, sp, int(row_len), _ptr(slot_node, C.c_int32), _ptr(pos_ids, C.c_int32),
                                _ptr(se, C.c_int32), _ptr(offs, C.c_int64), _ptr(ti, C.c_int32), len(ti)))
    return PackedLayout(slot_node[:row_len], pos_ids[:row_len], se[:row_len], offs, ti[:int(offs[-1])])


def tree_validate_subtree_end(subtree_end) -> None:
    se = np.ascontiguousarray(subtree_end, dtype=np.int32)
    _check(lib.tree_validate_subtree_end(_ptr(se if len(se) else np.zeros(1, np.int32), C.c_int32), len(se)))


# ---------------------------------------------------------------------------
# device entry points (torch tensors for memory and the current stream)
# ---------------------------------------------------------------------------

def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.float32:
        return TREE_F32
    if t.dtype == torch.bfloat16:
        return TREE_BF16
    raise TypeError(f"unsupported dtype {t.dtype}")


def _dev(t, name):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def _out(t, name, shape, dtype, like=None):
    """A caller-supplied output buffer: right shape and dtype, or ValueError before any launch
    (the kernels write the full extent the sizes imply)."""
    if t is None:
        return None
    if tuple(t.shape) != tuple(shape) or t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype} {list(shape)}, got {t.dtype} {list(t.shape)}")
    if like is not None and t.device != like.device:
        raise ValueError(f"{name} must be on {like.device}")
    return t


def _stream():
    torch = _torch()
    return torch.cuda.current_stream().cuda_stream


def tree_mfma_peak(blocks: int, iters: int, sink) -> float:
    """Enqueue the matrix-core rate probe on the current stream; returns the flops it performs."""
    flops = C.c_double(0.0)
    _check(lib.tree_mfma_peak(int(blocks), int(iters), sink.data_ptr(), C.byref(flops), _stream()))
    return flops.value


def tree_rope(x, pos_ids, theta: float = 10000.0):
    """Rotate x [B, N, H, D] in place at depth pos_ids [B, N] (int32)."""
    torch = _torch()
    if x.dim() != 4:
        raise ValueError("x must be [B, N, H, D]")
    B, N, H, D = x.shape
    if pos_ids.dtype != torch.int32 or tuple(pos_ids.shape) != (B, N):
        raise ValueError("pos_ids must be int32 [B, N]")
    _check(lib.tree_rope(_dtype_code(x), _dev(x, "x"), B, N, H, D, _dev(pos_ids, "pos_ids"), float(theta),
                         _stream()))
    return x


def tree_rope_qk(q, k, pos_ids, theta: float = 10000.0):
    """Rotate q [B, N, Hq, D] and k [B, N, Hkv, D] in place at depth pos_ids [B, N] (int32), one launch."""
    torch = _torch()
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("q and k must be [B, N, H, D]")
    B, N, Hq, D = q.shape
    Hkv = k.shape[2]
    if tuple(k.shape) != (B, N, Hkv, D) or k.dtype != q.dtype:
        raise ValueError("k must be [B, N, Hkv, D] with q's dtype")
    if pos_ids.dtype != torch.int32 or tuple(pos_ids.shape) != (B, N):
        raise ValueError("pos_ids must be int32 [B, N]")
    _check(lib.tree_rope_qk(_dtype_code(q), _dev(q, "q"), _dev(k, "k"), B, N, Hq, Hkv, D, _dev(pos_ids, "pos_ids"),
                            float(theta), _stream()))
    return q, k


def tree_attn_workspace_bytes(dtype_code: int, B, N, Hq, Hkv, D, bwd: bool) -> int:
    return int(lib.tree_attn_workspace_bytes(int(dtype_code), B, N, Hq, Hkv, D, 1 if bwd else 0))


def tree_attn_bwd_workspace_bytes_for(dtype_code: int, subtree_end, Hq, Hkv, D) -> int:
    """Backward workspace the dK/dV plan of these rows uses; subtree_end [B, N] (or [N]) int32 on the host."""
    se = np.ascontiguousarray(subtree_end, dtype=np.int32)
    if se.ndim == 1:
        se = se[None]
    B, N = se.shape
    return int(lib.tree_attn_bwd_workspace_bytes_for(int(dtype_code), _ptr(se if se.size else np.zeros(1, np.int32),
                                                                           C.c_int32), B, N, Hq, Hkv, D))


def _shapes(q, k, v, subtree_end):
    torch = _torch()
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be [B, N, H, D]")
    B, N, Hq, D = q.shape
    Hkv = k.shape[2]
    if tuple(k.shape) != (B, N, Hkv, D) or tuple(v.shape) != (B, N, Hkv, D):
        raise ValueError("k, v must be [B, N, Hkv, D] matching q")
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k, v must share a dtype")
    if subtree_end.dtype != torch.int32 or tuple(subtree_end.shape) != (B, N):
        raise ValueError("subtree_end must be int32 [B, N]")
    return B, N, Hq, Hkv, D


def _workspace(dt, B, N, Hq, Hkv, D, bwd, ws, device):
    """The caller's workspace, or the largest one these sizes can use.  A backward workspace smaller
    than that is the caller's choice (the library takes fewer partial-sum slots, down to its fixed
    part, and reports TREE_ERR_CAPACITY below it)."""
    torch = _torch()
    need = tree_attn_workspace_bytes(dt, B, N, Hq, Hkv, D, bwd)
    if ws is None:
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=device)
    if not bwd and ws.numel() * ws.element_size() < need:
        raise ValueError(f"workspace needs {need} bytes")
    return ws


def tree_attn_fwd(q, k, v, subtree_end, softmax_scale=None, out=None, lse=None, ws=None):
    """Returns (out [B,N,Hq,D], lse [B,Hq,N] fp32)."""
    torch = _torch()
    B, N, Hq, Hkv, D = _shapes(q, k, v, subtree_end)
    dt = _dtype_code(q)
    scale = D ** -0.5 if softmax_scale is None else float(softmax_scale)
    out = _out(out, "out", q.shape, q.dtype, q)
    lse = _out(lse, "lse", (B, Hq, N), torch.float32, q)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, Hq, N), dtype=torch.float32, device=q.device)
    ws = _workspace(dt, B, N, Hq, Hkv, D, False, ws, q.device)
    _check(lib.tree_attn_fwd(dt, _dev(q, "q"), _dev(k, "k"), _dev(v, "v"), _dev(subtree_end, "subtree_end"),
                             B, N, Hq, Hkv, D, scale, _dev(out, "out"), _dev(lse, "lse"), ws.data_ptr(),
                             ws.numel() * ws.element_size(), _stream()))
    return out, lse


def tree_attn_fwd_noalloc(q, k, v, subtree_end, softmax_scale=None, out=None, lse=None):
    """tree_attn_fwd with the library's fixed per-GPU table array instead of a workspace; returns (out, lse)."""
    torch = _torch()
    B, N, Hq, Hkv, D = _shapes(q, k, v, subtree_end)
    dt = _dtype_code(q)
    scale = D ** -0.5 if softmax_scale is None else float(softmax_scale)
    out = _out(out, "out", q.shape, q.dtype, q)
    lse = _out(lse, "lse", (B, Hq, N), torch.float32, q)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, Hq, N), dtype=torch.float32, device=q.device)
    _check(lib.tree_attn_fwd_noalloc(dt, _dev(q, "q"), _dev(k, "k"), _dev(v, "v"), _dev(subtree_end, "subtree_end"),
                                     B, N, Hq, Hkv, D, scale, _dev(out, "out"), _dev(lse, "lse"), _stream()))
    return out, lse


def tree_attn_bwd(q, k, v, subtree_end, out, lse, dout, softmax_scale=None, dq=None, dk=None, dv=None, ws=None):
    """Returns (dq, dk, dv)."""
    torch = _torch()
    B, N, Hq, Hkv, D = _shapes(q, k, v, subtree_end)
    dt = _dtype_code(q)
    scale = D ** -0.5 if softmax_scale is None else float(softmax_scale)
    for t, nm in ((out, "out"), (dout, "dout")):
        if tuple(t.shape) != tuple(q.shape) or t.dtype != q.dtype:
            raise ValueError(f"{nm} must match q")
    if lse.dtype != torch.float32 or tuple(lse.shape) != (B, Hq, N):
        raise ValueError("lse must be fp32 [B, Hq, N]")
    dq = torch.empty_like(q) if dq is None else _out(dq, "dq", q.shape, q.dtype, q)
    dk = torch.empty_like(k) if dk is None else _out(dk, "dk", k.shape, k.dtype, q)
    dv = torch.empty_like(v) if dv is None else _out(dv, "dv", v.shape, v.dtype, q)
    ws = _workspace(dt, B, N, Hq, Hkv, D, True, ws, q.device)
    _check(lib.tree_attn_bwd(dt, _dev(q, "q"), _dev(k, "k"), _dev(v, "v"), _dev(subtree_end, "subtree_end"),
                             _dev(out, "out"), _dev(lse, "lse"), _dev(dout, "dout"), B, N, Hq, Hkv, D, scale,
                             _dev(dq, "dq"), _dev(dk, "dk"), _dev(dv, "dv"), ws.data_ptr(),
                             ws.numel() * ws.element_size(), _stream()))
    return dq, dk, dv


# ---------------------------------------------------------------------------
# gated-delta-rule mixing
# ---------------------------------------------------------------------------

GDN_DIM = 128


@dataclass
class GdnPlan:
    n: int
    parent_slot: np.ndarray     # [n] int32
    segments: np.ndarray        # [n_segments, 4] int32: first chunk, chunk count, parent state slot, own state slot
    chunks: np.ndarray          # [n_chunks, 2] int32: first slot, length
    depth_offsets: np.ndarray   # [n_depths + 1] int32
    n_states: int               # chains whose final state is kept (those with children)

    @property
    def n_segments(self) -> int:
        return int(self.segments.shape[0])

    @property
    def n_chunks(self) -> int:
        return int(self.chunks.shape[0])

    @property
    def n_depths(self) -> int:
        return int(self.depth_offsets.shape[0]) - 1

    def device_tables(self, device):
        """(parent_slot, segments, chunks) as int32 device tensors."""
        torch = _torch()
        return tuple(torch.from_numpy(np.ascontiguousarray(a)).to(device)
                     for a in (self.parent_slot, self.segments, self.chunks))


def tree_gdn_plan(subtree_end, n: int) -> GdnPlan:
    """Chains, chunks and depth buckets of the first ``n`` slots of a row (host)."""
    se = np.ascontiguousarray(np.asarray(subtree_end)[:n], dtype=np.int32)
    if len(se) != n:
        raise ValueError("subtree_end shorter than n")
    ns, nc, nd, nst = C.c_int64(0), C.c_int64(0), C.c_int64(0), C.c_int64(0)
    _check(lib.tree_gdn_plan(n, _ptr(se, C.c_int32), None, None, 0, C.byref(ns), None, 0, C.byref(nc), None, 0,
                             C.byref(nd), C.byref(nst)))
    parent = np.empty(n, np.int32)
    segs = np.empty((ns.value, 4), np.int32)
    chunks = np.empty((nc.value, 2), np.int32)
    offs = np.empty(nd.value + 1, np.int32)
    _check(lib.tree_gdn_plan(n, _ptr(se, C.c_int32), _ptr(parent, C.c_int32), _ptr(segs, C.c_int32), ns.value,
                             C.byref(ns), _ptr(chunks, C.c_int32), nc.value, C.byref(nc), _ptr(offs, C.c_int32),
                             nd.value, C.byref(nd), C.byref(nst)))
    return GdnPlan(n=n, parent_slot=parent, segments=segs, chunks=chunks, depth_offsets=offs, n_states=nst.value)


def tree_gdn_workspace_bytes(n, n_states, n_chunks, Hk, Hv, dk=GDN_DIM, dv=GDN_DIM) -> int:
    return int(lib.tree_gdn_workspace_bytes(n, n_states, n_chunks, Hk, Hv, dk, dv))


def tree_gdn_fwd(x, conv_w, g, beta, plan: GdnPlan, Hk: int, Hv: int, out=None, ws=None, tables=None):
    """Gated-delta-rule mixing over the plan's row.

    x [>= n, C] bf16 (C = (2 Hk + Hv) 128, channels q | k | v), conv_w [C, W] fp32,
    g, beta [>= n, Hv] fp32.  Returns out [n, Hv, 128] bf16 (``out`` may be given,
    first dimension >= n).  ``tables``: device copies from plan.device_tables()."""
    torch = _torch()
    n = plan.n
    Cc = (2 * Hk + Hv) * GDN_DIM
    if x.dtype != torch.bfloat16 or x.dim() != 2 or x.shape[1] != Cc or x.shape[0] < n:
        raise ValueError(f"x must be bf16 [>= {n}, {Cc}]")
    if conv_w.dtype != torch.float32 or conv_w.dim() != 2 or conv_w.shape[0] != Cc:
        raise ValueError(f"conv_w must be fp32 [{Cc}, W]")
    for t, nm in ((g, "g"), (beta, "beta")):
        if t.dtype != torch.float32 or t.dim() != 2 or t.shape[1] != Hv or t.shape[0] < n:
            raise ValueError(f"{nm} must be fp32 [>= {n}, {Hv}]")
    if out is None:
        out = torch.empty((n, Hv, GDN_DIM), dtype=torch.bfloat16, device=x.device)
    if out.dtype != torch.bfloat16 or out.dim() != 3 or tuple(out.shape[1:]) != (Hv, GDN_DIM) or out.shape[0] < n:
        raise ValueError(f"out must be bf16 [>= {n}, {Hv}, {GDN_DIM}]")
    need = tree_gdn_workspace_bytes(n, plan.n_states, plan.n_chunks, Hk, Hv)
    if ws is None:
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=x.device)
    if ws.numel() * ws.element_size() < need:
        raise ValueError(f"workspace needs {need} bytes")
    par, segs, chunks = plan.device_tables(x.device) if tables is None else tables
    offs = np.ascontiguousarray(plan.depth_offsets, dtype=np.int32)
    _check(lib.tree_gdn_fwd(TREE_BF16, _dev(x, "x"), _dev(conv_w, "conv_w"), conv_w.shape[1], _dev(g, "g"),
                            _dev(beta, "beta"), _dev(par, "parent_slot"), _dev(segs, "segments"), plan.n_segments,
                            _dev(chunks, "chunks"), plan.n_chunks, _ptr(offs, C.c_int32), plan.n_depths,
                            plan.n_states, n, Hk, Hv,
                            GDN_DIM, GDN_DIM, _dev(out, "out"), ws.data_ptr(), ws.numel() * ws.element_size(),
                            _stream()))
    return out
