"""GPU: tree_attn_fwd_noalloc (tables in the library's fixed per-GPU array) against tree_attn_fwd (tables in a
caller workspace), through the C ABI: the same kernels, so the same results bit for bit, on calls in a row
whose sizes shrink (the second call must not depend on what the first left in the array)."""

import numpy as np
import pytest

from synth import from_sequences, grpo_group

from .pipeline import log

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import prefix_tree_packed_dfs_amd  # noqa: F401  (fails loudly if the library is not built)
    yield


def _row(w):
    import torch

    import prefix_tree_packed_dfs_amd as lib
    parent, seq_last = lib.tree_build_trie(w.sequences, min_shared=64)
    R = w.row_length(len(parent))
    lay = lib.tree_pack_layout(parent, seq_last, R)
    se = torch.from_numpy(lay.subtree_end.astype(np.int32)).view(1, R).cuda()
    g = torch.Generator().manual_seed(R)
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    mk = lambda H: torch.randn(1, R, H, w.D, generator=g).to(tdt).cuda()  # noqa: E731
    return mk(w.Hq), mk(w.Hkv), mk(w.Hkv), se


def _small_tree(dtype, Hq, Hkv, D):
    rng = np.random.default_rng(3)
    seqs = [np.repeat(rng.integers(0, 2, size=L // 40 + 1), 40)[:L].astype(np.int32)
            for L in rng.integers(50, 600, size=6)]
    return from_sequences(seqs, Hq=Hq, Hkv=Hkv, D=D, dtype=dtype, seed_base=23_000, name="small_tree")


def test_noalloc_forward_equals_forward_on_shrinking_calls():
    import torch

    import prefix_tree_packed_dfs_amd as lib
    cases = [grpo_group(), _small_tree("bf16", 4, 2, 128), _small_tree("bf16", 8, 1, 64),
             _small_tree("f32", 2, 2, 64)]
    for w in cases:
        q, k, v, se = _row(w)
        log(f"case noalloc {w.name}: dtype={w.dtype} Hq={w.Hq} Hkv={w.Hkv} D={w.D} N={q.shape[1]}")
        ref_out, ref_lse = lib.tree_attn_fwd(q, k, v, se)
        for rep in range(2):
            out, lse = lib.tree_attn_fwd_noalloc(q, k, v, se)
            torch.cuda.synchronize()
            assert torch.equal(out, ref_out), f"{w.name}: out differs (call {rep})"
            assert torch.equal(lse, ref_lse), f"{w.name}: lse differs (call {rep})"
        log("    out and lse bitwise equal to tree_attn_fwd on two calls")
