"""Attention and gated-delta-rule mixing over prefix-tree-packed rows on AMD Instinct MI355X (gfx950).

The Python names mirror the C entry points of include/tree_attn.h; all work
happens in libtreeattn.so (host C++ for the integer layout, HIP kernels for
everything on the device).
"""

from ._lib import (  # noqa: F401
    EXPORTED,
    GdnPlan,
    TREE_BF16,
    TREE_F32,
    PackedLayout,
    TreeAttnError,
    lib,
    tree_attn_bwd,
    tree_attn_fwd,
    tree_attn_fwd_noalloc,
    tree_attn_workspace_bytes,
    tree_attn_bwd_workspace_bytes_for,
    tree_build_trie,
    tree_gdn_fwd,
    tree_gdn_plan,
    tree_gdn_workspace_bytes,
    tree_mfma_peak,
    tree_place_leaves,
    tree_plan_rows,
    tree_pack_layout,
    tree_rope,
    tree_rope_qk,
    tree_validate_subtree_end,
)
