"""Hybrid tree-verification attention for AMD Instinct MI355X (gfx950).

The computation lives in ``libltree.so`` (HIP kernels behind the C ABI of
``include/ltree.h``); this package is its thin Python binding.  Importing the
package loads the library and raises if it is not built.
"""

from ._binding import (  # noqa: F401
    EXPORTED,
    LIBRARY_PATH,
    LTREE_BF16,
    LTREE_ERR_HIP,
    LTREE_ERR_INVALID_ARG,
    LTREE_ERR_UNSUPPORTED,
    LTREE_ERR_WORKSPACE,
    LTREE_F32,
    LTREE_MAX_TREE,
    LTREE_OK,
    LTreeError,
    attn,
    attn_paged,
    attn_strided,
    build_mask,
    ltree_attn,
    ltree_attn_merge,
    ltree_attn_paged,
    ltree_attn_paged_workspace_bytes,
    ltree_attn_partials,
    ltree_attn_strided,
    ltree_attn_strided_workspace_bytes,
    ltree_attn_workspace_bytes,
    ltree_build_mask,
    ltree_commit_kv,
    ltree_prefix_attn,
    ltree_status_string,
    ltree_tree_rope,
    ltree_version,
    ltree_window_attn,
    ltree_window_attn_paged,
    ltree_window_attn_paged_workspace_bytes,
    ltree_window_attn_workspace_bytes,
    mask_shape,
    mask_words,
    prefix_attn,
    window_attn,
    workspace_for,
)
