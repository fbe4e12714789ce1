"""ctypes binding of libltree (include/ltree.h).

Argument marshalling only: every step of the computation runs in the HIP
kernels of libltree.so.  PyTorch supplies device memory and the stream.  The
functions named like the C entry points take torch tensors in the layouts the
header states and return the C status code; ``build_mask`` and ``attn``
allocate their outputs with torch and raise ``LTreeError`` on a bad status.

There is no fallback: if libltree.so is missing or cannot be loaded, importing
this module raises.
"""

from __future__ import annotations

import ctypes
import os

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libltree.so")

LTREE_OK = 0
LTREE_ERR_INVALID_ARG = -1
LTREE_ERR_UNSUPPORTED = -2
LTREE_ERR_WORKSPACE = -3
LTREE_ERR_HIP = -4
LTREE_ERR_SCRATCH = -5
LTREE_NOALLOC_SCRATCH_BYTES = 96 << 20
LTREE_F32 = 0
LTREE_BF16 = 1
LTREE_MAX_TREE = 256

EXPORTED = ("ltree_version", "ltree_status_string", "ltree_build_mask",
            "ltree_attn_workspace_bytes", "ltree_attn", "ltree_attn_noalloc", "ltree_attn_partials",
            "ltree_attn_merge", "ltree_prefix_attn", "ltree_attn_strided_workspace_bytes",
            "ltree_attn_strided", "ltree_attn_paged_workspace_bytes",
            "ltree_attn_paged", "ltree_window_attn_paged_workspace_bytes",
            "ltree_window_attn_paged", "ltree_window_attn_workspace_bytes",
            "ltree_window_attn", "ltree_commit_kv", "ltree_tree_rope")


class LTreeError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {ltree_status_string(status)} ({status})")
        self.status = status


def _load() -> ctypes.CDLL:
    if not os.path.exists(_LIB_PATH):
        raise ImportError(
            f"{_LIB_PATH} is not built; run `python tree_attention_amd/build.py` "
            "(hipcc, gfx950) first")
    lib = ctypes.CDLL(_LIB_PATH)
    P, I, S, F = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t, ctypes.c_float
    L = ctypes.c_int64
    sig = {
        "ltree_version": (I, []),
        "ltree_status_string": (ctypes.c_char_p, [I]),
        "ltree_build_mask": (I, [P, I, I, P, P, P]),
        "ltree_attn_workspace_bytes": (S, [I, I, I, I, I, I]),
        "ltree_attn": (I, [I, I, I, I, I, I, F, P, P, P, P, I, P, P, P, P, P, P, S, P]),
        "ltree_attn_noalloc": (I, [I, I, I, I, I, I, F, P, P, P, P, I, P, P, P, P, P, P]),
        "ltree_attn_partials": (I, [I, I, I, I, I, I, F, P, P, P, P, I, P, P, P, P, S, P]),
        "ltree_attn_merge": (I, [I, I, I, I, I, I, P, I, P, P, P, S, P]),
        "ltree_prefix_attn": (I, [I, I, I, I, I, I, F, P, P, P, P, I, P, P, P, S, P]),
        "ltree_attn_strided_workspace_bytes": (S, [I, I, I, I, I, I, L, L]),
        "ltree_attn_strided": (I, [I, I, I, I, I, I, F, P, P, P, L, L, P, I, P, P, P, P, P, P,
                                   S, P]),
        "ltree_attn_paged_workspace_bytes": (S, [I, I, I, I, I, I, I]),
        "ltree_attn_paged": (I, [I, I, I, I, I, I, F, P, P, P, I, I, P, I, P, I, P, P, P, P, P, P,
                                 S, P]),
        "ltree_window_attn_paged_workspace_bytes": (S, [I, I, I, I, I, I, I]),
        "ltree_window_attn_paged": (I, [I, I, I, I, I, I, F, I, P, P, P, I, I, P, I, P, P, P, P,
                                        P, P, P, S, P]),
        "ltree_window_attn_workspace_bytes": (S, [I, I, I, I, I, I]),
        "ltree_window_attn": (I, [I, I, I, I, I, I, F, I, P, P, P, P, P, P, P, P, P, P, S, P]),
        "ltree_commit_kv": (I, [I, I, I, I, I, P, P, P, P, P, P, P, I, P, P]),
        "ltree_tree_rope": (I, [I, I, I, I, I, I, P, P, P, P, ctypes.c_double, P]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype, fn.argtypes = res, args
    return lib


_lib = _load()
LIBRARY_PATH = _LIB_PATH


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _dev(t, name, dtype=None):
    if t is None:
        return
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")


def _dtype_code(t):
    if t.dtype == torch.bfloat16:
        return LTREE_BF16
    if t.dtype == torch.float32:
        return LTREE_F32
    raise ValueError(f"unsupported input dtype {t.dtype}")


# ------------------------------------------------------------ C entry points

def ltree_version() -> int:
    return _lib.ltree_version()


def ltree_status_string(status: int) -> str:
    return _lib.ltree_status_string(int(status)).decode()


def mask_words(T) -> int:
    """64-bit words of one mask row for a tree of T nodes."""
    return (int(T) + 63) // 64


def mask_shape(B, T):
    """[B, T] for trees of up to 64 nodes, [B, T, W] beyond."""
    W = mask_words(T)
    return (B, T) if W == 1 else (B, T, W)


def _check_mask(mask, B, T):
    if tuple(mask.shape) not in ((B, T, mask_words(T)), mask_shape(B, T)):
        raise ValueError(f"mask must be {list(mask_shape(B, T))}")


def ltree_build_mask(parent, mask, status=None, stream=None) -> int:
    """parent int32 [B, T] -> mask int64 [B, T] or [B, T, W] (uint64 bits);
    status int32 [1]."""
    _dev(parent, "parent", torch.int32)
    _dev(mask, "mask", torch.int64)
    _dev(status, "status", torch.int32)
    B, T = parent.shape
    _check_mask(mask, B, T)
    return _lib.ltree_build_mask(_ptr(parent), B, T, _ptr(mask), _ptr(status), _stream(stream))


def ltree_attn_workspace_bytes(B, T, Hq, Hkv, D, max_prefix_len) -> int:
    return int(_lib.ltree_attn_workspace_bytes(B, T, Hq, Hkv, D, max_prefix_len))


def _check_attn_inputs(q, k_prefix, v_prefix, prefix_offsets, k_tree, v_tree, mask):
    dt = q.dtype
    for name, t in (("q", q), ("k_prefix", k_prefix), ("v_prefix", v_prefix),
                    ("k_tree", k_tree), ("v_tree", v_tree)):
        _dev(t, name, dt)
    _dev(prefix_offsets, "prefix_offsets", torch.int32)
    _dev(mask, "mask", torch.int64)
    B, T, Hq, D = q.shape
    Hkv = k_tree.shape[2]
    if k_tree.shape != (B, T, Hkv, D) or v_tree.shape != (B, T, Hkv, D):
        raise ValueError("k_tree/v_tree must be [B, T, Hkv, D]")
    if k_prefix.dim() != 3 or k_prefix.shape[1:] != (Hkv, D) or v_prefix.shape != k_prefix.shape:
        raise ValueError("k_prefix/v_prefix must be [sum L, Hkv, D]")
    if prefix_offsets.shape != (B + 1,):
        raise ValueError("prefix_offsets must be [B+1]")
    _check_mask(mask, B, T)
    return B, T, Hq, Hkv, D


def ltree_attn_partials(q, k_prefix, v_prefix, prefix_offsets, max_prefix_len, k_tree, v_tree,
                        mask, workspace, scale, stream=None) -> int:
    B, T, Hq, Hkv, D = _check_attn_inputs(q, k_prefix, v_prefix, prefix_offsets, k_tree,
                                          v_tree, mask)
    _dev(workspace, "workspace")
    kp = k_prefix if k_prefix.numel() else None
    vp = v_prefix if v_prefix.numel() else None
    return _lib.ltree_attn_partials(
        _dtype_code(q), B, T, Hq, Hkv, D, float(scale), _ptr(q), _ptr(kp), _ptr(vp),
        _ptr(prefix_offsets), int(max_prefix_len), _ptr(k_tree), _ptr(v_tree), _ptr(mask),
        _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream))


def ltree_attn_merge(dtype, B, T, Hq, Hkv, D, prefix_offsets, max_prefix_len, o, lse, workspace,
                     stream=None) -> int:
    """dtype: the torch dtype of the inputs given to ltree_attn_partials."""
    _dev(prefix_offsets, "prefix_offsets", torch.int32)
    _dev(o, "o", torch.float32)
    _dev(lse, "lse", torch.float32)
    _dev(workspace, "workspace")
    code = {torch.float32: LTREE_F32, torch.bfloat16: LTREE_BF16}.get(dtype)
    if code is None:
        raise TypeError(f"unsupported dtype {dtype}")
    return _lib.ltree_attn_merge(
        code, B, T, Hq, Hkv, D, _ptr(prefix_offsets), int(max_prefix_len), _ptr(o), _ptr(lse),
        _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream))


def ltree_attn(q, k_prefix, v_prefix, prefix_offsets, max_prefix_len, k_tree, v_tree, mask,
               o, lse, workspace, scale, stream=None) -> int:
    B, T, Hq, Hkv, D = _check_attn_inputs(q, k_prefix, v_prefix, prefix_offsets, k_tree,
                                          v_tree, mask)
    _dev(o, "o", torch.float32)
    _dev(lse, "lse", torch.float32)
    _dev(workspace, "workspace")
    if o.shape != (B, T, Hq, D) or lse.shape != (B, Hq, T):
        raise ValueError("o must be [B, T, Hq, D] and lse [B, Hq, T]")
    kp = k_prefix if k_prefix.numel() else None
    vp = v_prefix if v_prefix.numel() else None
    return _lib.ltree_attn(
        _dtype_code(q), B, T, Hq, Hkv, D, float(scale), _ptr(q), _ptr(kp), _ptr(vp),
        _ptr(prefix_offsets), int(max_prefix_len), _ptr(k_tree), _ptr(v_tree), _ptr(mask),
        _ptr(o), _ptr(lse), _ptr(workspace), workspace.numel() * workspace.element_size(),
        _stream(stream))


def ltree_attn_noalloc(q, k_prefix, v_prefix, prefix_offsets, max_prefix_len, k_tree, v_tree,
                       mask, o, lse, scale, stream=None) -> int:
    """ltree_attn with its partials in the library's static per-device array
    (no workspace argument; nothing is allocated)."""
    B, T, Hq, Hkv, D = _check_attn_inputs(q, k_prefix, v_prefix, prefix_offsets, k_tree,
                                          v_tree, mask)
    _dev(o, "o", torch.float32)
    _dev(lse, "lse", torch.float32)
    if o.shape != (B, T, Hq, D) or lse.shape != (B, Hq, T):
        raise ValueError("o must be [B, T, Hq, D] and lse [B, Hq, T]")
    kp = k_prefix if k_prefix.numel() else None
    vp = v_prefix if v_prefix.numel() else None
    return _lib.ltree_attn_noalloc(
        _dtype_code(q), B, T, Hq, Hkv, D, float(scale), _ptr(q), _ptr(kp), _ptr(vp),
        _ptr(prefix_offsets), int(max_prefix_len), _ptr(k_tree), _ptr(v_tree), _ptr(mask),
        _ptr(o), _ptr(lse), _stream(stream))


def ltree_prefix_attn(q, k_prefix, v_prefix, prefix_offsets, max_prefix_len, o, lse, workspace,
                      scale, stream=None) -> int:
    """q [B, T, Hq, D] over the prefix alone (no tree part); o, lse as ltree_attn."""
    dt = q.dtype
    for name, t in (("q", q), ("k_prefix", k_prefix), ("v_prefix", v_prefix)):
        _dev(t, name, dt)
    _dev(prefix_offsets, "prefix_offsets", torch.int32)
    _dev(o, "o", torch.float32)
    _dev(lse, "lse", torch.float32)
    _dev(workspace, "workspace")
    B, T, Hq, D = q.shape
    if k_prefix.dim() != 3 or k_prefix.shape[2] != D or v_prefix.shape != k_prefix.shape:
        raise ValueError("k_prefix/v_prefix must be [sum L, Hkv, D]")
    Hkv = k_prefix.shape[1]
    if prefix_offsets.shape != (B + 1,):
        raise ValueError("prefix_offsets must be [B+1]")
    if o.shape != (B, T, Hq, D) or lse.shape != (B, Hq, T):
        raise ValueError("o must be [B, T, Hq, D] and lse [B, Hq, T]")
    kp = k_prefix if k_prefix.numel() else None
    vp = v_prefix if v_prefix.numel() else None
    return _lib.ltree_prefix_attn(
        _dtype_code(q), B, T, Hq, Hkv, D, float(scale), _ptr(q), _ptr(kp), _ptr(vp),
        _ptr(prefix_offsets), int(max_prefix_len), _ptr(o), _ptr(lse), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(stream))


def _row_view(t, name, Hkv, D, dtype):
    """A [rows, Hkv, D] device view whose (Hkv, D) part is packed; returns its
    row stride in elements."""
    if t is None or not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    # (a dimension of size one has no meaningful stride)
    packed = (D == 1 or t.stride(2) == 1) and (Hkv == 1 or t.stride(1) == D)
    if t.dim() != 3 or t.shape[1:] != (Hkv, D) or not packed:
        raise ValueError(f"{name} must be a [rows, Hkv, D] view with packed (Hkv, D)")
    return t.stride(0) if t.shape[0] > 1 else Hkv * D


def ltree_attn_strided_workspace_bytes(B, T, Hq, Hkv, D, max_prefix_len, k_row_stride,
                                       v_row_stride) -> int:
    return int(_lib.ltree_attn_strided_workspace_bytes(B, T, Hq, Hkv, D, int(max_prefix_len),
                                                       int(k_row_stride), int(v_row_stride)))


def ltree_attn_strided(q, k_prefix, v_prefix, prefix_offsets, max_prefix_len, k_tree, v_tree,
                       mask, o, lse, workspace, scale, stream=None) -> int:
    """ltree_attn over prefix views [rows, Hkv, D] whose rows are `stride(0)`
    elements apart (e.g. kv[:, 0] and kv[:, 1] of an interleaved cache
    [rows, 2, Hkv, D]).  k_tree, v_tree and mask all None: prefix only."""
    dt = q.dtype
    _dev(q, "q", dt)
    B, T, Hq, D = q.shape
    has_tree = k_tree is not None
    if has_tree:
        _dev(k_tree, "k_tree", dt)
        _dev(v_tree, "v_tree", dt)
        _dev(mask, "mask", torch.int64)
        Hkv = k_tree.shape[2]
        if k_tree.shape != (B, T, Hkv, D) or v_tree.shape != (B, T, Hkv, D):
            raise ValueError("k_tree/v_tree must be [B, T, Hkv, D]")
        _check_mask(mask, B, T)
    else:
        Hkv = k_prefix.shape[1]
    ks = _row_view(k_prefix, "k_prefix", Hkv, D, dt)
    vs = _row_view(v_prefix, "v_prefix", Hkv, D, dt)
    _dev(prefix_offsets, "prefix_offsets", torch.int32)
    _dev(o, "o", torch.float32)
    _dev(lse, "lse", torch.float32)
    _dev(workspace, "workspace")
    if o.shape != (B, T, Hq, D) or lse.shape != (B, Hq, T):
        raise ValueError("o must be [B, T, Hq, D] and lse [B, Hq, T]")
    kp = k_prefix if k_prefix.numel() else None
    vp = v_prefix if v_prefix.numel() else None
    return _lib.ltree_attn_strided(
        _dtype_code(q), B, T, Hq, Hkv, D, float(scale), _ptr(q), _ptr(kp), _ptr(vp), int(ks),
        int(vs), _ptr(prefix_offsets), int(max_prefix_len), _ptr(k_tree), _ptr(v_tree),
        _ptr(mask), _ptr(o), _ptr(lse), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(stream))


def ltree_attn_paged_workspace_bytes(B, T, Hq, Hkv, D, max_prefix_len, page_size) -> int:
    return int(_lib.ltree_attn_paged_workspace_bytes(B, T, Hq, Hkv, D, int(max_prefix_len),
                                                     int(page_size)))


def ltree_attn_paged(q, k_pages, v_pages, block_table, seq_lens, max_prefix_len, k_tree, v_tree,
                     mask, o, lse, workspace, scale, stream=None) -> int:
    """Tree-verification attention over a paged prefix: k_pages/v_pages
    [num_pages, page_size, Hkv, D], block_table int32 [B, max_pages_per_seq],
    seq_lens int32 [B].  k_tree, v_tree and mask all None: prefix only."""
    dt = q.dtype
    for name, t in (("q", q), ("k_pages", k_pages), ("v_pages", v_pages)):
        _dev(t, name, dt)
    for name, t in (("block_table", block_table), ("seq_lens", seq_lens)):
        _dev(t, name, torch.int32)
    _dev(o, "o", torch.float32)
    _dev(lse, "lse", torch.float32)
    _dev(workspace, "workspace")
    B, T, Hq, D = q.shape
    if k_pages.dim() != 4 or k_pages.shape[3] != D or v_pages.shape != k_pages.shape:
        raise ValueError("k_pages/v_pages must be [num_pages, page_size, Hkv, D]")
    num_pages, page_size, Hkv = k_pages.shape[:3]
    if block_table.dim() != 2 or block_table.shape[0] != B or seq_lens.shape != (B,):
        raise ValueError("block_table must be [B, max_pages] and seq_lens [B]")
    tree = (k_tree, v_tree, mask)
    if any(t is not None for t in tree):
        for name, t in (("k_tree", k_tree), ("v_tree", v_tree)):
            _dev(t, name, dt)
            if t.shape != (B, T, Hkv, D):
                raise ValueError(f"{name} must be [B, T, Hkv, D]")
        _dev(mask, "mask", torch.int64)
        _check_mask(mask, B, T)
    if o.shape != (B, T, Hq, D) or lse.shape != (B, Hq, T):
        raise ValueError("o must be [B, T, Hq, D] and lse [B, Hq, T]")
    return _lib.ltree_attn_paged(
        _dtype_code(q), B, T, Hq, Hkv, D, float(scale), _ptr(q), _ptr(k_pages), _ptr(v_pages),
        num_pages, page_size, _ptr(block_table), block_table.shape[1], _ptr(seq_lens),
        int(max_prefix_len), _ptr(k_tree), _ptr(v_tree), _ptr(mask), _ptr(o), _ptr(lse),
        _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream))


def ltree_window_attn_paged_workspace_bytes(B, T, Hq, Hkv, D, window, page_size) -> int:
    return int(_lib.ltree_window_attn_paged_workspace_bytes(B, T, Hq, Hkv, D, int(window),
                                                            int(page_size)))


def ltree_window_attn_paged(q, k_pages, v_pages, block_table, seq_lens, k_tree, v_tree, mask, o,
                            lse, workspace, scale, window, stream=None) -> int:
    """Sliding-window self-attention of the tree tokens over a paged cache
    (pools [num_pages, page_size, Hkv, D], block_table [B, max_pages],
    seq_lens [B])."""
    dt = q.dtype
    for name, t in (("q", q), ("k_pages", k_pages), ("v_pages", v_pages), ("k_tree", k_tree),
                    ("v_tree", v_tree)):
        _dev(t, name, dt)
    for name, t in (("block_table", block_table), ("seq_lens", seq_lens)):
        _dev(t, name, torch.int32)
    _dev(mask, "mask", torch.int64)
    _dev(o, "o", torch.float32)
    _dev(lse, "lse", torch.float32)
    _dev(workspace, "workspace")
    B, T, Hq, D = q.shape
    if k_pages.dim() != 4 or k_pages.shape[3] != D or v_pages.shape != k_pages.shape:
        raise ValueError("k_pages/v_pages must be [num_pages, page_size, Hkv, D]")
    num_pages, page_size, Hkv = k_pages.shape[:3]
    if block_table.dim() != 2 or block_table.shape[0] != B or seq_lens.shape != (B,):
        raise ValueError("block_table must be [B, max_pages] and seq_lens [B]")
    if k_tree.shape != (B, T, Hkv, D) or v_tree.shape != (B, T, Hkv, D):
        raise ValueError("k_tree/v_tree must be [B, T, Hkv, D]")
    _check_mask(mask, B, T)
    if o.shape != (B, T, Hq, D) or lse.shape != (B, Hq, T):
        raise ValueError("o must be [B, T, Hq, D] and lse [B, Hq, T]")
    return _lib.ltree_window_attn_paged(
        _dtype_code(q), B, T, Hq, Hkv, D, float(scale), int(window), _ptr(q), _ptr(k_pages),
        _ptr(v_pages), num_pages, page_size, _ptr(block_table), block_table.shape[1],
        _ptr(seq_lens), _ptr(k_tree), _ptr(v_tree), _ptr(mask), _ptr(o), _ptr(lse),
        _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream))


def ltree_window_attn_workspace_bytes(B, T, Hq, Hkv, D, window) -> int:
    return _lib.ltree_window_attn_workspace_bytes(B, T, Hq, Hkv, D, int(window))


def ltree_window_attn(q, k_cache, v_cache, cache_offsets, k_tree, v_tree, mask, o, lse,
                      workspace, scale, window, stream=None) -> int:
    """Sliding-window self-attention of the tree tokens: node i sees the keys
    of its branch within `window` positions (the last window - depth(i) cache
    rows of its sequence and its ancestors); o, lse as ltree_attn."""
    B, T, Hq, Hkv, D = _check_attn_inputs(q, k_cache, v_cache, cache_offsets, k_tree,
                                          v_tree, mask)
    _dev(o, "o", torch.float32)
    _dev(lse, "lse", torch.float32)
    _dev(workspace, "workspace")
    if o.shape != (B, T, Hq, D) or lse.shape != (B, Hq, T):
        raise ValueError("o must be [B, T, Hq, D] and lse [B, Hq, T]")
    # an empty cache (every L_b = 0) has no storage; the library reads no row
    # of it then, and takes the tree arrays as the non-null stand-in
    kc = k_cache if k_cache.numel() else k_tree
    vc = v_cache if v_cache.numel() else v_tree
    return _lib.ltree_window_attn(
        _dtype_code(q), B, T, Hq, Hkv, D, float(scale), int(window), _ptr(q), _ptr(kc),
        _ptr(vc), _ptr(cache_offsets), _ptr(k_tree), _ptr(v_tree), _ptr(mask), _ptr(o),
        _ptr(lse), _ptr(workspace), workspace.numel() * workspace.element_size(),
        _stream(stream))


def ltree_commit_kv(k_tree, v_tree, accepted, n_accepted, dst_row, k_cache, v_cache,
                    status=None, stream=None) -> int:
    """Copy accepted tree rows into the cache: k_cache[dst_row[b] + j] =
    k_tree[b, accepted[b, j]] for j < n_accepted[b] (same for v)."""
    dt = k_tree.dtype
    for name, t in (("k_tree", k_tree), ("v_tree", v_tree), ("k_cache", k_cache),
                    ("v_cache", v_cache)):
        _dev(t, name, dt)
    for name, t in (("accepted", accepted), ("n_accepted", n_accepted), ("dst_row", dst_row)):
        _dev(t, name, torch.int32)
    _dev(status, "status", torch.int32)
    B, T, Hkv, D = k_tree.shape
    if v_tree.shape != k_tree.shape or accepted.shape != (B, T) or n_accepted.shape != (B,) \
            or dst_row.shape != (B,):
        raise ValueError("k_tree/v_tree [B,T,Hkv,D], accepted [B,T], n_accepted/dst_row [B]")
    if k_cache.dim() != 3 or k_cache.shape[1:] != (Hkv, D) or v_cache.shape != k_cache.shape:
        raise ValueError("k_cache/v_cache must be [rows, Hkv, D]")
    return _lib.ltree_commit_kv(
        _dtype_code(k_tree), B, T, Hkv, D, _ptr(k_tree), _ptr(v_tree), _ptr(accepted),
        _ptr(n_accepted), _ptr(dst_row), _ptr(k_cache), _ptr(v_cache), k_cache.shape[0],
        _ptr(status), _stream(stream))


def ltree_tree_rope(q, k_tree, mask, prefix_offsets, rope_base, stream=None) -> int:
    """Rotate q [B,T,Hq,D] and k_tree [B,T,Hkv,D] in place to the tree positions
    L_b + depth(i) - 1 (depth = popcount of the mask row)."""
    _dev(q, "q")
    _dev(k_tree, "k_tree", q.dtype)
    _dev(mask, "mask", torch.int64)
    _dev(prefix_offsets, "prefix_offsets", torch.int32)
    B, T, Hq, D = q.shape
    if k_tree.dim() != 4 or k_tree.shape[:2] != (B, T) or k_tree.shape[3] != D:
        raise ValueError("k_tree must be [B, T, Hkv, D]")
    if prefix_offsets.shape != (B + 1,):
        raise ValueError("prefix_offsets must be [B+1]")
    _check_mask(mask, B, T)
    return _lib.ltree_tree_rope(_dtype_code(q), B, T, Hq, k_tree.shape[2], D, _ptr(q),
                                _ptr(k_tree), _ptr(mask), _ptr(prefix_offsets),
                                float(rope_base), _stream(stream))


# --------------------------------------------------- allocating conveniences

def build_mask(parent, with_status=True, stream=None):
    """Allocate and build the mask; returns (mask int64 [B, T] or [B, T, W], status
    int32 [1])."""
    B, T = parent.shape
    mask = torch.empty(mask_shape(B, T), dtype=torch.int64, device=parent.device)
    status = torch.empty((1,), dtype=torch.int32, device=parent.device) if with_status else None
    st = ltree_build_mask(parent, mask, status, stream)
    if st != LTREE_OK:
        raise LTreeError(st, "ltree_build_mask")
    return mask, status


def workspace_for(q, k_tree, max_prefix_len):
    B, T, Hq, D = q.shape
    n = ltree_attn_workspace_bytes(B, T, Hq, k_tree.shape[2], D, max_prefix_len)
    if n == 0:
        raise LTreeError(LTREE_ERR_INVALID_ARG, "ltree_attn_workspace_bytes")
    return torch.empty((n,), dtype=torch.uint8, device=q.device)


def attn(q, k_prefix, v_prefix, prefix_offsets, max_prefix_len, k_tree, v_tree, mask, scale,
         workspace=None, stream=None):
    """Allocate o [B,T,Hq,D] fp32 and lse [B,Hq,T] fp32 and run ltree_attn."""
    B, T, Hq, D = q.shape
    o = torch.empty((B, T, Hq, D), dtype=torch.float32, device=q.device)
    lse = torch.empty((B, Hq, T), dtype=torch.float32, device=q.device)
    if workspace is None:
        workspace = workspace_for(q, k_tree, max_prefix_len)
    st = ltree_attn(q, k_prefix, v_prefix, prefix_offsets, max_prefix_len, k_tree, v_tree,
                    mask, o, lse, workspace, scale, stream)
    if st != LTREE_OK:
        raise LTreeError(st, "ltree_attn")
    return o, lse


def prefix_attn(q, k_prefix, v_prefix, prefix_offsets, max_prefix_len, scale, workspace=None,
                stream=None):
    """Allocate o and lse and run ltree_prefix_attn (attention over the prefix alone)."""
    B, T, Hq, D = q.shape
    Hkv = k_prefix.shape[1]
    o = torch.empty((B, T, Hq, D), dtype=torch.float32, device=q.device)
    lse = torch.empty((B, Hq, T), dtype=torch.float32, device=q.device)
    if workspace is None:
        n = ltree_attn_workspace_bytes(B, T, Hq, Hkv, D, max_prefix_len)
        if n == 0:
            raise LTreeError(LTREE_ERR_INVALID_ARG, "ltree_attn_workspace_bytes")
        workspace = torch.empty((n,), dtype=torch.uint8, device=q.device)
    st = ltree_prefix_attn(q, k_prefix, v_prefix, prefix_offsets, max_prefix_len, o, lse,
                           workspace, scale, stream)
    if st != LTREE_OK:
        raise LTreeError(st, "ltree_prefix_attn")
    return o, lse


def attn_strided(q, k_prefix, v_prefix, prefix_offsets, max_prefix_len, k_tree, v_tree, mask,
                 scale, workspace=None, stream=None):
    """Allocate o and lse (and the workspace) and run ltree_attn_strided."""
    B, T, Hq, D = q.shape
    Hkv = k_prefix.shape[1]
    o = torch.empty((B, T, Hq, D), dtype=torch.float32, device=q.device)
    lse = torch.empty((B, Hq, T), dtype=torch.float32, device=q.device)
    if workspace is None:
        ks = _row_view(k_prefix, "k_prefix", Hkv, D, q.dtype)
        vs = _row_view(v_prefix, "v_prefix", Hkv, D, q.dtype)
        n = ltree_attn_strided_workspace_bytes(B, T, Hq, Hkv, D, max_prefix_len, ks, vs)
        if n == 0:
            raise LTreeError(LTREE_ERR_INVALID_ARG, "ltree_attn_strided_workspace_bytes")
        workspace = torch.empty((n,), dtype=torch.uint8, device=q.device)
    st = ltree_attn_strided(q, k_prefix, v_prefix, prefix_offsets, max_prefix_len, k_tree,
                            v_tree, mask, o, lse, workspace, scale, stream)
    if st != LTREE_OK:
        raise LTreeError(st, "ltree_attn_strided")
    return o, lse


def window_attn(q, k_cache, v_cache, cache_offsets, k_tree, v_tree, mask, scale, window,
                workspace=None, stream=None):
    """Allocate o and lse (and the workspace) and run ltree_window_attn."""
    B, T, Hq, D = q.shape
    o = torch.empty((B, T, Hq, D), dtype=torch.float32, device=q.device)
    lse = torch.empty((B, Hq, T), dtype=torch.float32, device=q.device)
    if workspace is None:
        n = ltree_window_attn_workspace_bytes(B, T, Hq, k_tree.shape[2], D, window)
        if n == 0:
            raise LTreeError(LTREE_ERR_INVALID_ARG, "ltree_window_attn_workspace_bytes")
        workspace = torch.empty((n,), dtype=torch.uint8, device=q.device)
    st = ltree_window_attn(q, k_cache, v_cache, cache_offsets, k_tree, v_tree, mask, o, lse,
                           workspace, scale, window, stream)
    if st != LTREE_OK:
        raise LTreeError(st, "ltree_window_attn")
    return o, lse


def attn_paged(q, k_pages, v_pages, block_table, seq_lens, max_prefix_len, k_tree, v_tree, mask,
               scale, workspace=None, stream=None):
    """Allocate o and lse (and the workspace) and run ltree_attn_paged."""
    B, T, Hq, D = q.shape
    Hkv = k_pages.shape[2]
    o = torch.empty((B, T, Hq, D), dtype=torch.float32, device=q.device)
    lse = torch.empty((B, Hq, T), dtype=torch.float32, device=q.device)
    if workspace is None:
        n = ltree_attn_paged_workspace_bytes(B, T, Hq, Hkv, D, max_prefix_len, k_pages.shape[1])
        if n == 0:
            raise LTreeError(LTREE_ERR_INVALID_ARG, "ltree_attn_paged_workspace_bytes")
        workspace = torch.empty((n,), dtype=torch.uint8, device=q.device)
    st = ltree_attn_paged(q, k_pages, v_pages, block_table, seq_lens, max_prefix_len, k_tree,
                          v_tree, mask, o, lse, workspace, scale, stream)
    if st != LTREE_OK:
        raise LTreeError(st, "ltree_attn_paged")
    return o, lse
