"""libltree.so loads and exports every entry point include/ltree.h declares;
host-side argument checks and workspace sizing work without a GPU (no kernel
is launched by any call here)."""

import ctypes
import os
import re

import pytest
import torch

# The argument-error cases below pass fake device addresses that the library
# must reject before any launch.  They run only where no GPU is visible, so a
# regression in the checks can never turn into a launch on fake pointers; the
# GPU tests repeat the error paths with real tensors.
no_gpu = pytest.mark.skipif(torch.cuda.is_available(), reason="fake pointers: CPU-only check")

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ltree.h")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(ltree_[a-z_]+)\s*\(", src)))


def test_header_declares_the_entry_points():
    names = _declared()
    for n in ("ltree_build_mask", "ltree_attn", "ltree_attn_workspace_bytes",
              "ltree_attn_partials", "ltree_attn_merge", "ltree_status_string",
              "ltree_version", "ltree_prefix_attn", "ltree_window_attn",
              "ltree_window_attn_workspace_bytes", "ltree_attn_paged",
              "ltree_attn_paged_workspace_bytes", "ltree_window_attn_paged",
              "ltree_window_attn_paged_workspace_bytes", "ltree_tree_rope", "ltree_commit_kv",
              "ltree_attn_strided", "ltree_attn_strided_workspace_bytes",
              "ltree_attn_noalloc"):
        assert n in names


def test_library_exports_every_declared_symbol():
    import tree_attention_amd as ta
    lib = ctypes.CDLL(ta.LIBRARY_PATH)
    for n in _declared():
        assert hasattr(lib, n), n
    assert set(_declared()) == set(ta.EXPORTED)


def test_version_and_status_strings():
    import tree_attention_amd as ta
    assert ta.ltree_version() == 130
    assert ta.ltree_status_string(0) == "ok"
    assert "workspace" in ta.ltree_status_string(ta.LTREE_ERR_WORKSPACE)
    assert "scratch" in ta.ltree_status_string(ta.LTREE_ERR_SCRATCH)
    assert ta.ltree_status_string(12345) == "unknown status"


def test_workspace_sizing():
    import tree_attention_amd as ta
    n = ta.ltree_attn_workspace_bytes(1, 64, 40, 8, 128, 32768)
    assert n > 0 and n % 256 == 0
    # bigger prefixes never need less
    assert ta.ltree_attn_workspace_bytes(1, 64, 40, 8, 128, 65536) >= n
    assert ta.ltree_attn_workspace_bytes(1, 64, 40, 8, 128, 0) > 0
    for bad in [(0, 64, 40, 8, 128, 10), (1, 0, 40, 8, 128, 10), (1, 64, 40, 7, 128, 10),
                (1, 64, 40, 8, 96, 10), (1, 257, 40, 8, 128, 10), (1, 64, 40, 8, 128, -1)]:
        assert ta.ltree_attn_workspace_bytes(*bad) == 0, bad


def _raw():
    import tree_attention_amd as ta
    return ctypes.CDLL(ta.LIBRARY_PATH), ta


@no_gpu
@pytest.mark.parametrize("case,expect", [
    (dict(B=0), -1), (dict(T=0), -1), (dict(Hkv=3), -1), (dict(scale=0.0), -1),
    (dict(scale=float("nan")), -1), (dict(D=96), -2), (dict(T=257), -2), (dict(dtype=7), -1),
    (dict(q=None), -1), (dict(workspace=None), -1), (dict(ws_bytes=16), -3),
    (dict(workspace=0x1010), -3), (dict(q=0x1008), -1), (dict(max_prefix_len=-5), -1),
])
def test_attn_argument_errors(case, expect):
    lib, ta = _raw()
    fn = lib.ltree_attn
    P, I, S, F = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t, ctypes.c_float
    fn.restype = I
    fn.argtypes = [I, I, I, I, I, I, F, P, P, P, P, I, P, P, P, P, P, P, S, P]
    a = dict(dtype=1, B=1, T=8, Hq=8, Hkv=2, D=128, scale=0.1, q=0x1000, kp=0x2000,
             vp=0x3000, off=0x4000, max_prefix_len=100, kt=0x5000, vt=0x6000, mask=0x7000,
             o=0x8000, lse=0x9000, workspace=0x100000, ws_bytes=1 << 40, stream=None)
    a.update(case)
    st = fn(a["dtype"], a["B"], a["T"], a["Hq"], a["Hkv"], a["D"], a["scale"], a["q"], a["kp"],
            a["vp"], a["off"], a["max_prefix_len"], a["kt"], a["vt"], a["mask"], a["o"],
            a["lse"], a["workspace"], a["ws_bytes"], a["stream"])
    assert st == expect


@no_gpu
def test_build_mask_argument_errors():
    lib, ta = _raw()
    fn = lib.ltree_build_mask
    P, I = ctypes.c_void_p, ctypes.c_int
    fn.restype = I
    fn.argtypes = [P, I, I, P, P, P]
    assert fn(None, 1, 8, 0x1000, None, None) == -1
    assert fn(0x1000, 1, 8, None, None, None) == -1
    assert fn(0x1000, 0, 8, 0x2000, None, None) == -1
    assert fn(0x1000, 1, 257, 0x2000, None, None) == -2


def test_strided_workspace_sizing():
    import tree_attention_amd as ta
    packed = ta.ltree_attn_workspace_bytes(1, 64, 40, 8, 128, 32768)
    # an interleaved cache (stride 2 * Hkv * D) plans like the packed one
    assert ta.ltree_attn_strided_workspace_bytes(1, 64, 40, 8, 128, 32768, 2048, 2048) == packed
    for ks, vs in [(1023, 1024), (1024, 1000), (1028, 1024), (0, 1024), (1 << 25, 1024)]:
        assert ta.ltree_attn_strided_workspace_bytes(1, 64, 40, 8, 128, 32768, ks, vs) == 0, (ks, vs)


@no_gpu
@pytest.mark.parametrize("ks,vs,expect", [
    (1024, 1024, -3), (2048, 1024, -3),        # valid strides: stopped by the tiny workspace
    (1023, 1024, -1), (1024, 1020, -1), (1032 + 4, 1024, -1), (1 << 25, 1024, -2),
])
def test_strided_argument_errors(ks, vs, expect):
    lib, ta = _raw()
    fn = lib.ltree_attn_strided
    P, I, S, F, L = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t, ctypes.c_float, ctypes.c_int64
    fn.restype = I
    fn.argtypes = [I, I, I, I, I, I, F, P, P, P, L, L, P, I, P, P, P, P, P, P, S, P]
    st = fn(1, 1, 8, 8, 8, 128, 0.1, 0x1000, 0x2000, 0x3000, ks, vs, 0x4000, 100, 0x5000,
            0x6000, 0x7000, 0x8000, 0x9000, 0x100000, 16, None)
    assert st == expect


def test_noalloc_scratch_limit_matches_header():
    import tree_attention_amd as ta
    src = open(HEADER).read()
    m = re.search(r"#define LTREE_NOALLOC_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)", src)
    assert m and int(m.group(1)) << int(m.group(2)) == ta.LTREE_NOALLOC_SCRATCH_BYTES
    # the five benchmark workloads fit; a 256-node tree over 32768 keys does not
    for sizes in [(1, 8, 4, 4, 64, 512), (1, 64, 32, 8, 128, 16384), (1, 64, 32, 8, 128, 131072),
                  (1, 64, 40, 8, 128, 32768), (4, 32, 32, 8, 128, 131072)]:
        assert 0 < ta.ltree_attn_workspace_bytes(*sizes) <= ta.LTREE_NOALLOC_SCRATCH_BYTES
    assert ta.ltree_attn_workspace_bytes(1, 256, 40, 8, 128, 32768) > ta.LTREE_NOALLOC_SCRATCH_BYTES


@no_gpu
def test_noalloc_argument_errors():
    """Rejected before any HIP call: bad sizes, and partials beyond the array."""
    lib, ta = _raw()
    fn = lib.ltree_attn_noalloc
    P, I, F = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
    fn.restype = I
    fn.argtypes = [I, I, I, I, I, I, F, P, P, P, P, I, P, P, P, P, P, P]
    fake = P(1 << 20)

    def call(B=1, T=64, Hq=40, Hkv=8, D=128, L=32768):
        return fn(ta.LTREE_BF16, B, T, Hq, Hkv, D, 0.088, fake, fake, fake, fake, L, fake, fake,
                  fake, fake, fake, None)

    assert call(B=0) == ta.LTREE_ERR_INVALID_ARG
    assert call(Hkv=7) == ta.LTREE_ERR_INVALID_ARG
    assert call(D=96) == ta.LTREE_ERR_UNSUPPORTED
    assert call(T=256) == ta.LTREE_ERR_SCRATCH
    assert call(B=8) == ta.LTREE_ERR_SCRATCH
