"""The draft model's sliding-window self-attention over a draft tree on the
GPU, through the C ABI, against the fp64 oracle.

Small cases cover windows shorter and longer than the cache, an empty cache,
a window equal to T (the deepest node sees no cache key), windows that are
not multiples of the 64-key tile, several splits, bf16 and fp32, D = 64 and
128.  The QwQ-shaped case (window 512 after a 32768-row cache, 64 tree
tokens, 40/8 heads) is checked on every row in test_gpu_full_sizes.py."""

import zlib

import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import BF16_O_TOL, F32_O_TOL, LSE_TOL, say
from workloads import make_workload

pytestmark = pytest.mark.gpu

SMALL = {
    # name: (B, T, Hq, Hkv, D, cache_lens, trees, dtype, window)
    "w64_chain_eq_T": (1, 64, 8, 2, 128, [1000], "chain", "bf16", 64),
    "w200_ragged_empty": (3, 40, 8, 2, 128, [700, 0, 150], ("bounded", 6, 4), "bf16", 200),
    "w512_eight_splits": (1, 64, 10, 2, 128, [3000], ("bounded", 8, 3), "bf16", 512),
    "w130_d64": (2, 33, 8, 2, 64, [129, 1000], "uniform", "bf16", 130),
    "w100_fp32_d64": (2, 16, 6, 3, 64, [300, 50], "forest", "f32", 100),
    "w90_fp32_d128": (2, 24, 4, 2, 128, [500, 20], ("bounded", 6, 4), "f32", 90),
    "w_covers_all": (2, 32, 8, 2, 128, [100, 37], ("bounded", 6, 4), "bf16", 200),
    "w64_empty_cache": (1, 20, 4, 2, 128, [0], "uniform", "bf16", 64),
    # node depth up to 40 against a window 2 keys longer than the cache: rows
    # near the root see every cache key, deep rows lose the first ones
    "w_just_past_cache": (1, 40, 8, 2, 128, [300], "chain", "bf16", 302),
}


def _case(name):
    B, T, Hq, Hkv, D, lens, trees, dtype, window = SMALL[name]
    rng = np.random.default_rng(zlib.crc32(name.encode()))
    w = make_workload(rng, B=B, T=T, Hq=Hq, Hkv=Hkv, D=D, prefix_lens=lens, trees=trees,
                      dtype=dtype, name=name)
    return w, window


def _run(w, window):
    import tree_attention_amd as ta
    dev = "cuda"
    mask, _ = ta.build_mask(w.parent.to(dev))
    o, lse = ta.window_attn(w.q.to(dev), w.k_prefix.to(dev), w.v_prefix.to(dev),
                            w.offsets.to(dev), w.k_tree.to(dev), w.v_tree.to(dev), mask,
                            w.scale, window)
    torch.cuda.synchronize()
    return o.cpu().double().numpy(), lse.cpu().double().numpy()


def _reference(w, window, heads=None):
    """Oracle over all KV heads, or over the listed KV heads only (their query
    heads: a sub-problem of the same definition)."""
    off = w.offsets.numpy()
    if heads is None:
        return oracle.oracle_window_attn(w.q, w.k_prefix, w.v_prefix, off, w.k_tree, w.v_tree,
                                         w.parent.numpy(), w.scale, window)
    G = w.q.shape[2] // w.k_tree.shape[2]
    out = []
    for g in heads:
        hs = slice(g * G, (g + 1) * G)
        out.append((hs, oracle.oracle_window_attn(
            w.q[:, :, hs], w.k_prefix[:, g:g + 1], w.v_prefix[:, g:g + 1], off,
            w.k_tree[:, :, g:g + 1], w.v_tree[:, :, g:g + 1], w.parent.numpy(), w.scale,
            window)))
    return out


def _check(w, o, lse, o_ref, lse_ref):
    tol = BF16_O_TOL if w.dtype == "bf16" else F32_O_TOL
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
    eo = np.max(np.abs(o - o_ref))
    el = np.max(np.abs(lse - lse_ref))
    assert eo <= tol, f"o max-abs error {eo:.3e} > {tol}"
    assert el <= LSE_TOL, f"lse max-abs error {el:.3e} > {LSE_TOL}"


@pytest.mark.parametrize("name", sorted(SMALL))
def test_small_parity(name):
    w, window = _case(name)
    say("window attn small", name)
    o, lse = _run(w, window)
    o_ref, lse_ref = _reference(w, window)
    _check(w, o, lse, o_ref, lse_ref)


@pytest.mark.parametrize("window,lens", [(512, [2000, 400]), (20000, [20000, 400])])
def test_split_sizes(window, lens):
    """Splits of one tile (window 512: 511 keys over 128 splits per head,
    rounded up to 64) and of three tiles (window 20000: 19999 keys, 192-key
    splits), on a 256-CU device; the first split is the window's per-row
    masked head tile."""
    rng = np.random.default_rng(window)
    w = make_workload(rng, B=2, T=64, Hq=8, Hkv=2, D=128, prefix_lens=lens,
                      trees=("bounded", 8, 3), dtype="bf16", outlier_frac=0.01)
    say("window attn split", window)
    o, lse = _run(w, window)
    o_ref, lse_ref = _reference(w, window)
    _check(w, o, lse, o_ref, lse_ref)


def test_window_covering_everything_equals_tree_attention():
    """A window longer than cache plus tree: the same result as ltree_attn."""
    import tree_attention_amd as ta
    w, window = _case("w_covers_all")
    say("window attn vs tree attn")
    o, lse = _run(w, window)
    dev = "cuda"
    mask, _ = ta.build_mask(w.parent.to(dev))
    o2, lse2 = ta.attn(w.q.to(dev), w.k_prefix.to(dev), w.v_prefix.to(dev), w.offsets.to(dev),
                       max(w.prefix_lens), w.k_tree.to(dev), w.v_tree.to(dev), mask, w.scale)
    torch.cuda.synchronize()
    assert np.max(np.abs(o - o2.cpu().double().numpy())) <= BF16_O_TOL
    assert np.max(np.abs(lse - lse2.cpu().double().numpy())) <= LSE_TOL


def test_window_shorter_than_tree_is_rejected():
    """window < T is an argument error, reported before any launch."""
    import tree_attention_amd as ta
    rng = np.random.default_rng(3)
    w = make_workload(rng, B=1, T=16, Hq=4, Hkv=2, D=128, prefix_lens=[40], trees="chain",
                      dtype="bf16")
    dev = "cuda"
    assert ta.ltree_window_attn_workspace_bytes(1, 16, 4, 2, 128, 15) == 0
    mask, _ = ta.build_mask(w.parent.to(dev))
    o = torch.empty((1, 16, 4, 128), dtype=torch.float32, device=dev)
    lse = torch.empty((1, 4, 16), dtype=torch.float32, device=dev)
    ws = torch.empty((1 << 20,), dtype=torch.uint8, device=dev)
    say("window attn rejects window < T")
    st = ta.ltree_window_attn(w.q.to(dev), w.k_prefix.to(dev), w.v_prefix.to(dev),
                              w.offsets.to(dev), w.k_tree.to(dev), w.v_tree.to(dev), mask, o,
                              lse, ws, w.scale, 15)
    assert st == ta.LTREE_ERR_INVALID_ARG


@pytest.mark.parametrize("P,name", [(16, "w200_ragged_empty"), (64, "w512_eight_splits"),
                                    (48, "w90_fp32_d128"), (32, "w_just_past_cache")])
def test_window_over_paged_cache(P, name):
    """The draft cache in pages shuffled through a pool: the same result as
    the packed window call, and the oracle's on the gathered keys."""
    import tree_attention_amd as ta
    from test_gpu_paged import _paginate
    w, window = _case(name)
    rng = np.random.default_rng(P)
    kp, vp, bt, lens = _paginate(w, P, rng)
    dev = "cuda"
    B, T, Hq, D = w.q.shape
    Hkv = w.k_tree.shape[2]
    mask, _ = ta.build_mask(w.parent.to(dev))
    o = torch.empty((B, T, Hq, D), dtype=torch.float32, device=dev)
    lse = torch.empty((B, Hq, T), dtype=torch.float32, device=dev)
    ws = torch.empty((ta.ltree_window_attn_paged_workspace_bytes(B, T, Hq, Hkv, D, window, P),),
                     dtype=torch.uint8, device=dev)
    say("window attn paged", name, P)
    assert ta.ltree_window_attn_paged(w.q.to(dev), kp.to(dev), vp.to(dev), bt.to(dev),
                                      lens.to(dev), w.k_tree.to(dev), w.v_tree.to(dev), mask, o,
                                      lse, ws, w.scale, window) == 0
    torch.cuda.synchronize()
    o, lse = o.cpu().double().numpy(), lse.cpu().double().numpy()
    o2, lse2 = _run(w, window)
    assert np.max(np.abs(o - o2)) <= 1e-5 and np.max(np.abs(lse - lse2)) <= 1e-5
    kg, off = oracle.gather_paged(kp.float().numpy(), bt.numpy(), lens.numpy(), P)
    vg, _ = oracle.gather_paged(vp.float().numpy(), bt.numpy(), lens.numpy(), P)
    o_ref, lse_ref = oracle.oracle_window_attn(w.q, kg, vg, off, w.k_tree, w.v_tree,
                                               w.parent.numpy(), w.scale, window)
    _check(w, o, lse, o_ref, lse_ref)


def test_window_paged_sequence_past_block_table_gives_nan():
    """A sequence with more keys than its block-table row reaches (L_b above
    max_pages_per_seq * page_size) gets NaN rows and none of its pages is
    looked up; the other sequences stay exact.  The last sequence is the one
    past its row, so a lookup would have gone past the end of the table."""
    import tree_attention_amd as ta
    from test_gpu_paged import _paginate
    w, window = _case("w200_ragged_empty")            # lens [700, 0, 150], window 200
    P = 16
    rng = np.random.default_rng(5)
    kp, vp, bt, lens = _paginate(w, P, rng)
    reach = bt.shape[1] * P                           # 44 pages of 16 keys: 704
    lens_bad = lens.clone()
    lens_bad[2] = reach + 1
    dev = "cuda"
    B, T, Hq, D = w.q.shape
    Hkv = w.k_tree.shape[2]
    mask, _ = ta.build_mask(w.parent.to(dev))
    o = torch.empty((B, T, Hq, D), dtype=torch.float32, device=dev)
    lse = torch.empty((B, Hq, T), dtype=torch.float32, device=dev)
    ws = torch.empty((ta.ltree_window_attn_paged_workspace_bytes(B, T, Hq, Hkv, D, window, P),),
                     dtype=torch.uint8, device=dev)
    say("window paged past the block table")
    assert ta.ltree_window_attn_paged(w.q.to(dev), kp.to(dev), vp.to(dev), bt.to(dev),
                                      lens_bad.to(dev), w.k_tree.to(dev), w.v_tree.to(dev), mask,
                                      o, lse, ws, w.scale, window) == 0
    torch.cuda.synchronize()
    o, lse = o.cpu().double().numpy(), lse.cpu().double().numpy()
    assert np.all(np.isnan(o[2])) and np.all(np.isnan(lse[2]))
    kg, off = oracle.gather_paged(kp.float().numpy(), bt.numpy(), lens.numpy(), P)
    vg, _ = oracle.gather_paged(vp.float().numpy(), bt.numpy(), lens.numpy(), P)
    o_ref, lse_ref = oracle.oracle_window_attn(w.q, kg, vg, off, w.k_tree, w.v_tree,
                                               w.parent.numpy(), w.scale, window)
    assert np.max(np.abs(o[:2] - o_ref[:2])) <= BF16_O_TOL
    assert np.max(np.abs(lse[:2] - lse_ref[:2])) <= LSE_TOL
