"""Steps a2-a4 on the GPU, through the C ABI, against the fp64 oracle.

Small cases (the oracle finishes in seconds) cover several key tiles, ragged
split tails, every row-tile count of the MFMA kernel, D = 64 and 128, bf16
and fp32, empty prefixes, forests, single-node trees and a merge over more
partials than a wavefront has lanes.  Every output element at the full
workload sizes is checked in test_gpu_full_sizes.py."""

import zlib

import numpy as np
import pytest
import torch

from gpu_helpers import (LSE_TOL, check_parity, oracle_full, run_library, say, to_device)
from workloads import make_config, make_workload

pytestmark = pytest.mark.gpu

SMALL = {
    # name: (B, T, Hq, Hkv, D, prefix_lens, trees, dtype)
    "g5_t64_320rows": (1, 64, 10, 2, 128, [1000], ("bounded", 8, 3), "bf16"),
    "g4_t64_256rows_ragged": (2, 64, 8, 2, 128, [700, 0], ("bounded", 6, 4), "bf16"),
    "g2_t8_d64": (2, 8, 4, 2, 64, [129, 64], "uniform", "bf16"),
    "g8_t64_two_row_blocks": (1, 64, 8, 1, 128, [300], ("bounded", 6, 4), "bf16"),
    "single_node": (2, 1, 8, 2, 128, [257, 3], "chain", "bf16"),
    "forest_b3": (3, 20, 6, 3, 128, [65, 0, 191], "forest", "bf16"),
    "mha_g1_t33_d64": (1, 33, 4, 4, 64, [450], ("bounded", 5, 3), "bf16"),
    "g3_t48_tpw3": (1, 48, 12, 4, 128, [515], ("bounded", 6, 4), "bf16"),
    "g4_t32_tpw2_chain": (2, 32, 8, 2, 128, [900, 1300], "chain", "bf16"),
    "fp32_d128": (2, 16, 8, 2, 128, [300, 77], "uniform", "f32"),
    "fp32_d64_forest": (1, 9, 6, 2, 64, [40], "forest", "f32"),
    "no_prefix_at_all": (2, 12, 4, 2, 128, [0, 0], "uniform", "bf16"),
    # trees of 33-64 nodes after full and short last splits (256-key splits)
    "tree_split_t40_b3": (3, 40, 8, 2, 128, [512, 500, 300], ("bounded", 6, 4), "bf16"),
    "tree_split_t64_full": (1, 64, 10, 2, 128, [768], ("bounded", 8, 3), "bf16"),
}


def _small(name, seed=0):
    B, T, Hq, Hkv, D, lens, trees, dtype = SMALL[name]
    rng = np.random.default_rng(zlib.crc32(name.encode()) + seed)
    return make_workload(rng, B=B, T=T, Hq=Hq, Hkv=Hkv, D=D, prefix_lens=lens, trees=trees,
                         dtype=dtype, name=name)


@pytest.mark.parametrize("name", sorted(SMALL))
def test_small_parity(name):
    w = _small(name)
    say("small parity", name, w.shape)
    o, lse, mask, status = run_library(w)
    assert int(status[0]) == 0
    o_ref, lse_ref = oracle_full(w)
    check_parity(w, o, lse, o_ref, lse_ref)


def test_tiny_fp32_config():
    w = make_config(1)
    say("config 1 full parity")
    o, lse, _, _ = run_library(w)
    check_parity(w, o, lse, *oracle_full(w))


def test_many_splits_merge():
    """One KV head over 20224 keys: 79 prefix splits of 256 keys on a
    256-CU device (one per compute unit, each at least 256 keys), so the
    merge takes more partials per row than a wavefront has lanes."""
    rng = np.random.default_rng(3)
    w = make_workload(rng, B=1, T=16, Hq=8, Hkv=1, D=128, prefix_lens=[20224],
                      trees=("bounded", 4, 3), dtype="bf16")
    say("many splits")
    o, lse, _, _ = run_library(w)
    check_parity(w, o, lse, *oracle_full(w))


def test_outlier_rows_small():
    """The 1%-outlier recipe at a small size: softmax range stress."""
    rng = np.random.default_rng(4)
    w = make_workload(rng, B=1, T=64, Hq=10, Hkv=2, D=128, prefix_lens=[3000],
                      trees=("bounded", 8, 3), dtype="bf16", outlier_frac=0.01)
    say("outliers small")
    o, lse, _, _ = run_library(w)
    check_parity(w, o, lse, *oracle_full(w))


def test_grid_larger_than_lengths():
    """max_prefix_len above every L_b: the extra splits are empty."""
    import tree_attention_amd as ta
    w = _small("g4_t64_256rows_ragged")
    d = to_device(w)
    mask, _ = ta.build_mask(d["parent"])
    say("oversized max_prefix_len")
    o, lse = ta.attn(d["q"], d["k_prefix"], d["v_prefix"], d["offsets"], 9000, d["k_tree"],
                     d["v_tree"], mask, w.scale)
    torch.cuda.synchronize()
    check_parity(w, o.cpu(), lse.cpu(), *oracle_full(w))


def test_deterministic():
    import tree_attention_amd as ta
    w = _small("g5_t64_320rows")
    d = to_device(w)
    mask, _ = ta.build_mask(d["parent"])
    say("determinism")
    runs = [ta.attn(d["q"], d["k_prefix"], d["v_prefix"], d["offsets"], 1000, d["k_tree"],
                    d["v_tree"], mask, w.scale) for _ in range(3)]
    torch.cuda.synchronize()
    for o, lse in runs[1:]:
        assert torch.equal(o, runs[0][0]) and torch.equal(lse, runs[0][1])


def test_partials_then_merge_equals_attn():
    import tree_attention_amd as ta
    w = _small("forest_b3")
    d = to_device(w)
    mask, _ = ta.build_mask(d["parent"])
    B, T, Hq, D = w.q.shape
    Hkv = w.k_tree.shape[2]
    ws = ta.workspace_for(d["q"], d["k_tree"], 191)
    o = torch.empty((B, T, Hq, D), dtype=torch.float32, device="cuda")
    lse = torch.empty((B, Hq, T), dtype=torch.float32, device="cuda")
    say("partials + merge")
    assert ta.ltree_attn_partials(d["q"], d["k_prefix"], d["v_prefix"], d["offsets"], 191,
                                  d["k_tree"], d["v_tree"], mask, ws, w.scale) == 0
    assert ta.ltree_attn_merge(d["q"].dtype, B, T, Hq, Hkv, D, d["offsets"], 191, o, lse, ws) == 0
    o2, lse2 = ta.attn(d["q"], d["k_prefix"], d["v_prefix"], d["offsets"], 191, d["k_tree"],
                       d["v_tree"], mask, w.scale)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(lse, lse2)


def test_prefix_length_over_max_gives_nan():
    import tree_attention_amd as ta
    w = _small("forest_b3")
    d = to_device(w)
    mask, _ = ta.build_mask(d["parent"])
    say("L_b over max_prefix_len")
    # sequence 2 has L = 191 > 150: its rows become NaN, the others stay exact
    o, lse = ta.attn(d["q"], d["k_prefix"], d["v_prefix"], d["offsets"], 150, d["k_tree"],
                     d["v_tree"], mask, w.scale)
    torch.cuda.synchronize()
    o, lse = o.cpu(), lse.cpu()
    assert torch.isnan(o[2]).all() and torch.isnan(lse[2]).all()
    o_ref, lse_ref = oracle_full(w)
    assert np.max(np.abs(o[:2].double().numpy() - o_ref[:2])) <= 2e-2
    assert np.max(np.abs(lse[:2].double().numpy() - lse_ref[:2])) <= LSE_TOL


@pytest.mark.parametrize("B", [256, 300])
def test_large_ragged_batch(B):
    """Many sequences of mixed lengths, every seventh empty and one longer than
    max_prefix_len.  Batches of up to 256 sequences hand out their
    (sequence, split) pairs in dispatch order, larger ones map workgroups to
    them directly: either way every sequence gets exactly its own splits, the
    long one NaN rows and the others the oracle's result."""
    import tree_attention_amd as ta
    rng = np.random.default_rng(B)
    lens = rng.integers(1, 700, size=B)
    lens[::7] = 0
    bad = B // 2 + 1
    lens[bad] = 900
    w = make_workload(rng, B=B, T=6, Hq=4, Hkv=2, D=128, prefix_lens=lens.tolist(), trees="uniform",
                      dtype="bf16")
    d = to_device(w)
    mask, _ = ta.build_mask(d["parent"])
    say("large ragged batch", B)
    o, lse = ta.attn(d["q"], d["k_prefix"], d["v_prefix"], d["offsets"], 800, d["k_tree"],
                     d["v_tree"], mask, w.scale)
    torch.cuda.synchronize()
    o, lse = o.cpu().double().numpy(), lse.cpu().double().numpy()
    assert np.isnan(o[bad]).all() and np.isnan(lse[bad]).all()
    keep = np.arange(B) != bad
    o_ref, lse_ref = oracle_full(w)
    assert np.all(np.isfinite(o[keep])) and np.all(np.isfinite(lse[keep]))
    assert np.max(np.abs(o[keep] - o_ref[keep])) <= 2e-2
    assert np.max(np.abs(lse[keep] - lse_ref[keep])) <= LSE_TOL


def test_every_prefix_over_max_gives_nan():
    """Every sequence longer than max_prefix_len: no split exists, every
    workgroup of the partial kernel finds none and returns, and every row is
    NaN."""
    import tree_attention_amd as ta
    w = _small("tree_split_t40_b3")
    d = to_device(w)
    mask, _ = ta.build_mask(d["parent"])
    say("every L_b over max_prefix_len")
    o, lse = ta.attn(d["q"], d["k_prefix"], d["v_prefix"], d["offsets"], 200, d["k_tree"],
                     d["v_tree"], mask, w.scale)
    torch.cuda.synchronize()
    assert torch.isnan(o.cpu()).all() and torch.isnan(lse.cpu()).all()


def test_error_paths_with_real_tensors():
    import tree_attention_amd as ta
    w = _small("g2_t8_d64")
    d = to_device(w)
    mask, _ = ta.build_mask(d["parent"])
    B, T, Hq, D = w.q.shape
    o = torch.empty((B, T, Hq, D), dtype=torch.float32, device="cuda")
    lse = torch.empty((B, Hq, T), dtype=torch.float32, device="cuda")
    small_ws = torch.empty((256,), dtype=torch.uint8, device="cuda")
    st = ta.ltree_attn(d["q"], d["k_prefix"], d["v_prefix"], d["offsets"], 129, d["k_tree"],
                       d["v_tree"], mask, o, lse, small_ws, w.scale)
    assert st == ta.LTREE_ERR_WORKSPACE
    ws = ta.workspace_for(d["q"], d["k_tree"], 129)
    assert ta.ltree_attn(d["q"], d["k_prefix"], d["v_prefix"], d["offsets"], 129, d["k_tree"],
                         d["v_tree"], mask, o, lse, ws, -1.0) == ta.LTREE_ERR_INVALID_ARG
    with pytest.raises(ta.LTreeError):
        ta.build_mask(torch.zeros((2, 257), dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
