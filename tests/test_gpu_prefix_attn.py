"""Prefix-only attention (the draft model's cross-attention into the target's
KV cache) on the GPU, through the C ABI, against the fp64 oracle.

Small cases cover several key tiles and splits, ragged tails, an empty prefix
(o = 0, lse = -inf), D = 64 and 128, bf16 and fp32.  The QwQ-shaped layer
(prefix 32768, 64 query tokens) is checked on every row in
test_gpu_full_sizes.py."""

import zlib

import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import BF16_O_TOL, F32_O_TOL, LSE_TOL, say
from workloads import make_workload

pytestmark = pytest.mark.gpu

SMALL = {
    # name: (B, T, Hq, Hkv, D, prefix_lens, dtype)
    "g5_t64_bf16": (1, 64, 10, 2, 128, [1000], "bf16"),
    "ragged_with_empty": (3, 16, 8, 2, 128, [700, 0, 131], "bf16"),
    "t1_decode_d64": (2, 1, 8, 2, 64, [257, 64], "bf16"),
    "fp32_d128": (2, 8, 4, 2, 128, [300, 77], "f32"),
    "fp32_d64_empty": (2, 5, 6, 3, 64, [0, 40], "f32"),
    # every prefix empty: one empty partial per sequence, o = 0 and lse = -inf everywhere
    "all_empty_b5": (5, 8, 4, 2, 128, [0, 0, 0, 0, 0], "bf16"),
}


def _case(name):
    B, T, Hq, Hkv, D, lens, dtype = SMALL[name]
    rng = np.random.default_rng(zlib.crc32(name.encode()))
    return make_workload(rng, B=B, T=T, Hq=Hq, Hkv=Hkv, D=D, prefix_lens=lens, trees="chain",
                         dtype=dtype, name=name)


def _run(w, max_len=None):
    import tree_attention_amd as ta
    dev = "cuda"
    o, lse = ta.prefix_attn(w.q.to(dev), w.k_prefix.to(dev), w.v_prefix.to(dev),
                            w.offsets.to(dev), max(w.prefix_lens) if max_len is None else max_len,
                            w.scale)
    torch.cuda.synchronize()
    return o.cpu().double().numpy(), lse.cpu().double().numpy()


def _check(w, o, lse, o_ref, lse_ref):
    tol = BF16_O_TOL if w.dtype == "bf16" else F32_O_TOL
    empty = np.isneginf(lse_ref)
    # rows of an empty prefix: exactly o = 0 and lse = -inf
    assert np.array_equal(np.isneginf(lse), empty)
    assert np.all(o[np.transpose(empty, (0, 2, 1))] == 0)
    assert np.all(np.isfinite(o))
    eo = np.max(np.abs(o - o_ref))
    el = np.max(np.abs(lse[~empty] - lse_ref[~empty]), initial=0.0)
    assert eo <= tol, f"o max-abs error {eo:.3e} > {tol}"
    assert el <= LSE_TOL, f"lse max-abs error {el:.3e} > {LSE_TOL}"


@pytest.mark.parametrize("name", sorted(SMALL))
def test_small_parity(name):
    w = _case(name)
    say("prefix attn small", name)
    o, lse = _run(w)
    o_ref, lse_ref = oracle.oracle_prefix_attn(w.q, w.k_prefix, w.v_prefix, w.offsets.numpy(),
                                               w.scale)
    _check(w, o, lse, o_ref, lse_ref)


def test_many_splits():
    """One KV head over 20224 keys: 79 splits of 256 keys on a 256-CU device,
    more partials per row than a wavefront has lanes."""
    rng = np.random.default_rng(5)
    w = make_workload(rng, B=1, T=16, Hq=8, Hkv=1, D=128, prefix_lens=[20224], trees="chain",
                      dtype="bf16", outlier_frac=0.01)
    say("prefix attn many splits")
    o, lse = _run(w)
    o_ref, lse_ref = oracle.oracle_prefix_attn(w.q, w.k_prefix, w.v_prefix, w.offsets.numpy(),
                                               w.scale)
    _check(w, o, lse, o_ref, lse_ref)


def test_prefix_attn_equals_tree_attn_prefix_part():
    """The prefix part of tree-verification attention: merging the prefix-only
    result with the tree-only oracle partial (log-sum-exp) gives ltree_attn's
    result."""
    import tree_attention_amd as ta
    rng = np.random.default_rng(6)
    w = make_workload(rng, B=2, T=32, Hq=8, Hkv=2, D=128, prefix_lens=[600, 350],
                      trees=("bounded", 6, 4), dtype="bf16")
    say("prefix attn vs tree attn")
    o_p, lse_p = _run(w)
    (_, _), (o_t, lse_t), _ = oracle.oracle_attn_split(
        w.q, w.k_prefix, w.v_prefix, w.offsets.numpy(), w.k_tree, w.v_tree, w.parent.numpy(),
        w.scale)
    o_m, lse_m = oracle.lse_merge([(np.transpose(o_p, (0, 2, 1, 3)), lse_p),
                                   (np.transpose(o_t, (0, 2, 1, 3)), lse_t)])
    dev = "cuda"
    mask, _ = ta.build_mask(w.parent.to(dev))
    o, lse = ta.attn(w.q.to(dev), w.k_prefix.to(dev), w.v_prefix.to(dev), w.offsets.to(dev),
                     600, w.k_tree.to(dev), w.v_tree.to(dev), mask, w.scale)
    torch.cuda.synchronize()
    assert np.max(np.abs(o.cpu().double().numpy() - np.transpose(o_m, (0, 2, 1, 3)))) <= BF16_O_TOL
    assert np.max(np.abs(lse.cpu().double().numpy() - lse_m)) <= LSE_TOL
