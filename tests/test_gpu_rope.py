"""Rotary position embedding at tree positions on the GPU, through the C ABI,
against the fp64 oracle: every output within one unit in the last place of
the storage type of the oracle's correctly rounded value (the angle is an
fp64 product on both sides, whose last-bit differences can move a value
across a rounding boundary), and nearly all of them identical."""

import zlib

import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import say
from workloads import make_config, make_workload

pytestmark = pytest.mark.gpu


def _run(w, base):
    import tree_attention_amd as ta
    dev = "cuda"
    q, kt = w.q.to(dev).clone(), w.k_tree.to(dev).clone()
    mask, _ = ta.build_mask(w.parent.to(dev))
    assert ta.ltree_tree_rope(q, kt, mask, w.offsets.to(dev), base) == 0
    torch.cuda.synchronize()
    return q.cpu().double().numpy(), kt.cpu().double().numpy()


def _check(w, got, ref):
    if w.dtype == "bf16":
        ref_r = oracle.round_bf16(ref)
        ulp = np.ldexp(1.0, np.frexp(np.abs(ref_r))[1] - 8)
    else:
        ref_r = ref.astype(np.float32).astype(np.float64)
        ulp = np.ldexp(1.0, np.frexp(np.abs(ref_r))[1] - 24)
    diff = np.abs(got - ref_r)
    assert np.all(diff <= ulp), f"max {np.max(diff / ulp):.2f} ulp"
    assert np.mean(diff == 0) >= 0.999


@pytest.mark.parametrize("name,dtype,D,lens,trees,base", [
    ("bf16_d128_bounded", "bf16", 128, [700, 0, 33], ("bounded", 6, 4), 1e6),
    ("bf16_d64_chain", "bf16", 64, [131072], "chain", 5e5),
    ("f32_d128_forest", "f32", 128, [9, 300], "forest", 1e4),
])
def test_tree_rope(name, dtype, D, lens, trees, base):
    rng = np.random.default_rng(zlib.crc32(name.encode()))
    w = make_workload(rng, B=len(lens), T=40, Hq=8, Hkv=2, D=D, prefix_lens=lens, trees=trees,
                      dtype=dtype, name=name)
    say("tree rope", name)
    q, kt = _run(w, base)
    rq, rk = oracle.oracle_tree_rope(w.q, w.k_tree, w.parent.numpy(), w.offsets.numpy(), base)
    _check(w, q, rq)
    _check(w, kt, rk)


@pytest.mark.parametrize("name,B,T,Hq,Hkv,D", [
    # 50 tokens, 12 passes of 4 heads: 5 workgroups per token, the last with no pass
    ("uneven_split", 1, 50, 40, 8, 128),
    # 9 * 64 tokens, more than the compute units: one workgroup per token
    ("many_tokens", 9, 64, 12, 4, 128),
    # 18 passes of 8 heads (D 64) in one workgroup: two batches of loads
    ("many_heads", 3, 100, 136, 8, 64),
])
def test_tree_rope_work_split(name, B, T, Hq, Hkv, D):
    """The token's head passes shared by several workgroups, by one, or in
    more than one batch of loads."""
    rng = np.random.default_rng(zlib.crc32(name.encode()))
    lens = [int(x) for x in rng.integers(0, 5000, size=B)]
    w = make_workload(rng, B=B, T=T, Hq=Hq, Hkv=Hkv, D=D, prefix_lens=lens, trees=("bounded", 9, 3),
                      dtype="bf16", name=name)
    say("tree rope work split", name)
    q, kt = _run(w, 1e6)
    rq, rk = oracle.oracle_tree_rope(w.q, w.k_tree, w.parent.numpy(), w.offsets.numpy(), 1e6)
    _check(w, q, rq)
    _check(w, kt, rk)


def test_tree_rope_qwq_shape():
    """The QwQ-shaped tree after the 32768-key prefix, rotary base 10^6."""
    w = make_config(4)
    say("tree rope qwq shape")
    q, kt = _run(w, 1e6)
    rq, rk = oracle.oracle_tree_rope(w.q, w.k_tree, w.parent.numpy(), w.offsets.numpy(), 1e6)
    _check(w, q, rq)
    _check(w, kt, rk)


def test_invalid_tree_rows_untouched():
    """A tree with an invalid parent has zero mask rows: its tokens stay as
    they were."""
    import tree_attention_amd as ta
    rng = np.random.default_rng(9)
    w = make_workload(rng, B=2, T=8, Hq=4, Hkv=2, D=128, prefix_lens=[10, 20], trees="uniform",
                      dtype="bf16")
    dev = "cuda"
    parent = w.parent.clone()
    parent[1, 5] = 6                 # not an earlier node
    mask, status = ta.build_mask(parent.to(dev))
    q = w.q.to(dev).clone()
    kt = w.k_tree.to(dev).clone()
    say("tree rope invalid tree")
    assert ta.ltree_tree_rope(q, kt, mask, w.offsets.to(dev), 1e4) == 0
    torch.cuda.synchronize()
    assert int(status.cpu()[0]) == 1 + 8 + 5
    assert torch.equal(q[1].cpu(), w.q[1]) and torch.equal(kt[1].cpu(), w.k_tree[1])
    assert not torch.equal(q[0].cpu(), w.q[0])
