"""Trees of more than 64 nodes (W = ceil(T/64) mask words per row) on the GPU,
through the C ABI, against the fp64 oracle: the mask bit-exact, attention
within the stated tolerances (several tree tiles per sequence, several row
blocks per KV head), RoPE within one unit in the last place, the commit
bit-exact, window attention within the tolerances."""

import zlib

import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import LSE_TOL, check_parity, oracle_full, run_library, say
from workloads import make_tree, make_workload

pytestmark = pytest.mark.gpu


def _mask(parent_np):
    import tree_attention_amd as ta
    p = torch.from_numpy(np.ascontiguousarray(parent_np, dtype=np.int32)).cuda()
    mask, status = ta.build_mask(p)
    torch.cuda.synchronize()
    B, T = parent_np.shape
    return mask.cpu().numpy().view(np.uint64).reshape(B, T, -1), int(status.cpu()[0])


@pytest.mark.parametrize("T", [65, 100, 128, 129, 200, 255, 256])
def test_mask_wide_trees(T):
    rng = np.random.default_rng(T)
    kinds = ["chain", "star", "uniform", "forest", ("bounded", 12, 3)]
    parent = np.stack([make_tree(rng, T, kinds[b % len(kinds)]) for b in range(9)])
    say("mask wide T", T)
    got, st = _mask(parent)
    assert st == 0
    assert np.array_equal(got, oracle.oracle_mask(parent))


def test_mask_wide_invalid_parents():
    rng = np.random.default_rng(1)
    parent = np.stack([make_tree(rng, 150, "uniform") for _ in range(4)])
    parent[2, 140] = 140   # self-parent
    parent[3, 70] = 99     # a later node
    say("mask wide invalid parents")
    got, st = _mask(parent)
    assert st == 1 + 2 * 150 + 140
    assert np.array_equal(got[:2], oracle.oracle_mask(parent[:2]))
    assert not got[2:].any()


SMALL = {
    # name: (B, T, Hq, Hkv, D, prefix_lens, trees, dtype)
    "t100_g4": (2, 100, 8, 2, 128, [700, 0], ("bounded", 12, 4), "bf16"),
    "t65_d64": (2, 65, 6, 3, 64, [129, 64], ("bounded", 10, 3), "bf16"),
    "t200_chain_g5": (1, 200, 10, 2, 128, [400], "chain", "bf16"),
    "t256_mha_d64": (1, 256, 4, 4, 64, [300], "uniform", "bf16"),
    "t130_fp32_forest": (2, 130, 4, 2, 128, [200, 31], "forest", "f32"),
    "t96_fp32_d64": (1, 96, 6, 2, 64, [70], ("bounded", 20, 2), "f32"),
}


def _small(name):
    B, T, Hq, Hkv, D, lens, trees, dtype = SMALL[name]
    rng = np.random.default_rng(zlib.crc32(name.encode()))
    return make_workload(rng, B=B, T=T, Hq=Hq, Hkv=Hkv, D=D, prefix_lens=lens, trees=trees,
                         dtype=dtype, name=name)


@pytest.mark.parametrize("name", sorted(SMALL))
def test_attention_parity(name):
    w = _small(name)
    say("big tree parity", name, w.shape)
    o, lse, mask, status = run_library(w)
    assert int(status[0]) == 0
    check_parity(w, o, lse, *oracle_full(w))


def test_rope_wide_tree():
    import tree_attention_amd as ta
    rng = np.random.default_rng(11)
    w = make_workload(rng, B=2, T=180, Hq=8, Hkv=2, D=128, prefix_lens=[1000, 5],
                      trees=("bounded", 30, 3), dtype="bf16")
    dev = "cuda"
    q, kt = w.q.to(dev).clone(), w.k_tree.to(dev).clone()
    mask, _ = ta.build_mask(w.parent.to(dev))
    say("rope wide tree")
    assert ta.ltree_tree_rope(q, kt, mask, w.offsets.to(dev), 1e6) == 0
    torch.cuda.synchronize()
    rq, rk = oracle.oracle_tree_rope(w.q, w.k_tree, w.parent.numpy(), w.offsets.numpy(), 1e6)
    for got, ref in ((q, rq), (kt, rk)):
        got = got.cpu().double().numpy()
        ref_r = oracle.round_bf16(ref)
        ulp = np.ldexp(1.0, np.frexp(np.abs(ref_r))[1] - 8)
        diff = np.abs(got - ref_r)
        assert np.all(diff <= ulp)
        assert np.mean(diff == 0) >= 0.999


def test_commit_wide_tree():
    import tree_attention_amd as ta
    rng = np.random.default_rng(12)
    B, T, Hkv, D, rows = 2, 200, 2, 128, 600
    parent = make_tree(rng, T, "chain")
    kt = torch.randn(B, T, Hkv, D).to(torch.bfloat16)
    vt = torch.randn(B, T, Hkv, D).to(torch.bfloat16)
    kc = torch.randn(rows, Hkv, D).to(torch.bfloat16)
    vc = torch.randn(rows, Hkv, D).to(torch.bfloat16)
    acc = torch.zeros(B, T, dtype=torch.int32)
    acc[0, :150] = torch.arange(150, dtype=torch.int32)        # a 150-token branch of the chain
    acc[1, :3] = torch.tensor([0, 1, 2], dtype=torch.int32)
    n_acc = torch.tensor([150, 3], dtype=torch.int32)
    dst = torch.tensor([100, 400], dtype=torch.int32)
    assert int(parent[149]) == 148
    dev = "cuda"
    kc_d, vc_d = kc.to(dev), vc.to(dev)
    status = torch.full((1,), -7, dtype=torch.int32, device=dev)
    say("commit wide tree")
    assert ta.ltree_commit_kv(kt.to(dev), vt.to(dev), acc.to(dev), n_acc.to(dev), dst.to(dev),
                              kc_d, vc_d, status) == 0
    torch.cuda.synchronize()
    as16 = lambda t: t.view(torch.int16).numpy()  # noqa: E731
    rk, rv, rst = oracle.oracle_commit_kv(as16(kt), as16(vt), acc.numpy(), n_acc.numpy(),
                                          dst.numpy(), as16(kc), as16(vc))
    assert int(status.cpu()[0]) == rst == 0
    assert np.array_equal(as16(kc_d.cpu()), rk) and np.array_equal(as16(vc_d.cpu()), rv)


@pytest.mark.parametrize("name,B,T,lens,trees,dtype,window", [
    ("w512_chain80_short_cache", 1, 80, [100], "chain", "bf16", 512),
    # chains of 200 / 130 nodes after long caches: the deepest rows hide 199 /
    # 129 cache keys, across four / three 64-key splits
    ("w256_chain200", 2, 200, [3000, 150], "chain", "bf16", 256),
    ("w300_fp32_chain130", 2, 130, [500, 0], "chain", "f32", 300),
    ("w256_t200_bounded", 1, 200, [1000], ("bounded", 40, 3), "bf16", 256),
])
def test_window_wide_tree(name, B, T, lens, trees, dtype, window):
    """Window attention over trees above 64 nodes: rows hide up to depth - 1
    cache keys, spread over several 64-key splits."""
    import tree_attention_amd as ta
    rng = np.random.default_rng(zlib.crc32(name.encode()))
    w = make_workload(rng, B=B, T=T, Hq=8, Hkv=2, D=128, prefix_lens=lens, trees=trees,
                      dtype=dtype, name=name)
    dev = "cuda"
    mask, _ = ta.build_mask(w.parent.to(dev))
    say("window wide tree", name)
    o, lse = ta.window_attn(w.q.to(dev), w.k_prefix.to(dev), w.v_prefix.to(dev),
                            w.offsets.to(dev), w.k_tree.to(dev), w.v_tree.to(dev), mask,
                            w.scale, window)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.oracle_window_attn(w.q, w.k_prefix, w.v_prefix, w.offsets.numpy(),
                                               w.k_tree, w.v_tree, w.parent.numpy(), w.scale,
                                               window)
    tol = 2e-2 if dtype == "bf16" else 1e-4
    assert np.max(np.abs(o.cpu().double().numpy() - o_ref)) <= tol
    assert np.max(np.abs(lse.cpu().double().numpy() - lse_ref)) <= LSE_TOL


def test_mask_wide_many_trees_invalid():
    """40 wide trees, one workgroup each; status from the spread build."""
    rng = np.random.default_rng(8)
    parent = np.stack([make_tree(rng, 200, ("bounded", 12, 3)) for _ in range(40)])
    parent[33, 150] = 180
    parent[21, 199] = -5
    say("mask wide 40 trees, invalid entries")
    got, st = _mask(parent)
    assert st == 1 + 21 * 200 + 199
    ok = [b for b in range(40) if b not in (21, 33)]
    assert np.array_equal(got[ok], oracle.oracle_mask(parent[ok]))
    assert not got[[21, 33]].any()
