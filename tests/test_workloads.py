"""The seeded input generator follows its recipe (CPU only)."""

import numpy as np
import pytest
import torch

from workloads import CONFIGS, make_config, make_tree, make_workload


def _depths(parent):
    d = []
    for i, p in enumerate(parent):
        d.append(1 if p < 0 else d[p] + 1)
    return np.array(d)


@pytest.mark.parametrize("kind,dmax,bmax", [(("bounded", 6, 4), 6, 4), (("bounded", 8, 3), 8, 3)])
def test_bounded_trees_respect_bounds(kind, dmax, bmax):
    rng = np.random.default_rng(0)
    for _ in range(50):
        p = make_tree(rng, 64, kind)
        assert p[0] == -1 and all(0 <= p[i] < i for i in range(1, 64))
        assert _depths(p).max() <= dmax
        assert np.bincount(p[1:], minlength=64).max() <= bmax


def test_tree_kinds():
    rng = np.random.default_rng(1)
    assert make_tree(rng, 5, "chain").tolist() == [-1, 0, 1, 2, 3]
    assert make_tree(rng, 4, "star").tolist() == [-1, 0, 0, 0]
    u = make_tree(rng, 30, "uniform")
    assert u[0] == -1 and all(0 <= u[i] < i for i in range(1, 30))
    f = make_tree(rng, 30, "forest")
    assert all(-1 <= f[i] < i for i in range(30))


def test_seeded_and_reproducible():
    a, b = make_config(1), make_config(1)
    assert torch.equal(a.q, b.q) and torch.equal(a.parent, b.parent)
    assert a.dtype == "f32" and a.q.dtype == torch.float32
    assert a.scale == 1.0 / 8.0 and a.q.shape == (1, 8, 4, 64)
    assert a.parent[0, 0] == -1


def test_outlier_rows_and_bf16_rounding():
    # A small stand-in for the QwQ-shaped workload's recipe: 1% of prefix rows x8.
    rng = np.random.default_rng(5)
    w = make_workload(rng, B=1, T=4, Hq=2, Hkv=1, D=8, prefix_lens=[1000],
                      trees="chain", dtype="bf16", outlier_frac=0.01)
    assert w.q.dtype == torch.bfloat16
    big = (w.k_prefix.float().abs().amax(dim=(1, 2)) > 0).sum()
    assert big == 1000
    # replay the draws in the recipe's order to find the outlier rows
    rng = np.random.default_rng(5)
    make_tree(rng, 4, "chain")
    rng.standard_normal((1, 4, 2, 8), dtype=np.float32)          # q
    kp = rng.standard_normal((1000, 1, 8), dtype=np.float32)     # k_prefix
    for shape in [(1000, 1, 8), (1, 4, 1, 8), (1, 4, 1, 8)]:      # v_prefix, k_tree, v_tree
        rng.standard_normal(shape, dtype=np.float32)
    rows = rng.choice(1000, size=10, replace=False)
    ref = torch.from_numpy(kp.copy())
    ref[rows] *= 8
    assert torch.equal(w.k_prefix, ref.to(torch.bfloat16))


def test_config_table_shapes():
    assert CONFIGS[4]["Hq"] == 40 and CONFIGS[4]["prefix_lens"] == [32768]
    assert CONFIGS[4]["outlier_frac"] == 0.01
    assert CONFIGS[5]["prefix_lens"] == [8192, 32768, 65536, 131072]
    assert CONFIGS[5]["trees"][0] == "chain"
