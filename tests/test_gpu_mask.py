"""Step a1 on the GPU: the ancestor bitmask is bit-exact against the oracle."""

import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import mask_words, say
from workloads import CONFIGS, make_tree

pytestmark = pytest.mark.gpu


def _build(parent_np):
    import tree_attention_amd as ta
    p = torch.from_numpy(np.ascontiguousarray(parent_np, dtype=np.int32)).cuda()
    mask, status = ta.build_mask(p)
    torch.cuda.synchronize()
    return mask_words(mask.cpu()), int(status.cpu()[0])


@pytest.mark.parametrize("k", sorted(CONFIGS))
def test_mask_configs(k):
    spec = CONFIGS[k]
    rng = np.random.default_rng(1000 + k)
    trees = spec["trees"] if isinstance(spec["trees"], list) else [spec["trees"]] * spec["B"]
    parent = np.stack([make_tree(rng, spec["T"], t) for t in trees])
    say("mask config", k)
    got, st = _build(parent)
    assert st == 0
    assert np.array_equal(got, oracle.oracle_mask(parent)[:, :, 0])


@pytest.mark.parametrize("T", [1, 2, 3, 7, 31, 32, 33, 63, 64])
def test_mask_random_trees(T):
    rng = np.random.default_rng(T)
    kinds = ["chain", "star", "uniform", "forest", ("bounded", 6, 3)]
    parent = np.stack([make_tree(rng, T, kinds[b % len(kinds)]) for b in range(37)])
    say("mask random T", T)
    got, st = _build(parent)
    assert st == 0
    assert np.array_equal(got, oracle.oracle_mask(parent)[:, :, 0])


def test_mask_invalid_parents_status():
    parent = np.stack([make_tree(np.random.default_rng(0), 16, "uniform") for _ in range(5)])
    parent[3, 9] = 9     # self-parent
    parent[4, 2] = -3    # below -1
    parent[1, 0] = 0     # the first node cannot have a parent inside the tree
    say("mask invalid parents")
    got, st = _build(parent)
    assert st == 1 + 1 * 16 + 0
    ok = oracle.oracle_mask(parent[[0, 2]])[:, :, 0]
    assert np.array_equal(got[[0, 2]], ok)
    assert not got[[1, 3, 4]].any()


def test_mask_many_trees():
    rng = np.random.default_rng(5)
    parent = np.stack([make_tree(rng, 64, ("bounded", 8, 3)) for _ in range(300)])
    say("mask 300 trees")
    got, st = _build(parent)
    assert st == 0
    assert np.array_equal(got, oracle.oracle_mask(parent)[:, :, 0])


def test_mask_many_trees_invalid_status():
    """300 trees spread over workgroups: the status names the first invalid
    entry of the first invalid tree, every other tree is built."""
    rng = np.random.default_rng(6)
    parent = np.stack([make_tree(rng, 64, ("bounded", 8, 3)) for _ in range(300)])
    parent[250, 3] = 7      # a later node
    parent[137, 40] = 40    # self-parent
    parent[137, 12] = -2    # below -1: the first invalid entry of tree 137
    say("mask 300 trees, invalid entries")
    got, st = _build(parent)
    assert st == 1 + 137 * 64 + 12
    ok = [b for b in range(300) if b not in (137, 250)]
    assert np.array_equal(got[ok], oracle.oracle_mask(parent[ok])[:, :, 0])
    assert not got[[137, 250]].any()


def test_mask_seventeen_trees_first_tree_invalid():
    """The smallest batch that takes the spread build, with tree 0 invalid."""
    rng = np.random.default_rng(7)
    parent = np.stack([make_tree(rng, 33, "uniform") for _ in range(17)])
    parent[0, 32] = 32
    say("mask 17 trees, tree 0 invalid")
    got, st = _build(parent)
    assert st == 1 + 32
    assert np.array_equal(got[1:], oracle.oracle_mask(parent[1:])[:, :, 0])
    assert not got[0].any()
