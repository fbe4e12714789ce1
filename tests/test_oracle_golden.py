"""The oracle reproduces its committed regression fixtures (tests/golden/,
written by tests/golden/make_golden.py, which calls only oracle/)."""

import os

import numpy as np

import oracle
from workloads import make_config, make_workload

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _load(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            if not line.startswith("#") and line.strip():
                rows.append([float(x) for x in line.split()])
    return np.array(rows)


def test_tiny_fp32_regression():
    w = make_config(1)
    o, lse = oracle.oracle_attn(w.q, w.k_prefix, w.v_prefix, w.offsets.numpy(),
                                w.k_tree, w.v_tree, w.parent.numpy(), w.scale)
    g = _load("tiny_fp32_seed1001.txt")
    assert len(g) == 32
    for h, i, l, o0, o63, osum in g:
        h, i = int(h), int(i)
        assert abs(lse[0, h, i] - l) < 1e-12
        assert abs(o[0, i, h, 0] - o0) < 1e-12
        assert abs(o[0, i, h, 63] - o63) < 1e-12
        assert abs(o[0, i, h].sum() - osum) < 1e-12


def test_ragged_bf16_regression():
    rng = np.random.default_rng(77)
    w = make_workload(rng, B=3, T=5, Hq=6, Hkv=2, D=16, prefix_lens=[0, 7, 3],
                      trees=["forest", "chain", ("bounded", 3, 2)], dtype="bf16")
    o, lse = oracle.oracle_attn(w.q, w.k_prefix, w.v_prefix, w.offsets.numpy(),
                                w.k_tree, w.v_tree, w.parent.numpy(), w.scale)
    g = _load("ragged_bf16_seed77.txt")
    assert len(g) == 90
    for b, h, i, l, osum in g:
        b, h, i = int(b), int(h), int(i)
        assert abs(lse[b, h, i] - l) < 1e-12
        assert abs(o[b, i, h].sum() - osum) < 1e-12
