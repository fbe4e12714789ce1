"""KV-cache commit of the accepted draft tokens on the GPU, through the C ABI,
against the fp64 oracle: bit-exact (pure data movement), including the
status word for out-of-range arguments."""

import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import say
from workloads import make_config, make_tree

pytestmark = pytest.mark.gpu


def _path(parent_row, node):
    """Root-to-node path of a tree (the accepted branch ending at `node`)."""
    out = []
    while node != -1:
        out.append(node)
        node = int(parent_row[node])
    return out[::-1]


def _run(kt, vt, acc, n_acc, dst, kc, vc):
    import tree_attention_amd as ta
    dev = "cuda"
    kc_d, vc_d = kc.to(dev), vc.to(dev)
    status = torch.full((1,), -7, dtype=torch.int32, device=dev)
    st = ta.ltree_commit_kv(kt.to(dev), vt.to(dev), acc.to(dev), n_acc.to(dev), dst.to(dev),
                            kc_d, vc_d, status)
    assert st == 0
    torch.cuda.synchronize()
    return kc_d.cpu(), vc_d.cpu(), int(status.cpu()[0])


def _check(kt, vt, acc, n_acc, dst, kc, vc):
    k2, v2, st = _run(kt, vt, acc, n_acc, dst, kc, vc)
    as_np = lambda t: t.view(torch.int16).numpy() if t.dtype == torch.bfloat16 else t.numpy()
    rk, rv, rst = oracle.oracle_commit_kv(as_np(kt), as_np(vt), acc.numpy(), n_acc.numpy(),
                                          dst.numpy(), as_np(kc), as_np(vc))
    assert st == rst
    assert np.array_equal(as_np(k2), rk) and np.array_equal(as_np(v2), rv)
    return st


@pytest.mark.parametrize("dtype,D", [(torch.bfloat16, 128), (torch.bfloat16, 64),
                                     (torch.float32, 128), (torch.float32, 64)])
def test_random_branches(dtype, D):
    rng = np.random.default_rng(D + (1 if dtype == torch.float32 else 0))
    B, T, Hkv, rows = 4, 40, 3, 300
    parent = make_tree(rng, T, ("bounded", 7, 3))
    kt = torch.randn(B, T, Hkv, D).to(dtype)
    vt = torch.randn(B, T, Hkv, D).to(dtype)
    kc = torch.randn(rows, Hkv, D).to(dtype)
    vc = torch.randn(rows, Hkv, D).to(dtype)
    acc = torch.zeros(B, T, dtype=torch.int32)
    n_acc = torch.zeros(B, dtype=torch.int32)
    for b in range(B):
        p = _path(parent, int(rng.integers(0, T)))
        acc[b, :len(p)] = torch.tensor(p, dtype=torch.int32)
        n_acc[b] = len(p)
    n_acc[2] = 0                      # a sequence that accepts nothing
    dst = torch.tensor([0, 60, 120, 290 - int(n_acc[3])], dtype=torch.int32)
    say("commit random branches", dtype, D)
    assert _check(kt, vt, acc, n_acc, dst, kc, vc) == 0


def test_status_and_skipped_sequences():
    B, T, Hkv, D, rows = 3, 8, 2, 128, 30
    kt = torch.randn(B, T, Hkv, D).to(torch.bfloat16)
    kc = torch.zeros(rows, Hkv, D, dtype=torch.bfloat16)
    acc = torch.tensor([[0, 1, 2, 0, 0, 0, 0, 0], [0, 9, 0, 0, 0, 0, 0, 0],
                        [0, 3, 0, 0, 0, 0, 0, 0]], dtype=torch.int32)
    say("commit status")
    st = _check(kt, kt, acc, torch.tensor([3, 2, 2], dtype=torch.int32),
                torch.tensor([0, 5, 28], dtype=torch.int32), kc, kc)
    assert st == 2                    # sequence 1 names node 9 of an 8-node tree
    st = _check(kt, kt, acc, torch.tensor([3, 1, 2], dtype=torch.int32),
                torch.tensor([0, 5, 29], dtype=torch.int32), kc, kc)
    assert st == 3                    # sequence 2 runs past the last cache row


def test_qwq_shape_accepted_branch():
    """The QwQ-shaped tree (64 nodes, 8 KV heads, D = 128): a 4-token branch
    (about the accepted length the pages report) appended after a 32768-row
    prefix cache."""
    w = make_config(4)
    parent = w.parent[0].numpy()
    depth = [len(_path(parent, i)) for i in range(64)]
    leaf = int(np.argmax(np.array(depth) >= 4))
    p = _path(parent, leaf)[:4]
    rows = w.k_prefix.shape[0] + 64
    kc = torch.zeros(rows, 8, 128, dtype=torch.bfloat16)
    kc[:w.k_prefix.shape[0]] = w.k_prefix
    vc = torch.zeros_like(kc)
    vc[:w.v_prefix.shape[0]] = w.v_prefix
    acc = torch.zeros(1, 64, dtype=torch.int32)
    acc[0, :4] = torch.tensor(p, dtype=torch.int32)
    say("commit qwq shape")
    assert _check(w.k_tree, w.v_tree, acc, torch.tensor([4], dtype=torch.int32),
                  torch.tensor([w.k_prefix.shape[0]], dtype=torch.int32), kc, vc) == 0
