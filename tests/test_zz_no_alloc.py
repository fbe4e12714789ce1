"""ltree_attn_noalloc on the GPU, through the C ABI: the partials in the
library's static per-device scratch array instead of a workspace argument.
Two calls in a row, the second smaller than the first (so the array still
holds the first call's partials when the second starts), each bitwise equal
to ltree_attn on the same inputs; the smaller one also against the fp64
oracle.  A call whose partials exceed the array is refused before any launch."""

import zlib

import numpy as np
import pytest
import torch

from gpu_helpers import check_parity, oracle_full, say, to_device
from workloads import make_config, make_workload

pytestmark = pytest.mark.gpu


def _both(w, max_prefix_len=None):
    """(o, lse) of ltree_attn_noalloc and of ltree_attn on w."""
    import tree_attention_amd as ta
    d = to_device(w)
    mask, _ = ta.build_mask(d["parent"])
    B, T, Hq, D = w.q.shape
    mpl = max(w.prefix_lens) if max_prefix_len is None else max_prefix_len
    o = torch.full((B, T, Hq, D), float("nan"), dtype=torch.float32, device="cuda")
    lse = torch.full((B, Hq, T), float("nan"), dtype=torch.float32, device="cuda")
    st = ta.ltree_attn_noalloc(d["q"], d["k_prefix"], d["v_prefix"], d["offsets"], mpl,
                               d["k_tree"], d["v_tree"], mask, o, lse, w.scale)
    assert st == ta.LTREE_OK, ta.ltree_status_string(st)
    o2, lse2 = ta.attn(d["q"], d["k_prefix"], d["v_prefix"], d["offsets"], mpl, d["k_tree"],
                       d["v_tree"], mask, w.scale)
    return o, lse, o2, lse2


def test_two_calls_second_smaller():
    import tree_attention_amd as ta
    big = make_config(4)          # QwQ-shaped layer: 40.6 MiB of partials
    rng = np.random.default_rng(zlib.crc32(b"noalloc_small"))
    small = make_workload(rng, B=2, T=33, Hq=8, Hkv=2, D=128, prefix_lens=[700, 2100],
                          trees=("bounded", 5, 3), dtype="bf16", name="noalloc_small")
    assert ta.ltree_attn_workspace_bytes(1, 64, 40, 8, 128, 32768) <= ta.LTREE_NOALLOC_SCRATCH_BYTES
    say("noalloc: QwQ-shaped call, then a smaller one")
    o_big, lse_big, o_big2, lse_big2 = _both(big, 32768)
    o_small, lse_small, o_small2, lse_small2 = _both(small)
    torch.cuda.synchronize()
    assert torch.equal(o_big, o_big2) and torch.equal(lse_big, lse_big2)
    assert torch.equal(o_small, o_small2) and torch.equal(lse_small, lse_small2)
    check_parity(small, o_small.cpu(), lse_small.cpu(), *oracle_full(small))


def test_fp32_and_repeat():
    """fp32 inputs (the other kernel family) twice in a row: same bits both
    times and as ltree_attn."""
    rng = np.random.default_rng(zlib.crc32(b"noalloc_fp32"))
    w = make_workload(rng, B=2, T=16, Hq=8, Hkv=2, D=64, prefix_lens=[300, 77],
                      trees="uniform", dtype="f32", name="noalloc_fp32")
    say("noalloc: fp32 twice")
    first = _both(w)
    second = _both(w)
    torch.cuda.synchronize()
    for a, b in zip(first, second):
        assert torch.equal(a, b)
    assert torch.equal(first[0], first[2]) and torch.equal(first[1], first[3])
    check_parity(w, first[0].cpu(), first[1].cpu(), *oracle_full(w))


def test_call_beyond_scratch_is_refused():
    """A 256-node tree over a 32768-key prefix (162.5 MiB of partials) is
    refused with LTREE_ERR_SCRATCH before any launch: o and lse untouched."""
    import tree_attention_amd as ta
    B, T, Hq, Hkv, D, L = 1, 256, 40, 8, 128, 32768
    need = ta.ltree_attn_workspace_bytes(B, T, Hq, Hkv, D, L)
    assert need > ta.LTREE_NOALLOC_SCRATCH_BYTES
    dev = "cuda"
    q = torch.zeros((B, T, Hq, D), dtype=torch.bfloat16, device=dev)
    kp = torch.zeros((64, Hkv, D), dtype=torch.bfloat16, device=dev)
    kt = torch.zeros((B, T, Hkv, D), dtype=torch.bfloat16, device=dev)
    offsets = torch.tensor([0, 64], dtype=torch.int32, device=dev)
    parent = torch.arange(-1, T - 1, dtype=torch.int32, device=dev).view(1, T)
    mask, _ = ta.build_mask(parent)
    o = torch.full((B, T, Hq, D), 7.0, dtype=torch.float32, device=dev)
    lse = torch.full((B, Hq, T), 7.0, dtype=torch.float32, device=dev)
    say("noalloc: refused beyond the scratch array")
    st = ta.ltree_attn_noalloc(q, kp, kp, offsets, L, kt, kt, mask, o, lse, 0.088)
    torch.cuda.synchronize()
    assert st == ta.LTREE_ERR_SCRATCH
    assert bool((o == 7.0).all()) and bool((lse == 7.0).all())
