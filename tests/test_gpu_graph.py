"""Use under HIP graph capture and on several streams, through the C ABI.

The calls launch kernels only (no allocation, no memset), so they can be
captured: a graph of mask build + attention is replayed several times with
the program's own eager work and synchronisations between the replays, and
every replay must reproduce the eager result bit for bit.  Two calls on two
streams with their own workspaces run concurrently and each matches its
eager result."""

import numpy as np
import pytest
import torch

from gpu_helpers import say
from workloads import make_workload

pytestmark = pytest.mark.gpu


def _inputs(seed, T=64, lens=(1500, 700), paged=False):
    rng = np.random.default_rng(seed)
    w = make_workload(rng, B=len(lens), T=T, Hq=10, Hkv=2, D=128, prefix_lens=list(lens),
                      trees=("bounded", 8, 3), dtype="bf16", outlier_frac=0.01)
    dev = "cuda"
    return w, {k: getattr(w, k).to(dev) for k in ("q", "k_prefix", "v_prefix", "offsets",
                                                   "k_tree", "v_tree", "parent")}


def test_graph_replays_match_eager():
    import tree_attention_amd as ta
    w, d = _inputs(1)
    B, T, Hq, D = w.q.shape
    L = max(w.prefix_lens)
    mask = torch.empty(ta.mask_shape(B, T), dtype=torch.int64, device="cuda")
    status = torch.empty((1,), dtype=torch.int32, device="cuda")
    o = torch.empty((B, T, Hq, D), dtype=torch.float32, device="cuda")
    lse = torch.empty((B, Hq, T), dtype=torch.float32, device="cuda")
    ws = ta.workspace_for(d["q"], d["k_tree"], L)

    def step():
        assert ta.ltree_build_mask(d["parent"], mask, status) == 0
        assert ta.ltree_attn(d["q"], d["k_prefix"], d["v_prefix"], d["offsets"], L, d["k_tree"],
                             d["v_tree"], mask, o, lse, ws, w.scale) == 0

    say("graph: eager reference")
    step()
    torch.cuda.synchronize()
    o_ref, lse_ref = o.clone(), lse.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(4):
        # the program's own eager work between replays: clobber the outputs
        # and the workspace, and run an unrelated eager call
        o.fill_(float("nan"))
        lse.zero_()
        ws.random_(0, 255)
        ta.prefix_attn(d["q"], d["k_prefix"], d["v_prefix"], d["offsets"], L, w.scale)
        torch.cuda.synchronize()
        say("graph replay", rep)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref) and torch.equal(lse, lse_ref), rep
        assert int(status.item()) == 0


def test_paged_graph_replays_match_eager():
    import tree_attention_amd as ta
    w, d = _inputs(2, lens=(1024, 512))
    B, T, Hq, D = w.q.shape
    P = 128
    Hkv = w.k_prefix.shape[1]
    lens = torch.tensor(w.prefix_lens, dtype=torch.int32, device="cuda")
    npages = [n // P for n in w.prefix_lens]
    pool_k = d["k_prefix"].view(sum(npages), P, Hkv, D).flip(0).contiguous()
    pool_v = d["v_prefix"].view(sum(npages), P, Hkv, D).flip(0).contiguous()
    total = sum(npages)
    bt = torch.full((B, max(npages)), -1, dtype=torch.int32)
    first = 0
    for b, n in enumerate(npages):
        bt[b, :n] = torch.tensor([total - 1 - (first + j) for j in range(n)], dtype=torch.int32)
        first += n
    bt = bt.cuda()
    mask, _ = ta.build_mask(d["parent"])
    o = torch.empty((B, T, Hq, D), dtype=torch.float32, device="cuda")
    lse = torch.empty((B, Hq, T), dtype=torch.float32, device="cuda")
    ws = torch.empty((ta.ltree_attn_paged_workspace_bytes(B, T, Hq, Hkv, D, 1024, P),),
                     dtype=torch.uint8, device="cuda")

    def step():
        assert ta.ltree_attn_paged(d["q"], pool_k, pool_v, bt, lens, 1024, d["k_tree"],
                                   d["v_tree"], mask, o, lse, ws, w.scale) == 0

    say("paged graph: eager reference")
    step()
    torch.cuda.synchronize()
    o_ref, lse_ref = o.clone(), lse.clone()
    o2, lse2 = ta.attn(d["q"], d["k_prefix"], d["v_prefix"], d["offsets"], 1024, d["k_tree"],
                       d["v_tree"], mask, w.scale)
    torch.cuda.synchronize()
    assert (o_ref - o2).abs().max().item() <= 1e-5
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(3):
        o.zero_()
        ws.random_(0, 255)
        torch.cuda.synchronize()
        say("paged graph replay", rep)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref) and torch.equal(lse, lse_ref), rep


def test_two_streams_concurrently():
    import tree_attention_amd as ta
    runs = [_inputs(3), _inputs(4, T=33, lens=(300, 2500))]
    eager = []
    for w, d in runs:
        mask, _ = ta.build_mask(d["parent"])
        eager.append(ta.attn(d["q"], d["k_prefix"], d["v_prefix"], d["offsets"],
                             max(w.prefix_lens), d["k_tree"], d["v_tree"], mask, w.scale))
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs = [None, None]
    say("two streams")
    for rep in range(3):
        for k, ((w, d), s) in enumerate(zip(runs, streams)):
            s.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(s):
                mask, _ = ta.build_mask(d["parent"])
                outs[k] = ta.attn(d["q"], d["k_prefix"], d["v_prefix"], d["offsets"],
                                  max(w.prefix_lens), d["k_tree"], d["v_tree"], mask, w.scale)
        torch.cuda.synchronize()
        for k in range(2):
            assert torch.equal(outs[k][0], eager[k][0]) and torch.equal(outs[k][1], eager[k][1])
