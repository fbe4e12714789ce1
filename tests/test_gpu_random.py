"""Seeded random problems across the combinations of the calls: tree size
(below and above 64 nodes), GQA group, KV heads, head dimension, dtype,
ragged prefix lengths (empty ones included), packed, paged (page sizes that
are and are not multiples of 64) or strided cache (interleaved K/V, padded
rows), verification, prefix-only and window attention, and the
allocation-free call.  Each case is small enough for the oracle and is
checked against it with the stated tolerances."""

import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import BF16_O_TOL, F32_O_TOL, LSE_TOL, say
from workloads import make_workload

pytestmark = pytest.mark.gpu

KINDS = ["uniform", "chain", "star", "forest", ("bounded", 6, 3), ("bounded", 12, 2)]


def _draw(seed):
    r = np.random.default_rng(10_000 + seed)
    B = int(r.integers(1, 4))
    T = int(r.choice([1, 7, 33, 64, 65, 100, 160]))
    Hkv = int(r.choice([1, 2, 4]))
    G = int(r.choice([1, 3, 5, 8]))
    D = int(r.choice([64, 128]))
    dtype = "bf16" if r.random() < 0.75 else "f32"
    lens = [int(x) if r.random() > 0.15 else 0 for x in r.integers(1, 1500, size=B)]
    kind = KINDS[int(r.integers(len(KINDS)))]
    if isinstance(kind, tuple) and kind[0] == "bounded" and T > 2 ** kind[1]:
        kind = "uniform"
    mode = str(r.choice(["attn", "attn", "prefix", "window"]))
    window = int(max(T, r.integers(1, 700))) if mode == "window" else 0
    page = int(r.choice([0, 0, 16, 64, 100])) if mode != "window" or r.random() < 0.5 else 0
    return dict(B=B, T=T, Hkv=Hkv, G=G, D=D, dtype=dtype, lens=lens, kind=kind, mode=mode,
                window=window, page=page, seed=seed)


def _pages(w, P, seed):
    """Pages of P keys in shuffled order in a pool with two spare pages."""
    r = np.random.default_rng(seed)
    need = [(n + P - 1) // P for n in w.prefix_lens]
    total = sum(need) + 2
    order = r.permutation(total)
    Hkv, D = w.k_prefix.shape[1:]
    kp = torch.zeros(total, P, Hkv, D, dtype=w.k_prefix.dtype)
    vp = torch.zeros_like(kp)
    bt = torch.full((len(need), max(max(need), 1)), 0, dtype=torch.int32)
    off, used = 0, 0
    for b, n in enumerate(w.prefix_lens):
        for j in range(need[b]):
            page = int(order[used])
            used += 1
            bt[b, j] = page
            rows = min(P, n - j * P)
            kp[page, :rows] = w.k_prefix[off + j * P: off + j * P + rows]
            vp[page, :rows] = w.v_prefix[off + j * P: off + j * P + rows]
        off += n
    return kp, vp, bt, torch.tensor(w.prefix_lens, dtype=torch.int32)


@pytest.mark.parametrize("seed", range(256))
def test_random_problem(seed):
    import tree_attention_amd as ta
    c = _draw(seed)
    rng = np.random.default_rng(seed)
    w = make_workload(rng, B=c["B"], T=c["T"], Hq=c["G"] * c["Hkv"], Hkv=c["Hkv"], D=c["D"],
                      prefix_lens=c["lens"], trees=c["kind"], dtype=c["dtype"])
    say("random problem", c)
    dev = "cuda"
    B, T, Hq, D = w.q.shape
    L = max(w.prefix_lens)
    d = {k: getattr(w, k).to(dev) for k in ("q", "k_prefix", "v_prefix", "offsets", "k_tree",
                                             "v_tree", "parent")}
    mask, status = ta.build_mask(d["parent"])
    if c["page"]:
        kp, vp, bt, lens = (t.to(dev) for t in _pages(w, c["page"], seed))
    if c["mode"] == "attn":
        o_ref, lse_ref = oracle.oracle_attn(w.q, w.k_prefix, w.v_prefix, w.offsets.numpy(),
                                            w.k_tree, w.v_tree, w.parent.numpy(), w.scale)
        if c["page"]:
            o, lse = ta.attn_paged(d["q"], kp, vp, bt, lens, L, d["k_tree"], d["v_tree"], mask,
                                   w.scale)
        else:
            o, lse = ta.attn(d["q"], d["k_prefix"], d["v_prefix"], d["offsets"], L, d["k_tree"],
                             d["v_tree"], mask, w.scale)
    elif c["mode"] == "prefix":
        o_ref, lse_ref = oracle.oracle_prefix_attn(w.q, w.k_prefix, w.v_prefix,
                                                   w.offsets.numpy(), w.scale)
        if c["page"]:
            o, lse = ta.attn_paged(d["q"], kp, vp, bt, lens, L, None, None, None, w.scale)
        else:
            o, lse = ta.prefix_attn(d["q"], d["k_prefix"], d["v_prefix"], d["offsets"], L,
                                    w.scale)
    else:
        o_ref, lse_ref = oracle.oracle_window_attn(w.q, w.k_prefix, w.v_prefix,
                                                   w.offsets.numpy(), w.k_tree, w.v_tree,
                                                   w.parent.numpy(), w.scale, c["window"])
        if c["page"]:
            Hkv = w.k_tree.shape[2]
            o = torch.empty((B, T, Hq, D), dtype=torch.float32, device=dev)
            lse = torch.empty((B, Hq, T), dtype=torch.float32, device=dev)
            ws = torch.empty((ta.ltree_window_attn_paged_workspace_bytes(
                B, T, Hq, Hkv, D, c["window"], c["page"]),), dtype=torch.uint8, device=dev)
            assert ta.ltree_window_attn_paged(d["q"], kp, vp, bt, lens, d["k_tree"], d["v_tree"],
                                              mask, o, lse, ws, w.scale, c["window"]) == 0
        else:
            o, lse = ta.window_attn(d["q"], d["k_prefix"], d["v_prefix"], d["offsets"],
                                    d["k_tree"], d["v_tree"], mask, w.scale, c["window"])
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    o, lse = o.cpu().double().numpy(), lse.cpu().double().numpy()
    fin = np.isfinite(lse_ref)           # prefix-only rows of an empty prefix: -inf
    assert np.array_equal(np.isfinite(lse), fin)
    tol = BF16_O_TOL if c["dtype"] == "bf16" else F32_O_TOL
    assert np.max(np.abs(o - o_ref)) <= tol, c
    assert np.max(np.abs(lse[fin] - lse_ref[fin]), initial=0.0) <= LSE_TOL, c


LAYOUTS = ["interleaved", "padded_k", "padded_both", "noalloc"]


def _strided_views(w, layout, seed, dev="cuda"):
    """Device views [rows, Hkv, D] of the prefix K and V in `layout`, holding
    exactly w's packed rows (padding carries noise)."""
    r = np.random.default_rng(seed)
    rows, Hkv, D = w.k_prefix.shape
    if layout == "interleaved":
        kv = torch.stack([w.k_prefix, w.v_prefix], dim=1).contiguous().to(dev)
        return kv[:, 0], kv[:, 1]
    pads = (8 * int(r.integers(1, 9)), 0 if layout == "padded_k" else 8 * int(r.integers(1, 9)))
    out = []
    for x, pad in zip((w.k_prefix, w.v_prefix), pads):
        buf = torch.randn(max(rows, 1), Hkv * D + pad).to(x.dtype)
        buf[:rows, :Hkv * D] = x.reshape(rows, Hkv * D)
        buf = buf.to(dev)
        out.append(buf[:rows, :Hkv * D].view(rows, Hkv, D))
    return out[0], out[1]


@pytest.mark.parametrize("seed", range(100, 164))
def test_random_layout_problem(seed):
    """The same problem distribution over the prefix layouts of the strided
    call (interleaved K/V, padded K rows, both padded by different amounts)
    and over the allocation-free call; checked against the oracle on the
    packed rows, which is what the layouts hold."""
    import tree_attention_amd as ta
    c = _draw(seed)
    layout = LAYOUTS[seed % len(LAYOUTS)]
    mode = "attn" if layout == "noalloc" or c["mode"] != "prefix" else "prefix"
    rng = np.random.default_rng(seed)
    w = make_workload(rng, B=c["B"], T=c["T"], Hq=c["G"] * c["Hkv"], Hkv=c["Hkv"], D=c["D"],
                      prefix_lens=c["lens"], trees=c["kind"], dtype=c["dtype"])
    say("random layout problem", layout, mode, c)
    dev = "cuda"
    B, T, Hq, D = w.q.shape
    L = max(w.prefix_lens)
    d = {k: getattr(w, k).to(dev) for k in ("q", "k_prefix", "v_prefix", "offsets", "k_tree",
                                             "v_tree", "parent")}
    mask, status = ta.build_mask(d["parent"])
    if mode == "attn":
        o_ref, lse_ref = oracle.oracle_attn(w.q, w.k_prefix, w.v_prefix, w.offsets.numpy(),
                                            w.k_tree, w.v_tree, w.parent.numpy(), w.scale)
    else:
        o_ref, lse_ref = oracle.oracle_prefix_attn(w.q, w.k_prefix, w.v_prefix,
                                                   w.offsets.numpy(), w.scale)
    if layout == "noalloc":
        o = torch.empty((B, T, Hq, D), dtype=torch.float32, device=dev)
        lse = torch.empty((B, Hq, T), dtype=torch.float32, device=dev)
        assert ta.ltree_attn_noalloc(d["q"], d["k_prefix"], d["v_prefix"], d["offsets"], L,
                                     d["k_tree"], d["v_tree"], mask, o, lse, w.scale) == 0
    else:
        kv, vv = _strided_views(w, layout, seed)
        tree = (d["k_tree"], d["v_tree"], mask) if mode == "attn" else (None, None, None)
        o, lse = ta.attn_strided(d["q"], kv, vv, d["offsets"], L, *tree, w.scale)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    o, lse = o.cpu().double().numpy(), lse.cpu().double().numpy()
    fin = np.isfinite(lse_ref)
    assert np.array_equal(np.isfinite(lse), fin)
    tol = BF16_O_TOL if c["dtype"] == "bf16" else F32_O_TOL
    assert np.max(np.abs(o - o_ref)) <= tol, c
    assert np.max(np.abs(lse[fin] - lse_ref[fin]), initial=0.0) <= LSE_TOL, c
