"""Every output element at full workload sizes, against the fp64 oracle.

The four bf16 workloads (Llama-3-8B-shaped layers at 16k and 128k prefixes,
the QwQ-32B-shaped layer at 32k with 1% outlier rows, the ragged batch of four
prefixes up to 128k), a 256-node tree on the QwQ-shaped layer, the draft's
cross-attention and 512-key window attention over that layer, and the
verification call over a paged copy of its cache: the library's o and lse are
compared element by element with the oracle, which runs one KV head at a time
(its G query heads against that head's keys: a sub-problem of the same
definition, gist.science "LongSpec..." page, section 2 "Methodik", part C,
where the merged result equals one softmax over the whole visible set).

Each test prints its max-abs errors (`[parity] ...` lines, shown with
pytest -rP) so the margins to the tolerances are on record."""

import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import BF16_O_TOL, LSE_TOL, say
from workloads import make_config, make_workload

pytestmark = pytest.mark.gpu


def _report(case, w, eo, el):
    msg = (f"[parity] {case}: B={w.q.shape[0]} T={w.q.shape[1]} Hq={w.q.shape[2]} "
           f"Hkv={w.k_tree.shape[2]} lens={w.prefix_lens} o max-abs {eo:.3e} "
           f"(tol {BF16_O_TOL}) lse max-abs {el:.3e} (tol {LSE_TOL})")
    print(msg, flush=True)
    say(msg)


def _per_kv_head(w, fn):
    """Yield (query-head slice, o_ref, lse_ref) for every KV head g, from
    fn(q_g, k_prefix_g, v_prefix_g, k_tree_g, v_tree_g) on that head's
    G query heads and its keys."""
    Hq, Hkv = w.q.shape[2], w.k_tree.shape[2]
    G = Hq // Hkv
    for g in range(Hkv):
        hs = slice(g * G, (g + 1) * G)
        kv = slice(g, g + 1)
        yield hs, fn(w.q[:, :, hs], w.k_prefix[:, kv], w.v_prefix[:, kv], w.k_tree[:, :, kv],
                     w.v_tree[:, :, kv])


def _compare_all(w, o, lse, refs, empty_ok=False):
    """Max-abs errors over every element; o [B,T,Hq,D], lse [B,Hq,T] on the host."""
    o = o.double().numpy()
    lse = lse.double().numpy()
    eo = el = 0.0
    for hs, (o_ref, lse_ref) in refs:
        og, lg = o[:, :, hs], lse[:, hs]
        if empty_ok:  # empty softmax: lse -inf on both sides
            inf = np.isneginf(lse_ref)
            assert np.array_equal(np.isneginf(lg), inf)
            lg, lse_ref = np.where(inf, 0.0, lg), np.where(inf, 0.0, lse_ref)
        assert np.all(np.isfinite(og)) and np.all(np.isfinite(lg))
        eo = max(eo, float(np.max(np.abs(og - o_ref))))
        el = max(el, float(np.max(np.abs(lg - lse_ref))))
    return eo, el


def _tree_attn_refs(w):
    off = w.offsets.numpy()
    par = w.parent.numpy()
    return _per_kv_head(w, lambda q, kp, vp, kt, vt: oracle.oracle_attn(
        q, kp, vp, off, kt, vt, par, w.scale))


def _run_attn(w):
    import tree_attention_amd as ta
    dev = "cuda"
    mask, status = ta.build_mask(w.parent.to(dev))
    o, lse = ta.attn(w.q.to(dev), w.k_prefix.to(dev), w.v_prefix.to(dev), w.offsets.to(dev),
                     max(w.prefix_lens), w.k_tree.to(dev), w.v_tree.to(dev), mask, w.scale)
    torch.cuda.synchronize()
    assert int(status.cpu()[0]) == 0
    return o.cpu(), lse.cpu()


@pytest.mark.parametrize("k", [2, 3, 4, 5])
def test_config_all_rows(k):
    w = make_config(k)
    say("full config all rows", k, w.shape)
    o, lse = _run_attn(w)
    eo, el = _compare_all(w, o, lse, _tree_attn_refs(w))
    _report(f"config {k} ltree_attn", w, eo, el)
    assert eo <= BF16_O_TOL and el <= LSE_TOL


def _shard(w, name, heads=None, last_keys=None):
    """One GPU's share of w under 8-way sharding: KV head heads[0] with its
    query heads, or the last `last_keys` prefix keys with every head."""
    from dataclasses import replace
    Hq, Hkv = w.q.shape[2], w.k_tree.shape[2]
    G = Hq // Hkv
    if heads is not None:
        g = heads
        hs, kv = slice(g * G, (g + 1) * G), slice(g, g + 1)
        return replace(w, name=name, q=w.q[:, :, hs].contiguous(),
                       k_prefix=w.k_prefix[:, kv].contiguous(),
                       v_prefix=w.v_prefix[:, kv].contiguous(),
                       k_tree=w.k_tree[:, :, kv].contiguous(),
                       v_tree=w.v_tree[:, :, kv].contiguous())
    L = last_keys
    return replace(w, name=name, k_prefix=w.k_prefix[-L:].contiguous(),
                   v_prefix=w.v_prefix[-L:].contiguous(),
                   offsets=torch.tensor([0, L], dtype=torch.int32), prefix_lens=[L])


@pytest.mark.parametrize("share", ["kv_head_7", "context_last_4096"])
def test_qwq_shape_one_gpu_share_all_rows(share):
    """The shares `bench.py --row shard` times: KV head 7 alone (8-way tensor
    parallel: 5 query heads over all 32768 keys, 128 splits of 256 keys) and
    the last 4096 prefix keys with every head and the tree (8-way context
    parallel)."""
    w = make_config(4)
    w = _shard(w, share, heads=7) if share.startswith("kv") else _shard(w, share, last_keys=4096)
    say("one GPU share", share)
    o, lse = _run_attn(w)
    eo, el = _compare_all(w, o, lse, _tree_attn_refs(w))
    _report(f"qwq share {share} ltree_attn", w, eo, el)
    assert eo <= BF16_O_TOL and el <= LSE_TOL


def test_qwq_shape_256_node_tree_all_rows():
    """QwQ-shaped layer with a 256-node tree (depth <= 12, branching <= 3):
    1280 query rows per KV head in four row blocks, four tree tiles."""
    rng = np.random.default_rng(2024)
    w = make_workload(rng, B=1, T=256, Hq=40, Hkv=8, D=128, prefix_lens=[32768],
                      trees=("bounded", 12, 3), dtype="bf16", outlier_frac=0.01,
                      name="qwq-T256")
    say("big tree qwq shape, all rows")
    o, lse = _run_attn(w)
    eo, el = _compare_all(w, o, lse, _tree_attn_refs(w))
    _report("qwq L32k T256 ltree_attn", w, eo, el)
    assert eo <= BF16_O_TOL and el <= LSE_TOL


def test_qwq_shape_cross_attention_all_heads():
    """The draft's cross-attention into the QwQ-shaped layer's 32768-key cache."""
    import tree_attention_amd as ta
    w = make_config(4)
    dev = "cuda"
    say("cross-attention qwq shape, all heads")
    o, lse = ta.prefix_attn(w.q.to(dev), w.k_prefix.to(dev), w.v_prefix.to(dev),
                            w.offsets.to(dev), max(w.prefix_lens), w.scale)
    torch.cuda.synchronize()
    off = w.offsets.numpy()
    refs = _per_kv_head(w, lambda q, kp, vp, kt, vt: oracle.oracle_prefix_attn(
        q, kp, vp, off, w.scale))
    eo, el = _compare_all(w, o.cpu(), lse.cpu(), refs)
    _report("qwq L32k ltree_prefix_attn", w, eo, el)
    assert eo <= BF16_O_TOL and el <= LSE_TOL


def test_qwq_shape_window_all_heads():
    """Window 512 over the QwQ-shaped layer's cache (its last 511 rows are
    read), the 64-node tree, every KV head."""
    import tree_attention_amd as ta
    w = make_config(4)
    dev = "cuda"
    mask, _ = ta.build_mask(w.parent.to(dev))
    say("window 512 qwq shape, all heads")
    o, lse = ta.window_attn(w.q.to(dev), w.k_prefix.to(dev), w.v_prefix.to(dev),
                            w.offsets.to(dev), w.k_tree.to(dev), w.v_tree.to(dev), mask,
                            w.scale, 512)
    torch.cuda.synchronize()
    off = w.offsets.numpy()
    par = w.parent.numpy()
    refs = _per_kv_head(w, lambda q, kp, vp, kt, vt: oracle.oracle_window_attn(
        q, kp, vp, off, kt, vt, par, w.scale, 512))
    eo, el = _compare_all(w, o.cpu(), lse.cpu(), refs)
    _report("qwq L32k window 512 ltree_window_attn", w, eo, el)
    assert eo <= BF16_O_TOL and el <= LSE_TOL


@pytest.mark.parametrize("P", [256, 16])
def test_qwq_shape_paged_all_rows(P):
    """The QwQ-shaped layer's cache cut into P-key pages shuffled through a
    pool (with unused noise pages); the oracle runs on the keys gathered from
    the pool through the block table, not on the packed copy."""
    import tree_attention_amd as ta
    w = make_config(4)
    rng = np.random.default_rng(31 + P)
    L = w.prefix_lens[0]
    npg = (L + P - 1) // P
    total = npg + 3
    order = rng.permutation(total)
    Hkv, D = w.k_prefix.shape[1], w.k_prefix.shape[2]
    kp = torch.randn(total, P, Hkv, D).to(torch.bfloat16)
    vp = torch.randn(total, P, Hkv, D).to(torch.bfloat16)
    bt = torch.from_numpy(order[:npg].astype(np.int32)).reshape(1, npg)
    for j in range(npg):
        rows = min(P, L - j * P)
        kp[int(order[j]), :rows] = w.k_prefix[j * P: j * P + rows]
        vp[int(order[j]), :rows] = w.v_prefix[j * P: j * P + rows]
    lens = torch.tensor([L], dtype=torch.int32)
    dev = "cuda"
    mask, _ = ta.build_mask(w.parent.to(dev))
    say("paged qwq shape, all rows, page", P)
    o, lse = ta.attn_paged(w.q.to(dev), kp.to(dev), vp.to(dev), bt.to(dev), lens.to(dev), L,
                           w.k_tree.to(dev), w.v_tree.to(dev), mask, w.scale)
    torch.cuda.synchronize()
    kg, off = oracle.gather_paged(kp.float().numpy(), bt.numpy(), lens.numpy(), P)
    vg, _ = oracle.gather_paged(vp.float().numpy(), bt.numpy(), lens.numpy(), P)
    Hq = w.q.shape[2]
    G = Hq // Hkv
    par = w.parent.numpy()
    refs = []
    for g in range(Hkv):
        hs = slice(g * G, (g + 1) * G)
        refs.append((hs, oracle.oracle_attn(w.q[:, :, hs], kg[:, g:g + 1], vg[:, g:g + 1], off,
                                            w.k_tree[:, :, g:g + 1], w.v_tree[:, :, g:g + 1],
                                            par, w.scale)))
    eo, el = _compare_all(w, o.cpu(), lse.cpu(), refs)
    _report(f"qwq L32k paged P={P} ltree_attn_paged", w, eo, el)
    assert eo <= BF16_O_TOL and el <= LSE_TOL
