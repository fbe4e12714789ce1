"""Tree-verification attention over a paged prefix cache on the GPU, through
the C ABI: against the fp64 oracle on the gathered keys (`gather_paged`), and
against the packed-layout call on the same keys.  Pages are shuffled through
a pool with unused pages; page sizes 16 to 256 (multiples of 64 and others);
bf16 and fp32; D 64 and 128;
trees up to and beyond 64 nodes; prefix-only mode; a page number outside the
pool and a length above max_prefix_len give NaN rows for that sequence only."""

import zlib

import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import BF16_O_TOL, F32_O_TOL, LSE_TOL, say
from workloads import make_workload

pytestmark = pytest.mark.gpu


def _paginate(w, P, rng, spare=3):
    """Cut the packed prefix cache of w into pages of P keys, shuffled through
    a pool with `spare` unused pages.  Returns CPU tensors (k_pages, v_pages,
    block_table, seq_lens)."""
    lens = list(w.prefix_lens)
    need = [(n + P - 1) // P for n in lens]
    total = sum(need) + spare
    order = rng.permutation(total)
    Hkv, D = w.k_prefix.shape[1], w.k_prefix.shape[2]
    kp = torch.randn(total, P, Hkv, D).to(w.k_prefix.dtype)   # unused rows: noise
    vp = torch.randn(total, P, Hkv, D).to(w.k_prefix.dtype)
    bt = torch.full((len(lens), max(max(need), 1)), -1, dtype=torch.int32)
    off, used = 0, 0
    for b, n in enumerate(lens):
        for j in range(need[b]):
            page = int(order[used])
            used += 1
            bt[b, j] = page
            rows = min(P, n - j * P)
            kp[page, :rows] = w.k_prefix[off + j * P: off + j * P + rows]
            vp[page, :rows] = w.v_prefix[off + j * P: off + j * P + rows]
        off += n
    return kp, vp, bt, torch.tensor(lens, dtype=torch.int32)


def _run(w, kp, vp, bt, lens, max_len=None, tree=True):
    import tree_attention_amd as ta
    dev = "cuda"
    mask = ta.build_mask(w.parent.to(dev))[0] if tree else None
    o, lse = ta.attn_paged(w.q.to(dev), kp.to(dev), vp.to(dev), bt.to(dev), lens.to(dev),
                           max(w.prefix_lens) if max_len is None else max_len,
                           w.k_tree.to(dev) if tree else None,
                           w.v_tree.to(dev) if tree else None, mask, w.scale)
    torch.cuda.synchronize()
    return o.cpu().double().numpy(), lse.cpu().double().numpy()


def _oracle(w, kp, vp, bt, lens, P, tree=True):
    """The oracle over the keys gathered from the pages (not from w.k_prefix)."""
    kg, off = oracle.gather_paged(kp.float().numpy(), bt.numpy(), lens.numpy(), P)
    vg, _ = oracle.gather_paged(vp.float().numpy(), bt.numpy(), lens.numpy(), P)
    if tree:
        return oracle.oracle_attn(w.q, kg, vg, off, w.k_tree, w.v_tree, w.parent.numpy(),
                                  w.scale)
    return oracle.oracle_prefix_attn(w.q, kg, vg, off, w.scale)


def _close(w, o, lse, o_ref, lse_ref):
    tol = BF16_O_TOL if w.dtype == "bf16" else F32_O_TOL
    fin = np.isfinite(lse_ref)
    assert np.array_equal(np.isfinite(lse), fin)
    assert np.max(np.abs(o - o_ref)) <= tol
    assert np.max(np.abs(lse[fin] - lse_ref[fin]), initial=0.0) <= LSE_TOL


CASES = {
    # name: (B, T, Hq, Hkv, D, prefix_lens, trees, dtype, page_size)
    "p64_bf16_ragged": (3, 32, 8, 2, 128, [700, 0, 131], ("bounded", 6, 4), "bf16", 64),
    "p128_bf16_d64": (2, 17, 8, 2, 64, [1000, 129], "uniform", "bf16", 128),
    "p256_fp32": (2, 16, 4, 2, 128, [300, 77], "forest", "f32", 256),
    "p64_bf16_t100": (2, 100, 8, 2, 128, [500, 64], ("bounded", 12, 4), "bf16", 64),
    "p192_bf16_g5": (1, 64, 10, 2, 128, [2000], ("bounded", 8, 3), "bf16", 192),
    # page sizes that are not a multiple of 64: rows addressed lane by lane
    "p16_bf16_ragged": (3, 32, 8, 2, 128, [700, 0, 131], ("bounded", 6, 4), "bf16", 16),
    "p48_bf16_d64": (2, 17, 8, 2, 64, [1000, 129], "uniform", "bf16", 48),
    "p16_bf16_t100": (2, 100, 8, 2, 128, [500, 64], ("bounded", 12, 4), "bf16", 16),
    "p32_fp32": (2, 16, 4, 2, 128, [300, 77], "forest", "f32", 32),
    # a batch of 200 sequences (their splits handed out in dispatch order)
    "p64_bf16_b200": (200, 8, 4, 2, 128, [int(n) for n in np.random.default_rng(200).integers(0, 500, 200)],
                      "uniform", "bf16", 64),
}


def _case(name):
    B, T, Hq, Hkv, D, lens, trees, dtype, P = CASES[name]
    rng = np.random.default_rng(zlib.crc32(name.encode()))
    w = make_workload(rng, B=B, T=T, Hq=Hq, Hkv=Hkv, D=D, prefix_lens=lens, trees=trees,
                      dtype=dtype, name=name)
    return w, P, rng


@pytest.mark.parametrize("name", sorted(CASES))
def test_paged_parity(name):
    import tree_attention_amd as ta
    w, P, rng = _case(name)
    kp, vp, bt, lens = _paginate(w, P, rng)
    say("paged parity", name)
    o, lse = _run(w, kp, vp, bt, lens)
    _close(w, o, lse, *_oracle(w, kp, vp, bt, lens, P))
    # the same keys in the packed layout: the same partial splits, so the
    # same arithmetic
    dev = "cuda"
    mask, _ = ta.build_mask(w.parent.to(dev))
    o2, lse2 = ta.attn(w.q.to(dev), w.k_prefix.to(dev), w.v_prefix.to(dev), w.offsets.to(dev),
                       max(w.prefix_lens), w.k_tree.to(dev), w.v_tree.to(dev), mask, w.scale)
    torch.cuda.synchronize()
    assert np.max(np.abs(o - o2.cpu().double().numpy())) <= 1e-5
    assert np.max(np.abs(lse - lse2.cpu().double().numpy())) <= 1e-5


def test_paged_prefix_only():
    """No tree part: the draft's cross-attention into a paged target cache."""
    w, P, rng = _case("p64_bf16_ragged")
    kp, vp, bt, lens = _paginate(w, P, rng)
    say("paged prefix only")
    o, lse = _run(w, kp, vp, bt, lens, tree=False)
    o_ref, lse_ref = _oracle(w, kp, vp, bt, lens, P, tree=False)
    _close(w, o, lse, o_ref, lse_ref)
    assert np.all(o[1] == 0) and np.all(np.isneginf(lse[1]))   # the empty sequence


def test_paged_bad_page_and_length_give_nan_rows():
    """A page number outside the pool (sequence 0) and a length above
    max_prefix_len (sequence 2) turn only those sequences' rows into NaN."""
    w, P, rng = _case("p64_bf16_ragged")
    kp, vp, bt, lens = _paginate(w, P, rng)
    bt_bad = bt.clone()
    bt_bad[0, 3] = kp.shape[0] + 5
    lens_bad = lens.clone()
    lens_bad[2] = 800                        # above max_prefix_len = 700
    say("paged bad page / length")
    o, lse = _run(w, kp, vp, bt_bad, lens_bad, max_len=700)
    assert np.all(np.isnan(o[0])) and np.all(np.isnan(lse[0]))
    assert np.all(np.isnan(o[2])) and np.all(np.isnan(lse[2]))
    o_ref, lse_ref = _oracle(w, kp, vp, bt, lens, P)
    assert np.max(np.abs(o[1] - o_ref[1])) <= BF16_O_TOL
    assert np.max(np.abs(lse[1] - lse_ref[1])) <= LSE_TOL


@pytest.mark.parametrize("P", [256, 16])
def test_paged_qwq_shape_matches_packed(P):
    """The QwQ-shaped layer (40/8 heads, D 128, prefix 32768, 64-node tree)
    with 256- and 16-key pages shuffled through the pool: the same result as
    the packed call, which the oracle checks elsewhere."""
    import tree_attention_amd as ta
    from workloads import make_config
    w = make_config(4)
    rng = np.random.default_rng(31)
    kp, vp, bt, lens = _paginate(w, P, rng)
    say("paged qwq shape")
    o, lse = _run(w, kp, vp, bt, lens)
    dev = "cuda"
    mask, _ = ta.build_mask(w.parent.to(dev))
    o2, lse2 = ta.attn(w.q.to(dev), w.k_prefix.to(dev), w.v_prefix.to(dev), w.offsets.to(dev),
                       32768, w.k_tree.to(dev), w.v_tree.to(dev), mask, w.scale)
    torch.cuda.synchronize()
    assert np.max(np.abs(o - o2.cpu().double().numpy())) <= 1e-5
    assert np.max(np.abs(lse - lse2.cpu().double().numpy())) <= 1e-5


def test_paged_argument_errors():
    import tree_attention_amd as ta
    w, P, rng = _case("p64_bf16_ragged")
    kp, vp, bt, lens = _paginate(w, P, rng)
    dev = "cuda"
    assert ta.ltree_attn_paged_workspace_bytes(3, 32, 8, 2, 128, 700, 0) == 0   # no page size
    assert ta.ltree_attn_paged_workspace_bytes(3, 32, 8, 2, 128, 700, 48) > 0
    kp0 = torch.zeros(4, 0, 2, 128, dtype=torch.bfloat16, device=dev)
    o = torch.empty((3, 32, 8, 128), dtype=torch.float32, device=dev)
    lse = torch.empty((3, 8, 32), dtype=torch.float32, device=dev)
    ws = torch.empty((1 << 24,), dtype=torch.uint8, device=dev)
    mask, _ = ta.build_mask(w.parent.to(dev))
    say("paged argument errors")
    st = ta.ltree_attn_paged(w.q.to(dev), kp0, kp0, bt.to(dev), lens.to(dev), 700,
                             w.k_tree.to(dev), w.v_tree.to(dev), mask, o, lse, ws, w.scale)
    assert st == ta.LTREE_ERR_INVALID_ARG
    # max_prefix_len beyond what the block table can address
    st = ta.ltree_attn_paged(w.q.to(dev), kp.to(dev), vp.to(dev), bt.to(dev), lens.to(dev),
                             bt.shape[1] * P + 1, w.k_tree.to(dev), w.v_tree.to(dev), mask, o,
                             lse, ws, w.scale)
    assert st == ta.LTREE_ERR_INVALID_ARG
