"""Tree-verification attention over prefix caches whose key rows are not
packed (ltree_attn_strided) on the GPU, through the C ABI: an interleaved K/V
cache [rows, 2, Hkv, D] and caches with padded rows, against the fp64 oracle
on the rows gathered from the flat buffer (`gather_strided`, the definition
of the layout), and bitwise against ltree_attn on a packed copy (the same
arithmetic in the same order).  Trees up to 100 nodes (two tree tiles at the
packed tree stride after strided prefix tiles), prefix-only mode, bf16 and
fp32, the QwQ-shaped layer on every row."""

import zlib

import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import BF16_O_TOL, F32_O_TOL, LSE_TOL, say
from workloads import make_config, make_workload

pytestmark = pytest.mark.gpu


def _interleaved(w, dev="cuda"):
    """[rows, 2, Hkv, D] device cache holding w's prefix K (slot 0) and V (slot 1)."""
    kv = torch.stack([w.k_prefix, w.v_prefix], dim=1).contiguous()
    return kv.to(dev)


def _padded(x, pad, dev="cuda"):
    """[rows, Hkv, D] view of a device buffer whose rows carry `pad` extra
    elements of noise."""
    rows, Hkv, D = x.shape
    buf = torch.randn(rows, Hkv * D + pad).to(x.dtype)
    buf[:, :Hkv * D] = x.reshape(rows, Hkv * D)
    buf = buf.to(dev)
    return buf, buf[:, :Hkv * D].view(rows, Hkv, D) if rows else buf[:, :Hkv * D].reshape(0, Hkv, D)


def _oracle_from_flat(w, kflat, vflat, ks, vs, tree=True):
    Hkv, D = w.k_prefix.shape[1], w.k_prefix.shape[2]
    off = w.offsets.numpy()
    kp = oracle.gather_strided(kflat, off, ks, Hkv, D)
    vp = oracle.gather_strided(vflat, off, vs, Hkv, D)
    if tree:
        return oracle.oracle_attn(w.q, kp, vp, off, w.k_tree, w.v_tree, w.parent.numpy(), w.scale)
    return oracle.oracle_prefix_attn(w.q, kp, vp, off, w.scale)


def _check(w, o, lse, o_ref, lse_ref, empty_ok=False):
    o = o.cpu().double().numpy()
    lse = lse.cpu().double().numpy()
    tol = BF16_O_TOL if w.dtype == "bf16" else F32_O_TOL
    if empty_ok:
        inf = np.isneginf(lse_ref)
        assert np.array_equal(np.isneginf(lse), inf)
        lse, lse_ref = np.where(inf, 0.0, lse), np.where(inf, 0.0, lse_ref)
    eo = float(np.max(np.abs(o - o_ref)))
    el = float(np.max(np.abs(lse - lse_ref)))
    assert eo <= tol, f"o max-abs error {eo:.3e}"
    assert el <= LSE_TOL, f"lse max-abs error {el:.3e}"
    return eo, el


CASES = {
    # name: (B, T, Hq, Hkv, D, prefix_lens, trees, dtype)
    "g5_t64_ragged": (2, 64, 10, 2, 128, [1000, 333], ("bounded", 8, 3), "bf16"),
    "g4_t100_two_tree_tiles": (1, 100, 8, 2, 128, [700], ("bounded", 12, 4), "bf16"),
    "d64_forest_empty": (3, 20, 6, 3, 64, [65, 0, 191], "forest", "bf16"),
    "fp32_t16": (2, 16, 8, 2, 128, [300, 77], "uniform", "f32"),
}


def _case(name):
    B, T, Hq, Hkv, D, lens, trees, dtype = CASES[name]
    rng = np.random.default_rng(zlib.crc32(name.encode()))
    return make_workload(rng, B=B, T=T, Hq=Hq, Hkv=Hkv, D=D, prefix_lens=lens, trees=trees,
                         dtype=dtype, outlier_frac=0.01 if dtype == "bf16" else 0.0, name=name)


@pytest.mark.parametrize("name", sorted(CASES))
def test_interleaved_cache(name):
    import tree_attention_amd as ta
    w = _case(name)
    dev = "cuda"
    kv = _interleaved(w)
    Hkv, D = w.k_prefix.shape[1], w.k_prefix.shape[2]
    mask, _ = ta.build_mask(w.parent.to(dev))
    say("strided interleaved", name)
    o, lse = ta.attn_strided(w.q.to(dev), kv[:, 0], kv[:, 1], w.offsets.to(dev),
                             max(w.prefix_lens), w.k_tree.to(dev), w.v_tree.to(dev), mask, w.scale)
    torch.cuda.synchronize()
    flat = kv.cpu().float().numpy().reshape(-1)
    o_ref, lse_ref = _oracle_from_flat(w, flat, flat[Hkv * D:], 2 * Hkv * D, 2 * Hkv * D)
    _check(w, o, lse, o_ref, lse_ref)
    # the same arithmetic as the packed call
    o2, lse2 = ta.attn(w.q.to(dev), w.k_prefix.to(dev), w.v_prefix.to(dev), w.offsets.to(dev),
                       max(w.prefix_lens), w.k_tree.to(dev), w.v_tree.to(dev), mask, w.scale)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(lse, lse2)


@pytest.mark.parametrize("name,kpad,vpad", [("g5_t64_ragged", 64, 8), ("fp32_t16", 8, 256),
                                            ("g4_t100_two_tree_tiles", 0, 72)])
def test_padded_rows(name, kpad, vpad):
    """K and V rows padded by different amounts (one of them packed)."""
    import tree_attention_amd as ta
    w = _case(name)
    dev = "cuda"
    kbuf, kview = _padded(w.k_prefix, kpad)
    vbuf, vview = _padded(w.v_prefix, vpad)
    Hkv, D = w.k_prefix.shape[1], w.k_prefix.shape[2]
    mask, _ = ta.build_mask(w.parent.to(dev))
    say("strided padded", name, kpad, vpad)
    o, lse = ta.attn_strided(w.q.to(dev), kview, vview, w.offsets.to(dev), max(w.prefix_lens),
                             w.k_tree.to(dev), w.v_tree.to(dev), mask, w.scale)
    torch.cuda.synchronize()
    o_ref, lse_ref = _oracle_from_flat(w, kbuf.cpu().float().numpy().reshape(-1),
                                       vbuf.cpu().float().numpy().reshape(-1),
                                       Hkv * D + kpad, Hkv * D + vpad)
    _check(w, o, lse, o_ref, lse_ref)


def test_single_kv_head_row_view():
    """One KV head: a [rows, 1, D] view of a padded buffer whose size-one head
    dimension carries the row stride (any stride is valid there)."""
    import tree_attention_amd as ta
    rng = np.random.default_rng(zlib.crc32(b"hkv1_view"))
    w = make_workload(rng, B=2, T=24, Hq=8, Hkv=1, D=128, prefix_lens=[600, 130],
                      trees=("bounded", 6, 3), dtype="bf16", name="hkv1_view")
    dev = "cuda"
    D, pad = 128, 40
    rows = sum(w.prefix_lens)
    views, flats = [], []
    for x in (w.k_prefix, w.v_prefix):
        buf = torch.randn(rows, D + pad).to(x.dtype)
        buf[:, :D] = x.reshape(rows, D)
        buf = buf.to(dev)
        v = buf.view(rows, 1, D + pad)[:, :, :D]
        assert v.stride(1) == D + pad
        views.append(v)
        flats.append(buf.cpu().float().numpy().reshape(-1))
    mask, _ = ta.build_mask(w.parent.to(dev))
    say("strided single KV head view")
    o, lse = ta.attn_strided(w.q.to(dev), views[0], views[1], w.offsets.to(dev),
                             max(w.prefix_lens), w.k_tree.to(dev), w.v_tree.to(dev), mask,
                             w.scale)
    torch.cuda.synchronize()
    o_ref, lse_ref = _oracle_from_flat(w, flats[0], flats[1], D + pad, D + pad)
    _check(w, o, lse, o_ref, lse_ref)


def test_prefix_only():
    """Tree arguments NULL: attention over the strided prefix alone; an empty
    prefix gives o = 0 and lse = -inf."""
    import tree_attention_amd as ta
    w = _case("d64_forest_empty")
    dev = "cuda"
    kv = _interleaved(w)
    Hkv, D = w.k_prefix.shape[1], w.k_prefix.shape[2]
    say("strided prefix only")
    o, lse = ta.attn_strided(w.q.to(dev), kv[:, 0], kv[:, 1], w.offsets.to(dev),
                             max(w.prefix_lens), None, None, None, w.scale)
    torch.cuda.synchronize()
    flat = kv.cpu().float().numpy().reshape(-1)
    o_ref, lse_ref = _oracle_from_flat(w, flat, flat[Hkv * D:], 2 * Hkv * D, 2 * Hkv * D,
                                       tree=False)
    _check(w, o, lse, o_ref, lse_ref, empty_ok=True)


def test_qwq_shape_interleaved_all_rows():
    """The QwQ-shaped layer (prefix 32768, 64-node tree, 40/8 heads, 1% of
    rows x8) from an interleaved cache: every element against the oracle,
    one KV head at a time."""
    import tree_attention_amd as ta
    w = make_config(4)
    dev = "cuda"
    kv = _interleaved(w)
    Hq, Hkv, D = w.q.shape[2], w.k_prefix.shape[1], w.k_prefix.shape[2]
    G = Hq // Hkv
    mask, _ = ta.build_mask(w.parent.to(dev))
    say("strided qwq shape")
    o, lse = ta.attn_strided(w.q.to(dev), kv[:, 0], kv[:, 1], w.offsets.to(dev), 32768,
                             w.k_tree.to(dev), w.v_tree.to(dev), mask, w.scale)
    torch.cuda.synchronize()
    o, lse = o.cpu().double().numpy(), lse.cpu().double().numpy()
    flat = kv.cpu().float().numpy().reshape(-1)
    off = w.offsets.numpy()
    kp = oracle.gather_strided(flat, off, 2 * Hkv * D, Hkv, D)
    vp = oracle.gather_strided(flat[Hkv * D:], off, 2 * Hkv * D, Hkv, D)
    eo = el = 0.0
    for g in range(Hkv):
        hs = slice(g * G, (g + 1) * G)
        o_ref, lse_ref = oracle.oracle_attn(w.q[:, :, hs], kp[:, g:g + 1], vp[:, g:g + 1], off,
                                            w.k_tree[:, :, g:g + 1], w.v_tree[:, :, g:g + 1],
                                            w.parent.numpy(), w.scale)
        eo = max(eo, float(np.max(np.abs(o[:, :, hs] - o_ref))))
        el = max(el, float(np.max(np.abs(lse[:, hs] - lse_ref))))
    print(f"[parity] qwq L32k interleaved ltree_attn_strided: o max-abs {eo:.3e} "
          f"lse max-abs {el:.3e}", flush=True)
    assert eo <= BF16_O_TOL and el <= LSE_TOL


def test_strided_argument_errors():
    import tree_attention_amd as ta
    w = _case("g5_t64_ragged")
    dev = "cuda"
    B, T, Hq, D = w.q.shape
    Hkv = w.k_prefix.shape[1]
    q, kt, vt = w.q.to(dev), w.k_tree.to(dev), w.v_tree.to(dev)
    mask, _ = ta.build_mask(w.parent.to(dev))
    o = torch.empty((B, T, Hq, D), dtype=torch.float32, device=dev)
    lse = torch.empty((B, Hq, T), dtype=torch.float32, device=dev)
    ws = torch.empty((1 << 26,), dtype=torch.uint8, device=dev)
    # a row stride that is not a multiple of 8 elements (rows not 16-byte aligned)
    buf = torch.zeros((sum(w.prefix_lens), Hkv * D + 4), dtype=torch.bfloat16, device=dev)
    view = buf[:, :Hkv * D].view(-1, Hkv, D)
    say("strided argument errors")
    st = ta.ltree_attn_strided(q, view, view, w.offsets.to(dev), 1000, kt, vt, mask, o, lse, ws,
                               w.scale)
    assert st == ta.LTREE_ERR_INVALID_ARG
    # a view whose (Hkv, D) part is not packed is refused by the binding
    feature_major = torch.zeros((sum(w.prefix_lens), D, Hkv), dtype=torch.bfloat16,
                                device=dev).transpose(1, 2)
    with pytest.raises(ValueError):
        ta.attn_strided(q, feature_major, view, w.offsets.to(dev), 1000, kt, vt, mask, w.scale)
    torch.cuda.synchronize()
