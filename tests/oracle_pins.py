"""Pins of the fp64 oracle against facts fixed outside it.

Each ``pin_*`` takes the oracle module (``orc``) and raises AssertionError when
the oracle disagrees with a closed form, a library routine, an invariant or a
brute-force computation.  ``test_oracle_pins.py`` runs them on the real
oracle; ``test_oracle_mutations.py`` runs them on copies of the oracle with a
planted mistake and requires that every mistake is caught.

None of these checks re-types the oracle's formula: masks are checked against
closed forms, a hand-worked example and boolean matrix-power reachability;
attention is checked against torch's CPU fp64 ``scaled_dot_product_attention``
(with an explicit boolean mask), scipy's ``logsumexp``, closed forms for
uniform keys and a one-node tree, scalar loops, and invariances.
"""

from __future__ import annotations

import itertools
import math

import numpy as np
import torch
from scipy.special import logsumexp

from workloads import make_tree, make_workload

TOL = 1e-12


def _closure(parent_row: np.ndarray) -> np.ndarray:
    """Reachability by boolean matrix powers: R = (I + P)^T > 0 where
    P[i, parent(i)] = 1.  R[i, j] iff j is reachable from i by parent steps."""
    T = len(parent_row)
    A = np.eye(T, dtype=np.int64)
    for i, p in enumerate(parent_row):
        if p >= 0:
            A[i, p] = 1
    # (I + P)^(2^k) by repeated squaring; 2^k >= T covers every path
    R = A
    for _ in range(max(T, 2).bit_length()):
        R = np.minimum(R @ R, 1)
    return R.astype(bool)


def _unpack(mask_words: np.ndarray, T: int) -> np.ndarray:
    """uint64 [T, W] -> bool [T, T] (bit j%64 of word j//64)."""
    out = np.zeros((T, T), dtype=bool)
    for i in range(T):
        for j in range(T):
            out[i, j] = (int(mask_words[i, j // 64]) >> (j % 64)) & 1
    return out


# ----------------------------------------------------------------- masks

def pin_mask_hand_example(orc):
    """A small forest worked by hand from the ancestor-or-self definition."""
    parent = np.array([[-1, 0, 0, 1, 1, 2, -1, 6]], dtype=np.int32)
    expect = [{0}, {0, 1}, {0, 2}, {0, 1, 3}, {0, 1, 4}, {0, 2, 5}, {6}, {6, 7}]
    m = orc.oracle_mask(parent)
    assert m.shape == (1, 8, 1) and m.dtype == np.uint64
    for i, s in enumerate(expect):
        assert int(m[0, i, 0]) == sum(1 << j for j in s), (i, bin(int(m[0, i, 0])))


def pin_mask_chain_and_star(orc):
    """Chain: row i = bits 0..i (lower-triangular).  Star: row i = {0, i}.
    T = 70 crosses a 64-bit word boundary."""
    for T in (1, 2, 8, 63, 64, 65, 70):
        chain = np.array([[-1] + list(range(T - 1))], dtype=np.int32)
        m = orc.oracle_mask(chain)
        assert m.shape == (1, T, (T + 63) // 64)
        assert np.array_equal(_unpack(m[0], T), np.tril(np.ones((T, T), bool)))
        star = np.array([[-1] + [0] * (T - 1)], dtype=np.int32)
        m = orc.oracle_mask(star)
        want = np.eye(T, dtype=bool)
        want[:, 0] = True
        assert np.array_equal(_unpack(m[0], T), want)


def pin_mask_exhaustive_small(orc):
    """Every parent array with parent[i] in [-1, i-1] for T <= 6 (873 trees and
    forests) against matrix-power reachability, plus popcount == depth where
    depth is counted by the recursion depth(i) = 1 + depth(parent(i))."""
    for T in range(1, 7):
        for choice in itertools.product(*[range(-1, i) for i in range(T)]):
            p = np.array([choice], dtype=np.int32)
            got = _unpack(orc.oracle_mask(p)[0], T)
            assert np.array_equal(got, _closure(p[0])), choice
            depth = []
            for i in range(T):
                depth.append(1 if p[0, i] < 0 else depth[p[0, i]] + 1)
            assert list(got.sum(axis=1)) == depth, choice


def pin_mask_random_recursion(orc):
    """Random trees up to T = 64: row(i) == row(parent(i)) | bit(i) on the
    packed words, and a root row is just its own bit."""
    rng = np.random.default_rng(7)
    for T in (16, 33, 64):
        for kind in ("uniform", ("bounded", 6, 4), "forest"):
            p = make_tree(rng, T, kind)[None, :]
            m = orc.oracle_mask(p)[0, :, 0]
            for i in range(T):
                parent_row = int(m[p[0, i]]) if p[0, i] >= 0 else 0
                assert int(m[i]) == parent_row | (1 << i)


def pin_mask_multiword(orc):
    """Trees of more than 64 nodes (several words per row): a chain of 200 has
    rows 0..i set across words; for random trees row(i) == row(parent(i)) |
    bit(i) on the whole word vector; bits at j >= T stay zero."""
    T = 200
    chain = np.concatenate([[-1], np.arange(T - 1)]).astype(np.int32)[None, :]
    m = orc.oracle_mask(chain)[0]                       # [T, W]
    assert m.shape == (T, 4)
    for i in (0, 63, 64, 127, 150, 199):
        as_int = sum(int(m[i, w]) << (64 * w) for w in range(4))
        assert as_int == (1 << (i + 1)) - 1, i
    rng = np.random.default_rng(8)
    for T in (65, 130, 256):
        for kind in ("uniform", ("bounded", 9, 4), "forest"):
            p = make_tree(rng, T, kind)[None, :]
            m = orc.oracle_mask(p)[0]
            rows = [sum(int(m[i, w]) << (64 * w) for w in range(m.shape[1])) for i in range(T)]
            for i in range(T):
                parent_row = rows[p[0, i]] if p[0, i] >= 0 else 0
                assert rows[i] == parent_row | (1 << i)
                assert rows[i] >> T == 0


def pin_check_parent(orc):
    """Entries outside [-1, i-1] are reported by flat index, in order."""
    p = np.array([[-1, 0, 2, 1], [0, -1, -2, 3]], dtype=np.int32)
    assert orc.check_parent(p) == [2, 4, 6, 7]
    assert orc.check_parent(np.array([[-1, 0, 1, 0]], dtype=np.int32)) == []


# ----------------------------------------------------------- attention

def _case(seed, B=2, T=6, Hq=4, Hkv=2, D=8, prefix_lens=(5, 3), trees="uniform",
          dtype="f32"):
    rng = np.random.default_rng(seed)
    return make_workload(rng, B=B, T=T, Hq=Hq, Hkv=Hkv, D=D,
                         prefix_lens=list(prefix_lens), trees=trees, dtype=dtype)


def _run(orc, w, **over):
    args = dict(q=w.q, k_prefix=w.k_prefix, v_prefix=w.v_prefix,
                offsets=w.offsets.numpy(), k_tree=w.k_tree, v_tree=w.v_tree,
                parent=w.parent.numpy(), scale=w.scale)
    args.update(over)
    return orc.oracle_attn(**args)


def _sdpa_reference(w, visible_fn):
    """torch CPU fp64 SDPA over [prefix | tree] per sequence with the boolean
    mask visible_fn(b, L) -> bool [T, L + T]; GQA by repeating KV heads in
    contiguous groups.  LSE from scipy.special.logsumexp over the same mask."""
    B, T, Hq, D = w.q.shape
    Hkv = w.k_tree.shape[2]
    G = Hq // Hkv
    off = w.offsets.numpy()
    o = np.empty((B, T, Hq, D))
    lse = np.empty((B, Hq, T))
    for b in range(B):
        L = int(off[b + 1] - off[b])
        k = torch.cat([w.k_prefix[off[b]:off[b + 1]], w.k_tree[b]]).double()
        v = torch.cat([w.v_prefix[off[b]:off[b + 1]], w.v_tree[b]]).double()
        k = k.repeat_interleave(G, dim=1).transpose(0, 1).contiguous()  # [Hq, L+T, D]
        v = v.repeat_interleave(G, dim=1).transpose(0, 1).contiguous()
        q = w.q[b].double().transpose(0, 1).contiguous()                 # [Hq, T, D]
        vis = torch.from_numpy(visible_fn(b, L))
        out = torch.nn.functional.scaled_dot_product_attention(
            q, k, v, attn_mask=vis, scale=w.scale)
        o[b] = out.transpose(0, 1).numpy()
        s = (q @ k.transpose(1, 2)).numpy() * w.scale
        lse[b] = logsumexp(s, axis=-1, b=np.broadcast_to(vis.numpy(), s.shape))
    return o, lse


def _tree_visible(w):
    parent = w.parent.numpy()
    T = parent.shape[1]

    def fn(b, L):
        vis = np.ones((T, L + T), dtype=bool)
        vis[:, L:] = _closure(parent[b])
        return vis
    return fn


def pin_general_tree_vs_sdpa(orc):
    """Random trees (uniform, bounded, forest), ragged prefixes including an
    empty one, GQA: oracle == torch SDPA with an explicit reachability mask."""
    for seed, trees, lens, Hq, Hkv in (
            (1, "uniform", (5, 3), 4, 2),
            (2, ("bounded", 3, 2), (0, 9), 6, 3),
            (3, "forest", (4, 1), 4, 4),
            (4, ["chain", "star"], (7, 2), 8, 2)):
        w = _case(seed, trees=trees, prefix_lens=lens, Hq=Hq, Hkv=Hkv)
        o, lse = _run(orc, w)
        ro, rl = _sdpa_reference(w, _tree_visible(w))
        assert np.max(np.abs(o - ro)) < TOL, seed
        assert np.max(np.abs(lse - rl)) < TOL, seed


def pin_large_tree_vs_sdpa(orc):
    """A 100-node tree (two mask words per row) and a 70-node chain: oracle ==
    torch SDPA with the reachability / bottom-right causal mask."""
    w = _case(14, B=2, T=100, Hq=4, Hkv=2, D=8, prefix_lens=(9, 0), trees=("bounded", 12, 3))
    o, lse = _run(orc, w)
    ro, rl = _sdpa_reference(w, _tree_visible(w))
    assert np.max(np.abs(o - ro)) < TOL and np.max(np.abs(lse - rl)) < TOL
    T = 70
    w = _case(15, B=1, T=T, Hq=2, Hkv=1, D=8, prefix_lens=(5,), trees="chain")
    o, lse = _run(orc, w)

    def causal(b, L):
        return np.arange(L + T)[None, :] <= L + np.arange(T)[:, None]
    ro, rl = _sdpa_reference(w, causal)
    assert np.max(np.abs(o - ro)) < TOL and np.max(np.abs(lse - rl)) < TOL


def pin_chain_is_causal(orc):
    """A chain tree is causal attention over [prefix | tree] with the mask
    aligned to the bottom right: key j is visible to row i iff j <= L + i."""
    w = _case(11, T=7, trees="chain", prefix_lens=(6, 0))
    o, lse = _run(orc, w)
    T = 7

    def causal(b, L):
        i = np.arange(T)[:, None]
        j = np.arange(L + T)[None, :]
        return j <= L + i
    ro, rl = _sdpa_reference(w, causal)
    assert np.max(np.abs(o - ro)) < TOL and np.max(np.abs(lse - rl)) < TOL


def pin_single_node_is_decode(orc):
    """T = 1: one-token decode, softmax(q K^T * scale) V over L + 1 keys,
    computed here by a plain unmasked SDPA call."""
    w = _case(12, B=1, T=1, Hq=4, Hkv=2, prefix_lens=(13,))
    o, lse = _run(orc, w)
    k = torch.cat([w.k_prefix, w.k_tree[0]]).double()
    v = torch.cat([w.v_prefix, w.v_tree[0]]).double()
    for h in range(4):
        g = h // 2
        out = torch.nn.functional.scaled_dot_product_attention(
            w.q[0, :, h][None].double(), k[:, g][None], v[:, g][None], scale=w.scale)
        assert np.max(np.abs(o[0, 0, h] - out[0, 0].numpy())) < TOL
        s = (w.q[0, 0, h].double() @ k[:, g].T).numpy() * w.scale
        assert abs(lse[0, h, 0] - logsumexp(s)) < TOL


def pin_uniform_keys(orc):
    """All keys equal: every visible score is s0 = scale <q, k>, so o is the
    mean of the visible values and lse = s0 + ln(L + depth(i))."""
    w = _case(13, B=2, T=6, prefix_lens=(4, 0), trees=("bounded", 3, 2))
    key = torch.randn(w.k_tree.shape[-1], generator=torch.Generator().manual_seed(0))
    kp = key.expand_as(w.k_prefix).clone()
    kt = key.expand_as(w.k_tree).clone()
    o, lse = _run(orc, w, k_prefix=kp, k_tree=kt)
    parent = w.parent.numpy()
    off = w.offsets.numpy()
    G = w.q.shape[2] // w.k_tree.shape[2]
    for b in range(2):
        L = int(off[b + 1] - off[b])
        reach = _closure(parent[b])
        for i in range(6):
            for h in range(w.q.shape[2]):
                g = h // G
                vis = [w.v_prefix[off[b] + j, g].double() for j in range(L)]
                vis += [w.v_tree[b, j, g].double() for j in range(6) if reach[i, j]]
                mean = torch.stack(vis).mean(0).numpy()
                s0 = w.scale * float(w.q[b, i, h].double() @ key.double())
                assert np.max(np.abs(o[b, i, h] - mean)) < TOL
                assert abs(lse[b, h, i] - (s0 + math.log(len(vis)))) < TOL


def pin_brute_force(orc):
    """Scalar Python loops with math.exp and math.fsum on a tiny case; the
    visible set is enumerated by following parent links one step at a time."""
    w = _case(14, B=2, T=5, Hq=4, Hkv=2, D=3, prefix_lens=(3, 0), trees="forest")
    o, lse = _run(orc, w)
    q, kp, vp = w.q.double().tolist(), w.k_prefix.double().tolist(), w.v_prefix.double().tolist()
    kt, vt = w.k_tree.double().tolist(), w.v_tree.double().tolist()
    parent = w.parent.tolist()
    off = w.offsets.tolist()
    for b in range(2):
        for i in range(5):
            path, j = [], i
            while j != -1:
                path.append(j)
                j = parent[b][j]
            for h in range(4):
                g = h // 2
                keys = [kp[r][g] for r in range(off[b], off[b + 1])] + [kt[b][j][g] for j in path]
                vals = [vp[r][g] for r in range(off[b], off[b + 1])] + [vt[b][j][g] for j in path]
                sc = [w.scale * math.fsum(a * c for a, c in zip(q[b][i][h], kk)) for kk in keys]
                ex = [math.exp(x) for x in sc]
                z = math.fsum(ex)
                assert abs(lse[b][h][i] - math.log(z)) < TOL
                for d in range(3):
                    ref = math.fsum(e * vv[d] for e, vv in zip(ex, vals)) / z
                    assert abs(o[b, i, h, d] - ref) < TOL


def pin_split_merge_identity(orc):
    """Prefix partial (no mask) and tree partial (tree mask) joined by the
    log-sum-exp merge equal the single pass; each partial equals an SDPA call
    over its own key set; an empty prefix contributes nothing."""
    w = _case(15, B=2, T=6, Hq=6, Hkv=2, prefix_lens=(9, 0), trees=("bounded", 4, 2))
    (op, lp), (ot, lt), (om, lm) = orc.oracle_attn_split(
        w.q, w.k_prefix, w.v_prefix, w.offsets.numpy(), w.k_tree, w.v_tree,
        w.parent.numpy(), w.scale)
    o, lse = _run(orc, w)
    assert np.max(np.abs(om - o)) < TOL and np.max(np.abs(lm - lse)) < TOL
    assert np.all(np.isneginf(lp[1]))
    T = 6
    ro, rl = _sdpa_reference(w, lambda b, L: np.concatenate(
        [np.ones((T, L), bool), np.zeros((T, T), bool)], axis=1))
    assert np.max(np.abs(op[0] - ro[0])) < TOL and np.max(np.abs(lp[0] - rl[0])) < TOL
    parent = w.parent.numpy()
    rt, rlt = _sdpa_reference(w, lambda b, L: np.concatenate(
        [np.zeros((T, L), bool), _closure(parent[b])], axis=1))
    assert np.max(np.abs(ot - rt)) < TOL and np.max(np.abs(lt - rlt)) < TOL


def pin_lse_merge_closed_form(orc):
    """Two partials with known sums: lse = ln(e^a + e^b) and o is the weighted
    mean; an empty partial (-inf) is ignored."""
    a, b = np.array([0.3, -2.0]), np.array([1.1, -2.0])
    oa, ob = np.array([[1.0, 2.0], [3.0, 4.0]]), np.array([[5.0, 6.0], [7.0, 8.0]])
    o, lse = orc.lse_merge([(oa, a), (ob, b)])
    want = np.log(np.exp(a) + np.exp(b))
    assert np.max(np.abs(lse - want)) < TOL
    wa = np.exp(a) / (np.exp(a) + np.exp(b))
    assert np.max(np.abs(o - (wa[:, None] * oa + (1 - wa)[:, None] * ob))) < TOL
    o2, l2 = orc.lse_merge([(oa, a), (np.full_like(ob, np.nan), np.full(2, -np.inf))])
    assert np.max(np.abs(o2 - oa)) < TOL and np.max(np.abs(l2 - a)) < TOL


def pin_non_ancestor_invariance(orc):
    """Changing K/V of a tree node outside anc*(i) leaves row i bit-identical."""
    w = _case(16, B=1, T=8, prefix_lens=(5,), trees="uniform")
    o, lse = _run(orc, w)
    reach = _closure(w.parent.numpy()[0])
    for j in range(8):
        kt, vt = w.k_tree.clone(), w.v_tree.clone()
        kt[0, j] += 3.0
        vt[0, j] -= 2.0
        o2, l2 = _run(orc, w, k_tree=kt, v_tree=vt)
        for i in range(8):
            same = np.array_equal(o2[0, i], o[0, i]) and np.array_equal(l2[0, :, i], lse[0, :, i])
            assert same == (not reach[i, j]), (i, j)


def pin_prefix_permutation(orc):
    """Permuting prefix rows (K and V together) is invisible up to rounding."""
    w = _case(17, B=1, T=5, prefix_lens=(11,))
    o, lse = _run(orc, w)
    perm = torch.from_numpy(np.random.default_rng(0).permutation(11))
    o2, l2 = _run(orc, w, k_prefix=w.k_prefix[perm], v_prefix=w.v_prefix[perm])
    assert np.max(np.abs(o2 - o)) < TOL and np.max(np.abs(l2 - lse)) < TOL


def pin_gqa_equals_mha(orc):
    """GQA with Hkv heads equals MHA with every KV head repeated G times in
    contiguous order (query head h reads KV head h // G)."""
    w = _case(18, B=2, T=4, Hq=6, Hkv=2, prefix_lens=(3, 2))
    o, lse = _run(orc, w)
    rep = lambda t: t.repeat_interleave(3, dim=-2)  # noqa: E731
    o2, l2 = _run(orc, w, k_prefix=rep(w.k_prefix), v_prefix=rep(w.v_prefix),
                  k_tree=rep(w.k_tree), v_tree=rep(w.v_tree))
    assert np.max(np.abs(o2 - o)) < TOL and np.max(np.abs(l2 - lse)) < TOL


def pin_ragged_equals_separate(orc):
    """A ragged batch equals each sequence run alone."""
    w = _case(19, B=3, T=4, prefix_lens=(2, 0, 5))
    o, lse = _run(orc, w)
    off = w.offsets.numpy()
    for b in range(3):
        ob, lb = orc.oracle_attn(
            w.q[b:b + 1], w.k_prefix[off[b]:off[b + 1]], w.v_prefix[off[b]:off[b + 1]],
            np.array([0, off[b + 1] - off[b]]), w.k_tree[b:b + 1], w.v_tree[b:b + 1],
            w.parent.numpy()[b:b + 1], w.scale)
        assert np.max(np.abs(ob[0] - o[b])) < TOL and np.max(np.abs(lb[0] - lse[b])) < TOL


def pin_rows_vs_sdpa(orc):
    """The per-row form agrees with the SDPA reference on sampled rows."""
    w = _case(20, B=2, T=6, Hq=4, Hkv=2, prefix_lens=(7, 1), trees=("bounded", 3, 3))
    ro, rl = _sdpa_reference(w, _tree_visible(w))
    rows = [(0, 0, 0), (0, 3, 5), (1, 1, 2), (1, 2, 4)]
    o, lse = orc.oracle_attn_rows(w.q, w.k_prefix, w.v_prefix, w.offsets.numpy(),
                                  w.k_tree, w.v_tree, w.parent.numpy(), w.scale, rows)
    for n, (b, h, i) in enumerate(rows):
        assert np.max(np.abs(o[n] - ro[b, i, h])) < TOL
        assert abs(lse[n] - rl[b, h, i]) < TOL


def pin_bf16_inputs_exact(orc):
    """bf16 inputs are consumed exactly: the result equals the fp32 run on the
    same (bf16-representable) values."""
    w = _case(21, dtype="bf16")
    o, lse = _run(orc, w)
    o2, l2 = _run(orc, w, q=w.q.float(), k_prefix=w.k_prefix.float(),
                  v_prefix=w.v_prefix.float(), k_tree=w.k_tree.float(),
                  v_tree=w.v_tree.float())
    assert np.array_equal(o, o2) and np.array_equal(lse, l2)


# ------------------------------------------------- prefix-only attention

def pin_prefix_attn_vs_sdpa(orc):
    """Attention over the prefix alone == torch CPU fp64 SDPA without a mask
    (GQA by repeating KV heads in contiguous groups), lse == scipy logsumexp;
    an empty prefix gives o = 0 and lse = -inf."""
    w = _case(31, B=3, T=5, Hq=6, Hkv=3, prefix_lens=(7, 0, 4))
    o, lse = orc.oracle_prefix_attn(w.q, w.k_prefix, w.v_prefix, w.offsets.numpy(), w.scale)
    off = w.offsets.numpy()
    B, T, Hq, D = w.q.shape
    G = Hq // w.k_prefix.shape[1]
    for b in range(B):
        if off[b + 1] == off[b]:
            assert np.all(o[b] == 0) and np.all(lse[b] == -np.inf)
            continue
        k = w.k_prefix[off[b]:off[b + 1]].double().repeat_interleave(G, dim=1).transpose(0, 1).contiguous()
        v = w.v_prefix[off[b]:off[b + 1]].double().repeat_interleave(G, dim=1).transpose(0, 1).contiguous()
        q = w.q[b].double().transpose(0, 1).contiguous()
        out = torch.nn.functional.scaled_dot_product_attention(q, k, v, scale=w.scale)
        assert np.max(np.abs(o[b] - out.transpose(0, 1).numpy())) < TOL
        s = (q @ k.transpose(1, 2)).numpy() * w.scale
        assert np.max(np.abs(lse[b] - logsumexp(s, axis=-1))) < TOL


def pin_prefix_attn_uniform_keys(orc):
    """All prefix keys equal: o = mean of the sequence's values, lse = s0 + ln L."""
    w = _case(32, B=2, T=3, Hq=4, Hkv=2, prefix_lens=(5, 2))
    key = torch.randn(w.k_prefix.shape[-1], generator=torch.Generator().manual_seed(1))
    kp = key.expand_as(w.k_prefix).clone()
    o, lse = orc.oracle_prefix_attn(w.q, kp, w.v_prefix, w.offsets.numpy(), w.scale)
    off = w.offsets.numpy()
    for b in range(2):
        L = int(off[b + 1] - off[b])
        for h in range(4):
            g = h // 2
            mean = w.v_prefix[off[b]:off[b + 1], g].double().mean(0).numpy()
            for i in range(3):
                s0 = w.scale * float(w.q[b, i, h].double() @ key.double())
                assert np.max(np.abs(o[b, i, h] - mean)) < TOL
                assert abs(lse[b, h, i] - (s0 + math.log(L))) < TOL


# ------------------------------------------------------------ paged cache

def pin_gather_paged_hand_example(orc):
    """Two sequences over a pool of three 2-row pages, worked by hand: sequence
    0 (3 keys) uses pages 2 then 0, sequence 1 (2 keys) page 1."""
    pool = np.arange(3 * 2 * 1 * 1, dtype=np.float64).reshape(3, 2, 1, 1)  # value = 2*page + row
    packed, off = orc.gather_paged(pool, np.array([[2, 0], [1, 7]]), np.array([3, 2]), 2)
    assert off.tolist() == [0, 3, 5]
    assert packed[:, 0, 0].tolist() == [4.0, 5.0, 0.0, 2.0, 3.0]


def pin_gather_paged_contiguous_is_identity(orc):
    """Pages laid out in order (block_table[b, j] = first page of b + j) give
    back the packed cache they were cut from, ragged lengths included; a page
    outside the pool is an error."""
    rng = np.random.default_rng(61)
    P, lens = 4, [9, 0, 4]
    packed = rng.standard_normal((sum(lens), 2, 3))
    npages = [(n + P - 1) // P for n in lens]
    pool = np.zeros((sum(npages), P, 2, 3))
    bt = np.zeros((3, max(npages)), dtype=np.int64)
    first, row = 0, 0
    for b, n in enumerate(lens):
        for j in range(n):
            pool[first + j // P, j % P] = packed[row + j]
        bt[b, :npages[b]] = np.arange(first, first + npages[b])
        first += npages[b]
        row += n
    got, off = orc.gather_paged(pool, bt, np.array(lens), P)
    assert np.array_equal(got, packed) and off.tolist() == [0, 9, 9, 13]
    try:
        orc.gather_paged(pool, np.array([[5]]), np.array([1]), P)
    except ValueError:
        pass
    else:
        raise AssertionError("a page outside the pool was accepted")


# ------------------------------------------------------------ strided cache

def pin_gather_strided_hand_example(orc):
    """Three rows of an interleaved cache [rows, 2, Hkv=1, D=2] worked by hand:
    the buffer holds 0..11 in order, so K rows start at 0, 4, 8 and V rows at
    2, 6, 10 (stride 4 = 2 * Hkv * D)."""
    buf = np.arange(12, dtype=np.float64)
    k = orc.gather_strided(buf, np.array([0, 2, 3]), 4, 1, 2)
    v = orc.gather_strided(buf[2:], np.array([0, 2, 3]), 4, 1, 2)
    assert k[:, 0, :].tolist() == [[0.0, 1.0], [4.0, 5.0], [8.0, 9.0]]
    assert v[:, 0, :].tolist() == [[2.0, 3.0], [6.0, 7.0], [10.0, 11.0]]


def pin_gather_strided_packed_is_identity(orc):
    """Stride Hkv * D gives back the packed cache; padded rows (stride above
    Hkv * D, padding filled with noise) give the same rows; a stride shorter
    than a row is an error."""
    rng = np.random.default_rng(67)
    Hkv, D, lens = 3, 4, [5, 0, 2]
    off = np.concatenate([[0], np.cumsum(lens)])
    packed = rng.standard_normal((sum(lens), Hkv, D))
    assert np.array_equal(orc.gather_strided(packed.reshape(-1), off, Hkv * D, Hkv, D), packed)
    pad = 20
    padded = rng.standard_normal((sum(lens), Hkv * D + pad))
    padded[:, :Hkv * D] = packed.reshape(sum(lens), Hkv * D)
    assert np.array_equal(orc.gather_strided(padded.reshape(-1), off, Hkv * D + pad, Hkv, D), packed)
    try:
        orc.gather_strided(packed.reshape(-1), off, Hkv * D - 1, Hkv, D)
    except ValueError:
        pass
    else:
        raise AssertionError("a stride shorter than a row was accepted")


# ------------------------------------------------------------ sliding window

def _window_run(orc, w, window, **over):
    args = dict(q=w.q, k_cache=w.k_prefix, v_cache=w.v_prefix, offsets=w.offsets.numpy(),
                k_tree=w.k_tree, v_tree=w.v_tree, parent=w.parent.numpy(), scale=w.scale,
                window=window)
    args.update(over)
    return orc.oracle_window_attn(**args)


def pin_window_chain_is_banded_causal(orc):
    """A chain tree under a window W is causal attention over [cache | tree]
    restricted to a band: concatenated key j is visible to row i iff
    L + i - W < j <= L + i (torch CPU fp64 SDPA with that boolean mask)."""
    T = 7
    for seed, lens, window in ((41, (9, 3), 4), (42, (12, 0), 9), (43, (2, 5), 30), (44, (6, 6), 1)):
        w = _case(seed, T=T, trees="chain", prefix_lens=lens)
        o, lse = _window_run(orc, w, window)

        def band(b, L):
            i = np.arange(T)[:, None]
            j = np.arange(L + T)[None, :]
            return (j <= L + i) & (j > L + i - window)
        ro, rl = _sdpa_reference(w, band)
        assert np.max(np.abs(o - ro)) < TOL, (seed, window)
        assert np.max(np.abs(lse - rl)) < TOL, (seed, window)


def pin_window_covering_everything_is_tree_attention(orc):
    """A window at least as long as cache plus tree hides nothing: plain tree
    attention (SDPA with the reachability mask), for random trees, a forest
    and an empty cache."""
    for seed, trees, lens in ((45, "uniform", (5, 3)), (46, ("bounded", 3, 2), (0, 8)),
                              (47, "forest", (4, 1))):
        w = _case(seed, trees=trees, prefix_lens=lens)
        o, lse = _window_run(orc, w, max(lens) + 6)
        ro, rl = _sdpa_reference(w, _tree_visible(w))
        assert np.max(np.abs(o - ro)) < TOL and np.max(np.abs(lse - rl)) < TOL, seed


def pin_window_one_is_the_token_itself(orc):
    """Window 1: every token sees only itself, o = its own value row and
    lse = its own score."""
    w = _case(48, trees=("bounded", 3, 2), prefix_lens=(4, 2))
    o, lse = _window_run(orc, w, 1)
    G = w.q.shape[2] // w.k_tree.shape[2]
    for b in range(2):
        for i in range(6):
            for h in range(w.q.shape[2]):
                g = h // G
                assert np.array_equal(o[b, i, h], w.v_tree[b, i, g].double().numpy())
                s = w.scale * float(w.q[b, i, h].double() @ w.k_tree[b, i, g].double())
                assert abs(lse[b, h, i] - s) < TOL


def pin_window_uniform_keys(orc):
    """All keys equal: o is the mean of the values of the W most recent tokens
    on the row's branch (the cache in order, then the ancestors by depth, the
    token itself last) and lse = s0 + ln min(W, L + depth(i))."""
    w = _case(49, B=2, T=6, prefix_lens=(7, 2), trees=("bounded", 4, 2))
    key = torch.randn(w.k_tree.shape[-1], generator=torch.Generator().manual_seed(2))
    kp = key.expand_as(w.k_prefix).clone()
    kt = key.expand_as(w.k_tree).clone()
    parent = w.parent.numpy()
    off = w.offsets.numpy()
    G = w.q.shape[2] // w.k_tree.shape[2]
    for window in (3, 5, 9):
        o, lse = _window_run(orc, w, window, k_cache=kp, k_tree=kt)
        for b in range(2):
            L = int(off[b + 1] - off[b])
            reach = _closure(parent[b])
            for i in range(6):
                anc = [j for j in range(6) if reach[i, j]]      # topological = by depth
                for h in range(w.q.shape[2]):
                    g = h // G
                    branch = [w.v_prefix[off[b] + j, g].double() for j in range(L)]
                    branch += [w.v_tree[b, j, g].double() for j in anc]
                    recent = branch[-window:]
                    mean = torch.stack(recent).mean(0).numpy()
                    s0 = w.scale * float(w.q[b, i, h].double() @ key.double())
                    assert np.max(np.abs(o[b, i, h] - mean)) < TOL, (window, b, i)
                    assert abs(lse[b, h, i] - (s0 + math.log(min(window, L + len(anc))))) < TOL


# ------------------------------------------------------------ KV commit

def pin_commit_hand_example(orc):
    """Two sequences, one of them accepting nothing, worked by hand."""
    kt = np.arange(2 * 3 * 1 * 2, dtype=np.float32).reshape(2, 3, 1, 2)      # [B,T,Hkv,D]
    vt = -kt
    kc = np.full((6, 1, 2), 7.0, dtype=np.float32)
    vc = np.full((6, 1, 2), 9.0, dtype=np.float32)
    acc = np.array([[0, 2, 1], [1, 0, 0]], dtype=np.int32)
    k2, v2, st = orc.oracle_commit_kv(kt, vt, acc, np.array([2, 0]), np.array([3, 0]), kc, vc)
    assert st == 0
    expect = np.full((6, 1, 2), 7.0, dtype=np.float32)
    expect[3, 0] = [0.0, 1.0]     # tree row (b=0, node 0)
    expect[4, 0] = [4.0, 5.0]     # tree row (b=0, node 2)
    assert np.array_equal(k2, expect) and np.array_equal(v2[3:5], -expect[3:5])
    assert np.all(v2[[0, 1, 2, 5]] == 9.0) and np.all(kc == 7.0)


def pin_commit_chain_appends_tree(orc):
    """Accepting a whole chain in order appends the tree rows unchanged; rows
    outside the destination range keep their values."""
    rng = np.random.default_rng(41)
    kt = rng.standard_normal((2, 5, 3, 4))
    vt = rng.standard_normal((2, 5, 3, 4))
    kc = rng.standard_normal((20, 3, 4))
    vc = rng.standard_normal((20, 3, 4))
    acc = np.tile(np.arange(5, dtype=np.int32), (2, 1))
    k2, v2, st = orc.oracle_commit_kv(kt, vt, acc, np.array([5, 5]), np.array([2, 11]), kc, vc)
    assert st == 0
    assert np.array_equal(k2[2:7], kt[0]) and np.array_equal(k2[11:16], kt[1])
    assert np.array_equal(v2[2:7], vt[0]) and np.array_equal(v2[11:16], vt[1])
    keep = [r for r in range(20) if not (2 <= r < 7 or 11 <= r < 16)]
    assert np.array_equal(k2[keep], kc[keep]) and np.array_equal(v2[keep], vc[keep])


def pin_commit_status(orc):
    """Out-of-range arguments: the first bad sequence is reported and left
    unwritten; good sequences are still written."""
    kt = np.ones((3, 4, 1, 2))
    kc = np.zeros((8, 1, 2))
    acc = np.array([[0, 1, 2, 3], [0, 4, 0, 0], [3, 2, 0, 0]], dtype=np.int32)
    # sequence 1 names node 4 of a 4-node tree
    k2, _, st = orc.oracle_commit_kv(kt, kt, acc, np.array([1, 2, 2]), np.array([0, 2, 5]), kc, kc)
    assert st == 2 and np.all(k2[0] == 1) and np.all(k2[2:4] == 0) and np.all(k2[5:7] == 1)
    # destination past the end, and a negative count
    _, _, st = orc.oracle_commit_kv(kt, kt, acc, np.array([1, 0, 2]), np.array([0, 0, 7]), kc, kc)
    assert st == 3
    _, _, st = orc.oracle_commit_kv(kt, kt, acc, np.array([-1, 0, 0]), np.array([0, 0, 0]), kc, kc)
    assert st == 1
    # an id past n_accepted is ignored
    _, _, st = orc.oracle_commit_kv(kt, kt, acc, np.array([1, 1, 0]), np.array([0, 1, 2]), kc, kc)
    assert st == 0
    # a range ending exactly at the last cache row fits
    k2, _, st = orc.oracle_commit_kv(kt, kt, acc, np.array([0, 0, 2]), np.array([0, 0, 6]), kc, kc)
    assert st == 0 and np.all(k2[6:8] == 1)


# ------------------------------------------------------------ tree RoPE

def _rope_case(seed, trees, lens, D=8, Hq=4, Hkv=2, T=6):
    rng = np.random.default_rng(seed)
    return make_workload(rng, B=len(lens), T=T, Hq=Hq, Hkv=Hkv, D=D, prefix_lens=list(lens),
                         trees=trees, dtype="f32")


def pin_rope_position_zero_is_identity(orc):
    """Roots of a forest over an empty prefix sit at position 0: unchanged;
    every rotation keeps each channel pair's length."""
    w = _rope_case(51, "forest", (0,))
    q, k = orc.oracle_tree_rope(w.q, w.k_tree, w.parent.numpy(), w.offsets.numpy(), 10000.0)
    roots = np.where(w.parent.numpy()[0] == -1)[0]
    assert np.array_equal(q[0, roots], w.q[0, roots].double().numpy())
    assert np.array_equal(k[0, roots], w.k_tree[0, roots].double().numpy())
    for x, x0 in ((q, w.q), (k, w.k_tree)):
        x0 = x0.double().numpy()
        h = x.shape[-1] // 2
        assert np.max(np.abs(np.hypot(x[..., :h], x[..., h:]) - np.hypot(x0[..., :h], x0[..., h:]))) < 1e-12


def pin_rope_chain_positions_and_complex_rotation(orc):
    """A chain after a prefix of 5: node i sits at 5 + i; each pair (k, k+D/2)
    turns by (5 + i) * base^(-2k/D), checked with numpy's complex exponential
    and, for k = 0 (angle = position), with math.cos / math.sin."""
    w = _rope_case(52, "chain", (5,), D=4)
    base = 500.0
    q, _ = orc.oracle_tree_rope(w.q, w.k_tree, w.parent.numpy(), w.offsets.numpy(), base)
    x = w.q.double().numpy()
    for i in range(6):
        p = 5 + i
        c, s_ = math.cos(p), math.sin(p)
        assert np.allclose(q[0, i, :, 0], x[0, i, :, 0] * c - x[0, i, :, 2] * s_, rtol=0, atol=1e-12)
        assert np.allclose(q[0, i, :, 2], x[0, i, :, 2] * c + x[0, i, :, 0] * s_, rtol=0, atol=1e-12)
        z = (x[0, i, :, 1] + 1j * x[0, i, :, 3]) * np.exp(1j * p * base ** -0.5)
        assert np.allclose(q[0, i, :, 1], z.real, rtol=0, atol=1e-12)
        assert np.allclose(q[0, i, :, 3], z.imag, rtol=0, atol=1e-12)


def pin_rope_relative_positions(orc):
    """Scores depend on position differences only: shifting every position by a
    longer prefix leaves every query-key dot product of a sequence unchanged,
    and siblings (same position) score a shared key alike."""
    w = _rope_case(53, ("bounded", 3, 3), (7,), D=16, T=9)
    w2 = _rope_case(53, ("bounded", 3, 3), (7,), D=16, T=9)
    off_long = np.array([0, 1007])
    q1, k1 = orc.oracle_tree_rope(w.q, w.k_tree, w.parent.numpy(), w.offsets.numpy(), 10000.0)
    q2, k2 = orc.oracle_tree_rope(w2.q, w2.k_tree, w2.parent.numpy(), off_long, 10000.0)
    G = 2
    for h in range(4):
        s1 = q1[0, :, h] @ k1[0, :, h // G].T
        s2 = q2[0, :, h] @ k2[0, :, h // G].T
        assert np.max(np.abs(s1 - s2)) < 1e-9


def pin_round_bf16(orc):
    """Against torch's fp32 -> bf16 conversion (round to nearest even) on fp32
    values, ties included."""
    rng = np.random.default_rng(54)
    x = rng.standard_normal(4096).astype(np.float32)
    # exact ties: bf16 values plus half an ulp
    t = torch.tensor(x).to(torch.bfloat16).float().numpy()
    ties = (t.view(np.uint32) | np.uint32(0x8000)).view(np.float32)
    for v in (x, ties):
        ref = torch.tensor(v).to(torch.bfloat16).double().numpy()
        assert np.array_equal(orc.round_bf16(v.astype(np.float64)), ref)


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
