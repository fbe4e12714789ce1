"""Plain, slow, fp64 reference of hybrid tree-verification attention.

TEST INFRASTRUCTURE ONLY (see the package docstring): the product path never
imports this module.

What is computed.  A batch of B sequences; sequence b has a cached prefix of
L_b keys/values (the target model's KV cache) and a speculated tree of T draft
tokens.  Query head h reads KV head g = h // G with G = Hq // Hkv.  Tree node i
of sequence b sees

    V(b, i) = {all L_b prefix positions}  U  {tree nodes j in anc*(i)}

where anc*(i) is i itself and every ancestor of i in the tree.  With
s_j = scale * <q_i, k_j> over V(b, i),

    lse[b, h, i] = ln sum_{j in V} exp(s_j)        (natural log)
    o[b, i, h]   = sum_{j in V} exp(s_j - lse) * v_j

Citations are by page title and section:

* [GIST-2C] gist.science, "LongSpec: Long-Context Lossless Speculative
  Decoding with Efficient Drafting and Verification", section 2 "Methodik",
  part C "Schnelle Tree Attention".  Item 1 of its split: the cached part is
  the main KV cache and takes no mask.  Item 2: the speculative part is the
  few new draft tokens and takes a tree mask.  "Aggregation": the two partial
  results are joined exactly with a log-sum-exp step.
* [GIST-1] same page, section 1 "Problemstellung", item "Ineffiziente
  Verifikation": verification of a speculation tree uses a tree-attention mask.
* [ARXIV-ABS] mlsanity.com page of the same paper, section "Abstract
  (arXiv)": fast prefix computation combined with standard tree attention.
* [GIST-2A] the gist.science page, section 2 "Methodik", part A, item
  "Cross-Attention mit geteiltem KV-Cache": the draft model reads the target
  model's KV cache directly.
* [GIST-1P] the gist.science page, section 1 "Problemstellung", item
  "Trainings-Inferenz-Diskrepanz": positions enter through RoPE and the draft's
  positions must agree with the target's; [MLS-REF] the mlsanity.com page
  lists RoFormer (rotary position embedding) among the paper's references.
* [GIST-2AW] the gist.science page, section 2 "Methodik", part A, item
  "Sliding-Window Self-Attention": the draft model's self-attention sees a
  window of recent tokens (512 for instance), so its own cache stays bounded.
* [GIST-INTRO] the gist.science page, opening explanation: the target model
  keeps (writes down) the draft proposals it accepts; [GIST-3] its section 3
  "Wichtige Ergebnisse": about 3.5 to 4 tokens are accepted per pass.

Readings where the pages are silent:

* mask = ancestor-or-self ("standard tree attention": a draft token sees its
  own branch, itself included, and no sibling or cousin);
* parent[i] = -1 attaches node i directly to the prefix; otherwise
  0 <= parent[i] < i (nodes in topological order); several roots are allowed;
* every tree node sees every prefix key; L_b = 0 is allowed;
* GQA groups are contiguous: h -> h // (Hq // Hkv);
* lse uses the natural logarithm; o and lse are returned in fp64 here.
"""

from __future__ import annotations

import numpy as np

__all__ = [
    "check_parent",
    "ancestor_matrix",
    "tree_depth",
    "oracle_mask",
    "oracle_attn",
    "oracle_attn_rows",
    "oracle_attn_split",
    "lse_merge",
    "oracle_prefix_attn",
    "oracle_window_attn",
    "gather_paged",
    "gather_strided",
    "oracle_commit_kv",
    "oracle_tree_rope",
    "round_bf16",
]


# --------------------------------------------------------------------------
# Tree mask  ([GIST-1], [GIST-2C] item 2)
# --------------------------------------------------------------------------

def check_parent(parent) -> list[int]:
    """Return the flat indices b*T + i of invalid parent entries, in order.

    A parent entry is valid when -1 <= parent[b, i] <= i - 1: -1 hangs node i
    directly under the prefix, any other value names an earlier node.  This
    ordering rule also excludes cycles.
    """
    p = np.asarray(parent)
    if p.ndim != 2:
        raise ValueError("parent must be [B, T]")
    B, T = p.shape
    bad = []
    for b in range(B):
        for i in range(T):
            if not (-1 <= int(p[b, i]) <= i - 1):
                bad.append(b * T + i)
    return bad


def ancestor_matrix(parent) -> np.ndarray:
    """bool [B, T, T]; entry [b, i, j] is True iff j is i or an ancestor of i.

    Built by walking up from every node i along parent links until the walk
    leaves the tree (parent -1).  This is the tree mask of the speculative part
    ([GIST-2C] item 2) under the ancestor-or-self reading.
    """
    p = np.asarray(parent)
    bad = check_parent(p)
    if bad:
        raise ValueError(f"invalid parent entries at flat indices {bad[:8]}")
    B, T = p.shape
    anc = np.zeros((B, T, T), dtype=bool)
    for b in range(B):
        for i in range(T):
            j = i
            while j != -1:
                anc[b, i, j] = True
                j = int(p[b, j])
    return anc


def tree_depth(parent) -> np.ndarray:
    """int [B, T]: number of nodes on the path from the prefix to i (root = 1)."""
    return ancestor_matrix(parent).sum(axis=2).astype(np.int64)


def oracle_mask(parent) -> np.ndarray:
    """uint64 [B, T, W] with W = ceil(T / 64): bit (j % 64) of word j // 64 of
    row (b, i) is set iff j is i or an ancestor of i.  Bits at j >= T are 0."""
    anc = ancestor_matrix(parent)
    B, T, _ = anc.shape
    W = (T + 63) // 64
    out = np.zeros((B, T, W), dtype=np.uint64)
    for b in range(B):
        for i in range(T):
            for j in range(T):
                if anc[b, i, j]:
                    out[b, i, j // 64] |= np.uint64(1) << np.uint64(j % 64)
    return out


# --------------------------------------------------------------------------
# Attention over [prefix | tree]  ([GIST-2C], [ARXIV-ABS])
# --------------------------------------------------------------------------

def _f64(x) -> np.ndarray:
    """Exact upcast to fp64 (bf16 and fp32 values are fp64-representable)."""
    if hasattr(x, "detach"):  # a torch tensor: go through fp32, then numpy
        x = x.detach().cpu().float().numpy()
    return np.asarray(x, dtype=np.float64)


def _shapes(q, k_tree, offsets):
    B, T, Hq, D = q.shape
    Hkv = k_tree.shape[2]
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    off = np.asarray(offsets, dtype=np.int64)
    if off.shape != (B + 1,) or off[0] != 0 or np.any(np.diff(off) < 0):
        raise ValueError("offsets must be [B+1], start at 0 and not decrease")
    return B, T, Hq, Hkv, D, Hq // Hkv, off


def _masked_softmax_rows(s: np.ndarray, visible: np.ndarray, vals: np.ndarray):
    """Softmax of each row of s over its visible columns, applied to vals.

    Returns (o [n, D], lse [n]) with lse = ln sum_visible exp(s)."""
    s = np.where(visible, s, -np.inf)
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    z = e.sum(axis=1, keepdims=True)
    o = (e @ vals) / z
    lse = (m + np.log(z))[:, 0]
    return o, lse


def oracle_attn(q, k_prefix, v_prefix, offsets, k_tree, v_tree, parent, scale):
    """Full masked attention of every tree token over [prefix | tree].

    q [B,T,Hq,D]; k_prefix, v_prefix [sum L_b, Hkv, D] packed by `offsets`
    [B+1]; k_tree, v_tree [B,T,Hkv,D]; parent [B,T].  Returns fp64
    o [B,T,Hq,D] and lse [B,Hq,T].

    One softmax runs over the concatenated key list of each sequence: every
    prefix column is visible ([GIST-2C] item 1, the cached part has no mask)
    and tree column j is visible to row i iff j is in anc*(i) ([GIST-2C]
    item 2).  This is the plain definition that the split-and-merge method
    of [GIST-2C] reaches exactly.
    """
    q = _f64(q)
    kp, vp, kt, vt = _f64(k_prefix), _f64(v_prefix), _f64(k_tree), _f64(v_tree)
    B, T, Hq, Hkv, D, G, off = _shapes(q, kt, offsets)
    anc = ancestor_matrix(parent)
    o = np.empty((B, T, Hq, D))
    lse = np.empty((B, Hq, T))
    for b in range(B):
        L = int(off[b + 1] - off[b])
        visible = np.ones((T, L + T), dtype=bool)
        visible[:, L:] = anc[b]
        for g in range(Hkv):
            keys = np.concatenate([kp[off[b]:off[b + 1], g, :], kt[b, :, g, :]])
            vals = np.concatenate([vp[off[b]:off[b + 1], g, :], vt[b, :, g, :]])
            for h in range(g * G, (g + 1) * G):
                s = scale * (q[b, :, h, :] @ keys.T)
                o[b, :, h, :], lse[b, h, :] = _masked_softmax_rows(s, visible, vals)
    return o, lse


def oracle_attn_rows(q, k_prefix, v_prefix, offsets, k_tree, v_tree, parent,
                     scale, rows):
    """Same definition as `oracle_attn`, evaluated only for the query rows
    `rows` = iterable of (b, h, i).  Returns o [n, D] and lse [n] in fp64.

    Used at full workload sizes, where the sampled rows are computed one by
    one."""
    q = _f64(q)
    kt = _f64(k_tree)
    B, T, Hq, Hkv, D, G, off = _shapes(q, kt, offsets)
    anc = ancestor_matrix(parent)
    rows = list(rows)
    o = np.empty((len(rows), D))
    lse = np.empty(len(rows))
    vt = _f64(v_tree)
    cache = {}  # fp64 copies of one (sequence, KV head) key/value list
    for n, (b, h, i) in enumerate(rows):
        g = h // G
        if (b, g) not in cache:
            cache.clear()
            kpg = _f64(k_prefix[int(off[b]):int(off[b + 1]), g, :])
            vpg = _f64(v_prefix[int(off[b]):int(off[b + 1]), g, :])
            cache[(b, g)] = (np.concatenate([kpg, kt[b, :, g, :]]),
                             np.concatenate([vpg, vt[b, :, g, :]]), kpg.shape[0])
        keys, vals, L = cache[(b, g)]
        visible = np.ones((1, L + T), dtype=bool)
        visible[0, L:] = anc[b, i]
        s = scale * (q[b, i, h, :][None, :] @ keys.T)
        on, ln = _masked_softmax_rows(s, visible, vals)
        o[n], lse[n] = on[0], ln[0]
    return o, lse


# --------------------------------------------------------------------------
# Split form: cached part + speculative part + LSE aggregation ([GIST-2C])
# --------------------------------------------------------------------------

def lse_merge(parts):
    """Join partial softmax results over disjoint key sets.

    parts: list of (o_k, lse_k) where o_k is normalised over key set k and
    lse_k = ln sum_{j in set k} exp(s_j).  Sets whose lse is -inf (empty) are
    skipped.  Returns (o, lse) of the softmax over the union of the sets:
    lse = ln sum_k exp(lse_k) and o = sum_k exp(lse_k - lse) * o_k.  This is the
    log-sum-exp aggregation of [GIST-2C]."""
    lses = np.stack([p[1] for p in parts])            # [K, ...]
    m = lses.max(axis=0)
    w = np.exp(lses - m)                              # exp(-inf) -> 0
    z = w.sum(axis=0)
    lse = m + np.log(z)
    o = sum((w[k] / z)[..., None] * np.nan_to_num(parts[k][0])
            for k in range(len(parts)))
    return o, lse


def oracle_attn_split(q, k_prefix, v_prefix, offsets, k_tree, v_tree, parent,
                      scale):
    """The method's own decomposition ([GIST-2C]): attention of the tree
    queries over the prefix alone (no mask), attention over the tree tokens
    alone (tree mask), then `lse_merge`.  Returns the prefix partial, the tree
    partial and the merged result.  Used to test the aggregation identity;
    parity is checked against `oracle_attn`."""
    q = _f64(q)
    kp, vp, kt, vt = _f64(k_prefix), _f64(v_prefix), _f64(k_tree), _f64(v_tree)
    B, T, Hq, Hkv, D, G, off = _shapes(q, kt, offsets)
    anc = ancestor_matrix(parent)
    o_p = np.full((B, T, Hq, D), np.nan)
    lse_p = np.full((B, Hq, T), -np.inf)
    o_t = np.empty((B, T, Hq, D))
    lse_t = np.empty((B, Hq, T))
    for b in range(B):
        L = int(off[b + 1] - off[b])
        for g in range(Hkv):
            kpg, vpg = kp[off[b]:off[b + 1], g, :], vp[off[b]:off[b + 1], g, :]
            ktg, vtg = kt[b, :, g, :], vt[b, :, g, :]
            for h in range(g * G, (g + 1) * G):
                if L > 0:
                    s = scale * (q[b, :, h, :] @ kpg.T)
                    o_p[b, :, h, :], lse_p[b, h, :] = _masked_softmax_rows(
                        s, np.ones_like(s, dtype=bool), vpg)
                s = scale * (q[b, :, h, :] @ ktg.T)
                o_t[b, :, h, :], lse_t[b, h, :] = _masked_softmax_rows(
                    s, anc[b], vtg)
    # lse is [B,Hq,T]; o is [B,T,Hq,D] -> bring o to [B,Hq,T,D] for the merge
    parts = [(np.transpose(o_p, (0, 2, 1, 3)), lse_p),
             (np.transpose(o_t, (0, 2, 1, 3)), lse_t)]
    o_m, lse_m = lse_merge(parts)
    return ((o_p, lse_p), (o_t, lse_t),
            (np.transpose(o_m, (0, 2, 1, 3)), lse_m))


# --------------------------------------------------------------------------
# Draft cross-attention into the target's KV cache ([GIST-2A])
# --------------------------------------------------------------------------

def oracle_prefix_attn(q, k_prefix, v_prefix, offsets, scale):
    """Attention of T query tokens over the prefix keys alone, no mask.

    gist.science page, section 2 "Methodik", part A, item "Cross-Attention mit
    geteiltem KV-Cache": the draft model attends directly to the target
    model's KV cache.  q [B,T,Hq,D]; k_prefix, v_prefix [sum L_b, Hkv, D]
    packed by `offsets` [B+1].  Returns fp64 o [B,T,Hq,D] and lse [B,Hq,T]
    (natural log).  A sequence without prefix keys (L_b = 0) has an empty
    softmax: o = 0 and lse = -inf (the reading of the empty cached part in
    [GIST-2C], taken here for the whole call).
    """
    q = _f64(q)
    kp, vp = _f64(k_prefix), _f64(v_prefix)
    B, T, Hq, D = q.shape
    Hkv = kp.shape[1]
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    G = Hq // Hkv
    off = np.asarray(offsets, dtype=np.int64)
    if off.shape != (B + 1,) or off[0] != 0 or np.any(np.diff(off) < 0):
        raise ValueError("offsets must be [B+1], start at 0 and not decrease")
    o = np.zeros((B, T, Hq, D))
    lse = np.full((B, Hq, T), -np.inf)
    for b in range(B):
        if off[b + 1] == off[b]:
            continue
        for h in range(Hq):
            keys = kp[off[b]:off[b + 1], h // G, :]
            vals = vp[off[b]:off[b + 1], h // G, :]
            s = (q[b, :, h, :] @ keys.T) * scale          # [T, L_b]
            o[b, :, h, :], lse[b, h, :] = _masked_softmax_rows(
                s, np.ones_like(s, dtype=bool), vals)
    return o, lse


# --------------------------------------------------------------------------
# Paged prefix cache
# --------------------------------------------------------------------------

def gather_paged(pages, block_table, seq_lens, page_size):
    """The packed prefix layout of a paged cache.

    A paged cache keeps the prefix keys (or values) of every sequence in
    fixed-size pages of a shared pool: pages [num_pages, page_size, Hkv, D].
    Key j of sequence b lives in page block_table[b, j // page_size] at row
    j % page_size.  Returns (packed [sum L_b, Hkv, D], offsets [B+1]), the
    layout `oracle_attn` takes, so paged attention is attention over the
    gathered keys.  Raises on a page index outside the pool.
    """
    pages = np.asarray(pages)
    bt = np.asarray(block_table, dtype=np.int64)
    lens = np.asarray(seq_lens, dtype=np.int64)
    B = lens.shape[0]
    rows = []
    for b in range(B):
        for j in range(int(lens[b])):
            page = int(bt[b, j // page_size])
            if not 0 <= page < pages.shape[0]:
                raise ValueError(f"sequence {b}: page {page} outside the pool")
            rows.append(pages[page, j % page_size])
    off = np.zeros(B + 1, dtype=np.int64)
    off[1:] = np.cumsum(lens)
    packed = np.stack(rows) if rows else np.zeros((0,) + pages.shape[2:], dtype=pages.dtype)
    return packed, off


# --------------------------------------------------------------------------
# Strided prefix cache
# --------------------------------------------------------------------------

def gather_strided(buf, offsets, row_stride, Hkv, D):
    """The packed prefix layout of a cache whose key rows are not packed.

    buf is a flat array; key j of sequence b, KV head g, feature d is
    buf[(offsets[b] + j) * row_stride + g * D + d] (an interleaved K/V cache,
    or rows padded past Hkv * D).  Returns packed [offsets[-1], Hkv, D], the
    layout `oracle_attn` takes, so attention over a strided cache is attention
    over the gathered rows.  Raises when a row reaches past the buffer or the
    stride is shorter than a row.
    """
    flat = np.asarray(buf).reshape(-1)
    off = np.asarray(offsets, dtype=np.int64)
    rows = int(off[-1])
    if row_stride < Hkv * D:
        raise ValueError("row stride shorter than Hkv * D")
    out = np.empty((rows, Hkv, D), dtype=flat.dtype)
    for r in range(rows):
        start = r * row_stride
        if start + Hkv * D > flat.size:
            raise ValueError(f"row {r} reaches past the buffer")
        for g in range(Hkv):
            out[r, g, :] = flat[start + g * D: start + g * D + D]
    return out


# --------------------------------------------------------------------------
# Draft sliding-window self-attention over a draft tree ([GIST-2AW])
# --------------------------------------------------------------------------

def oracle_window_attn(q, k_cache, v_cache, offsets, k_tree, v_tree, parent, scale, window):
    """Sliding-window self-attention of the draft's tree tokens.

    Positions: key k of sequence b's draft cache (k = 0 .. L_b-1, packed by
    `offsets` [B+1], the last one the token just before the tree) is at
    position k; tree node i is at position L_b + depth(i) - 1 on its own
    branch (the position reading of the tree's rotary embedding).  Row i sees
    a key iff the key lies on its branch (every cache key does; a tree key iff
    it is in anc*(i)) and its position p obeys pos(i) - window < p <= pos(i)
    ([GIST-2AW]: a window of the most recent tokens).  q [B,T,Hq,D];
    k_cache, v_cache [sum L_b, Hkv, D]; k_tree, v_tree [B,T,Hkv,D];
    parent [B,T]; window >= 1.  Returns fp64 o [B,T,Hq,D], lse [B,Hq,T].
    """
    if int(window) < 1:
        raise ValueError("window must be at least 1")
    q = _f64(q)
    kc, vc, kt, vt = _f64(k_cache), _f64(v_cache), _f64(k_tree), _f64(v_tree)
    B, T, Hq, Hkv, D, G, off = _shapes(q, kt, offsets)
    anc = ancestor_matrix(parent)
    depth = anc.sum(axis=2)
    o = np.empty((B, T, Hq, D))
    lse = np.empty((B, Hq, T))
    for b in range(B):
        L = int(off[b + 1] - off[b])
        qpos = L + depth[b] - 1                                    # [T]
        kpos = np.concatenate([np.arange(L), L + depth[b] - 1])    # [L + T]
        on_branch = np.ones((T, L + T), dtype=bool)
        on_branch[:, L:] = anc[b]
        in_window = (kpos[None, :] <= qpos[:, None]) & (kpos[None, :] > qpos[:, None] - window)
        visible = on_branch & in_window
        for g in range(Hkv):
            keys = np.concatenate([kc[off[b]:off[b + 1], g, :], kt[b, :, g, :]])
            vals = np.concatenate([vc[off[b]:off[b + 1], g, :], vt[b, :, g, :]])
            for h in range(g * G, (g + 1) * G):
                s = (q[b, :, h, :] @ keys.T) * scale        # [T, L_b + T]
                o[b, :, h, :], lse[b, h, :] = _masked_softmax_rows(s, visible, vals)
    return o, lse


# --------------------------------------------------------------------------
# KV-cache commit of the accepted draft tokens ([GIST-INTRO], [GIST-3])
# --------------------------------------------------------------------------

def oracle_commit_kv(k_tree, v_tree, accepted, n_accepted, dst_row, k_cache, v_cache):
    """Copy the K/V rows of the accepted tree nodes into the cache.

    For every sequence b whose arguments are in range, and j < n_accepted[b]:
    cache row dst_row[b] + j takes tree row accepted[b, j] (all KV heads).
    k_tree, v_tree [B,T,Hkv,D]; accepted [B,T] int; n_accepted, dst_row [B];
    k_cache, v_cache [rows, Hkv, D] (not modified: copies are returned).

    Returns (k_cache', v_cache', status) with status 0, or 1 + the first
    sequence b with n_accepted[b] outside [0, T], an accepted id outside
    [0, T) among its first n_accepted[b] entries, or a destination range
    outside [0, rows); such a sequence is left unwritten.
    """
    kt, vt = np.asarray(k_tree), np.asarray(v_tree)
    acc = np.asarray(accepted)
    n_acc, dst = np.asarray(n_accepted), np.asarray(dst_row)
    kc, vc = np.array(k_cache, copy=True), np.array(v_cache, copy=True)
    B, T = acc.shape
    rows = kc.shape[0]
    status = 0
    for b in range(B):
        n, d = int(n_acc[b]), int(dst[b])
        ok = 0 <= n <= T and 0 <= d and d + n <= rows
        ok = ok and all(0 <= int(acc[b, j]) < T for j in range(n))
        if not ok:
            if status == 0:
                status = 1 + b
            continue
        for j in range(n):
            kc[d + j] = kt[b, int(acc[b, j])]
            vc[d + j] = vt[b, int(acc[b, j])]
    return kc, vc, status


# --------------------------------------------------------------------------
# Rotary position embedding at tree positions ([GIST-1P], [MLS-REF])
# --------------------------------------------------------------------------

def oracle_tree_rope(q, k_tree, parent, offsets, base):
    """Rotate the tree tokens' queries and keys to their tree positions.

    Node i of sequence b sits at p = L_b + depth(i) - 1 (a token continues the
    prefix along its own branch; root depth 1).  Channel pairs (k, k + D/2),
    k < D/2, are rotated by p * base^(-2k/D): written here as the complex
    product (x[k] + i x[k + D/2]) * exp(i p theta_k).  q [B,T,Hq,D],
    k_tree [B,T,Hkv,D]; returns fp64 copies (unrounded).
    """
    q = _f64(q).copy()
    kt = _f64(k_tree).copy()
    B, T, Hq, D = q.shape
    off = np.asarray(offsets, dtype=np.int64)
    depth = tree_depth(parent)                        # [B, T]
    half = D // 2
    theta = np.power(float(base), -2.0 * np.arange(half) / D)
    for b in range(B):
        L = int(off[b + 1] - off[b])
        for i in range(T):
            rot = np.exp(1j * (L + depth[b, i] - 1) * theta)          # [D/2]
            for x in (q[b, i], kt[b, i]):                             # [H, D] views
                z = (x[:, :half] + 1j * x[:, half:]) * rot
                x[:, :half], x[:, half:] = z.real, z.imag
    return q, kt


def round_bf16(x):
    """fp64 values rounded to the nearest bf16 value (8 significant bits, ties
    to even), returned as fp64."""
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)                                # x = m 2^e, 0.5 <= |m| < 1
    return np.ldexp(np.rint(m * 256.0) / 256.0, e)    # np.rint: ties to even
