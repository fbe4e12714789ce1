"""Seeded synthetic inputs for tree-verification attention.

This module only draws random numbers and shapes them into input tensors; it
holds none of the attention arithmetic.  Both the HIP path (through the tests,
the benchmark and the smoke check) and the fp64 oracle consume what it makes.

Workloads stand in for the long-context and long-reasoning runs of the LongSpec
pages (gist.science explainer, section 3 "Wichtige Ergebnisse": summarisation
and code-completion sets, math reasoning with QwQ-32B at up to 32k tokens;
mean accepted length about 3.5 to 4 tokens per step), whose datasets and model
weights are not available.  Shapes follow the attention layers of the named
model families (Llama-3-8B: 32 query heads / 8 KV heads / head_dim 128;
QwQ-32B: 40 / 8 / 128); values are N(0, 1).

Recipe (fixed):

* config k draws from ``numpy.random.default_rng(1000 + k)``;
* draw order: the tree(s), then q, k_prefix, v_prefix, k_tree, v_tree, each
  ``standard_normal(dtype=float32)``; then, if asked, the outlier rows;
* bf16 workloads round the fp32 draws to bf16 with round-to-nearest-even
  (``torch.Tensor.to(torch.bfloat16)``);
* outlier rows: ``round(frac * L)`` prefix positions chosen without
  replacement; K and V of those positions (all KV heads) are multiplied by 8
  before rounding (exact in bf16);
* trees: "uniform" gives parent[0] = -1 and parent[i] uniform in [0, i-1];
  "bounded(dmax, bmax)" gives node 0 as root and each later node a parent
  chosen uniformly among earlier nodes with depth < dmax and fewer than bmax
  children (depth counts nodes from the root, root = 1); "chain" gives
  parent[i] = i - 1; "star" gives parent[i] = 0.
"""

from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np
import torch

__all__ = ["CONFIGS", "Workload", "make_tree", "make_workload", "make_config"]


def make_tree(rng: np.random.Generator, T: int, kind) -> np.ndarray:
    """int32 parent array [T] of one speculation tree (see module recipe)."""
    parent = np.full(T, -1, dtype=np.int32)
    if T == 0:
        return parent
    if kind == "uniform":
        for i in range(1, T):
            parent[i] = rng.integers(0, i)
    elif kind == "chain":
        parent[1:] = np.arange(T - 1, dtype=np.int32)
    elif kind == "star":
        parent[1:] = 0
    elif kind == "forest":
        # several roots: every node picks uniformly among -1 and earlier nodes
        for i in range(1, T):
            parent[i] = rng.integers(-1, i)
    elif isinstance(kind, tuple) and kind[0] == "bounded":
        _, dmax, bmax = kind
        depth = np.zeros(T, dtype=np.int64)
        children = np.zeros(T, dtype=np.int64)
        depth[0] = 1
        for i in range(1, T):
            cand = [j for j in range(i) if depth[j] < dmax and children[j] < bmax]
            if not cand:
                raise ValueError("tree bounds too tight for T nodes")
            j = cand[int(rng.integers(0, len(cand)))]
            parent[i] = j
            depth[i] = depth[j] + 1
            children[j] += 1
    else:
        raise ValueError(f"unknown tree kind {kind!r}")
    return parent


@dataclass
class Workload:
    """Inputs of one tree-verification attention call (CPU tensors)."""
    name: str
    dtype: str                      # "bf16" or "f32"
    q: torch.Tensor                 # [B, T, Hq, D]
    k_prefix: torch.Tensor          # [sum L_b, Hkv, D]
    v_prefix: torch.Tensor          # [sum L_b, Hkv, D]
    offsets: torch.Tensor           # int32 [B + 1]
    k_tree: torch.Tensor            # [B, T, Hkv, D]
    v_tree: torch.Tensor            # [B, T, Hkv, D]
    parent: torch.Tensor            # int32 [B, T]
    scale: float
    prefix_lens: list = field(default_factory=list)

    @property
    def shape(self):
        B, T, Hq, D = self.q.shape
        return dict(B=B, T=T, Hq=Hq, Hkv=self.k_tree.shape[2], D=D,
                    max_prefix_len=max(self.prefix_lens) if self.prefix_lens else 0)


def make_workload(rng: np.random.Generator, *, B, T, Hq, Hkv, D, prefix_lens,
                  trees, dtype="bf16", scale=None, outlier_frac=0.0,
                  name="custom") -> Workload:
    """Draw one workload in the fixed order of the module recipe.

    `trees` is one tree kind for every sequence or a list of B kinds."""
    if not isinstance(trees, list):
        trees = [trees] * B
    assert len(trees) == B and len(prefix_lens) == B
    parent = np.stack([make_tree(rng, T, k) for k in trees]).astype(np.int32)
    total = int(sum(prefix_lens))
    f32 = np.float32
    q = rng.standard_normal((B, T, Hq, D), dtype=f32)
    kp = rng.standard_normal((total, Hkv, D), dtype=f32)
    vp = rng.standard_normal((total, Hkv, D), dtype=f32)
    kt = rng.standard_normal((B, T, Hkv, D), dtype=f32)
    vt = rng.standard_normal((B, T, Hkv, D), dtype=f32)
    if outlier_frac > 0 and total > 0:
        n_out = int(round(outlier_frac * total))
        rows = rng.choice(total, size=n_out, replace=False)
        kp[rows] *= 8.0
        vp[rows] *= 8.0
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    conv = lambda a: torch.from_numpy(a).to(tdt)  # noqa: E731  (RNE to bf16)
    offsets = np.zeros(B + 1, dtype=np.int32)
    offsets[1:] = np.cumsum(prefix_lens)
    return Workload(
        name=name, dtype=dtype, q=conv(q), k_prefix=conv(kp), v_prefix=conv(vp),
        offsets=torch.from_numpy(offsets), k_tree=conv(kt), v_tree=conv(vt),
        parent=torch.from_numpy(parent),
        scale=float(scale if scale is not None else 1.0 / np.sqrt(D)),
        prefix_lens=list(int(x) for x in prefix_lens))


# The five workloads: a tiny fp32 correctness case, Llama-3-8B-shaped layers at
# 16k and 128k prefixes, the QwQ-32B-shaped layer at 32k with outlier rows
# (the headline), and a ragged batch of four prefixes with T = 32 trees.
CONFIGS = {
    1: dict(name="tiny-fp32-h4-d64-L512-T8", B=1, T=8, Hq=4, Hkv=4, D=64,
            prefix_lens=[512], trees="uniform", dtype="f32"),
    2: dict(name="llama3-8b-gqa32/8-d128-L16k-T64", B=1, T=64, Hq=32, Hkv=8,
            D=128, prefix_lens=[16384], trees=("bounded", 6, 4), dtype="bf16"),
    3: dict(name="llama3-8b-gqa32/8-d128-L128k-T64", B=1, T=64, Hq=32, Hkv=8,
            D=128, prefix_lens=[131072], trees=("bounded", 6, 4), dtype="bf16"),
    4: dict(name="qwq32b-gqa40/8-d128-L32k-T64", B=1, T=64, Hq=40, Hkv=8,
            D=128, prefix_lens=[32768], trees=("bounded", 8, 3), dtype="bf16",
            outlier_frac=0.01),
    5: dict(name="ragged-b4-gqa32/8-d128-L8k/32k/64k/128k-T32", B=4, T=32,
            Hq=32, Hkv=8, D=128, prefix_lens=[8192, 32768, 65536, 131072],
            trees=["chain"] + [("bounded", 6, 4)] * 3, dtype="bf16"),
}


def make_config(k: int, seed: int | None = None) -> Workload:
    """Workload of config k (1..5), drawn from default_rng(1000 + k)."""
    spec = dict(CONFIGS[k])
    rng = np.random.default_rng(1000 + k if seed is None else seed)
    return make_workload(rng, **spec)
