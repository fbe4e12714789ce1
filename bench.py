"""Benchmark of hybrid tree-verification attention on one MI355X.

One step = one ltree_attn call (prefix splits + tree part, then the
log-sum-exp merge) over the QwQ-32B-shaped layer: batch 1, 40 query heads /
8 KV heads, head_dim 128, prefix 32768, a 64-node draft tree (depth <= 8,
branching <= 3), bf16 inputs with 1% of prefix rows scaled x8.  Inputs are
seeded synthetic data resident in HBM.  Each step reads a different one of
several copies of the prefix KV cache, together larger than the 256 MB
Infinity Cache, so every step streams its keys from HBM (cold-cache timing).

Prints one JSON line.  The throughput `value` is algorithmic TFLOP/s of the
whole call (wall clock over the timed steps, launched as one HIP graph;
`us_per_call_eager` gives the same steps launched call by call); `roofline`
rates the dominant kernel (the partial-attention kernel) against the bf16
MFMA peak, with its duration taken from HIP events recorded on the launch
stream around replays of a graph of K launches of it on the same rotating
inputs (median over the replays).  `us_per_call_spread` adds the median and
minimum per call over further replays of the timed graph, and the same steps
over a single KV copy that stays in the Infinity Cache (hot cache, labelled).
`cpu_baseline` times the fp64 oracle on a bounded sample of the same workload
on the host cores.

`--row NAME` measures one of the steps around the verification path instead
(the draft's cross-attention into the target cache, its sliding-window
self-attention, verification of a 256-node tree, verification over a paged
cache, the KV-cache commit, the tree rotary embedding, one GPU's share of the
layer under 8-way sharding) and prints that row's own JSON line.

The default warm-up (1000 untimed steps, about 75 ms) lets the GPU settle
at its sustained clocks; with 10 warm-up steps the timed steps run about 15%
slower than the same steps a few tens of milliseconds later.

    python bench.py [--gpus 1] [--steps 50] [--warmup 1000] [--config 4]
    python bench.py --row {xattn,window,bigtree,paged,commit,rope,shard}
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16/fp16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
REPS = 7                    # extra replays of the timed graphs for median / minimum
METRIC = "tree-verify attn µs/call + TFLOP/s @L=32k,T=64; % MFMA / HBM roofline"
KERNEL_SOURCES = ["attn_partial_mfma_impl.h", "attn_partial_mfma.hip", "ltree_api.hip",
                  "ltree_internal.h", "ltree_plan.cpp", "ltree_plan.h"]
# HBM traffic records (rocprofv3 FETCH_SIZE / WRITE_SIZE of the partial kernel),
# one per benchmark workload; written by --traffic-summary
TRAFFIC_SLUG = {2: "llama3_8b_L16k_T64", 3: "llama3_8b_L128k_T64", 4: "qwq32b_L32k_T64",
                5: "ragged_b4_L8k_128k_T32"}


def traffic_file(config: int) -> str:
    return os.path.join(ROOT, "profiles", f"traffic_partials_{TRAFFIC_SLUG.get(config, config)}.json")


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def kernel_hash() -> str:
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "tree_attention_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def depth_sum(parent_row) -> int:
    """Number of (node, visible tree node) pairs = sum of depths."""
    depth = []
    for i, p in enumerate(parent_row):
        depth.append(1 if p < 0 else depth[p] + 1)
    return sum(depth)


def algorithmic_counts(w):
    """FLOP and HBM bytes the method must move/compute (no split-K partials)."""
    B, T, Hq, D = w.q.shape
    Hkv = w.k_tree.shape[2]
    e = w.q.element_size()
    sum_l = sum(w.prefix_lens)
    anc = sum(depth_sum(w.parent[b].tolist()) for b in range(B))
    flop_prefix = 4 * D * Hq * T * sum_l
    flop_tree = 4 * D * Hq * anc
    W = (T + 63) // 64  # mask words per row
    bytes_ = (2 * sum_l * Hkv * D * e + B * T * Hq * D * e + 2 * B * T * Hkv * D * e
              + B * T * W * 8 + B * T * Hq * D * 4 + B * Hq * T * 4 + 4 * (B + 1))
    # the partial kernel reads q, prefix K/V, tree K/V and the mask
    bytes_partials = (2 * sum_l * Hkv * D * e + B * T * Hq * D * e + 2 * B * T * Hkv * D * e
                      + B * T * W * 8)
    return flop_prefix + flop_tree, bytes_, bytes_partials


def cpu_baseline(w, budget_s=15.0, min_s=10.0):
    """fp64 oracle on the same workload, one KV head (with its query heads) at
    a time, for about `budget_s` seconds: as many heads as fit, and when the
    whole layer takes less than `min_s`, whole passes over it repeated until
    `min_s` have gone by (at least one head)."""
    import numpy as np
    from threadpoolctl import threadpool_info

    import oracle

    B, T, Hq, D = w.q.shape
    Hkv = w.k_tree.shape[2]
    G = Hq // Hkv
    parent = w.parent.numpy()
    off = w.offsets.numpy()
    head_flop = 4 * D * G * T * sum(w.prefix_lens) + 4 * D * G * sum(
        depth_sum(parent[b].tolist()) for b in range(B))
    heads, flop, t_total, next_log = 0, 0, 0.0, 0.0
    while heads == 0 or (t_total < budget_s and (heads % Hkv != 0 or t_total < min_s)):
        g = heads % Hkv
        sl = slice(g, g + 1)
        t0 = time.perf_counter()
        oracle.oracle_attn(w.q[:, :, g * G:(g + 1) * G], w.k_prefix[:, sl], w.v_prefix[:, sl],
                           off, w.k_tree[:, :, sl], w.v_tree[:, :, sl], parent, w.scale)
        t_total += time.perf_counter() - t0
        heads += 1
        flop += head_flop
        if t_total >= next_log:  # a progress line every few seconds
            log(f"cpu oracle: {heads} KV-head evaluations ({heads / Hkv:.2f} layers), "
                f"{t_total:.1f} s")
            next_log = t_total + 3.0
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    passes = heads / Hkv
    what = (f"{heads // Hkv} full passes over the layer" if heads % Hkv == 0
            else f"{heads} of {Hkv} KV heads")
    return {
        "value": round(flop / t_total / 1e12, 6),
        "unit": "TFLOP/s",
        "cores": int(threads),
        "kind": "oracle",
        "cpu_model": cpu_model(),
        "sample": f"fp64 NumPy oracle, {what} ({passes:.2f} x {Hkv} KV heads, {Hq} query heads, "
                  f"all {T} tree rows, full {sum(w.prefix_lens)}-key prefix), {t_total:.2f} s "
                  f"wall; NumPy on {threads} BLAS threads",
    }


def cpu_model() -> str:
    """The host CPU's model name (first processor in /proc/cpuinfo)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def time_graph(fn, K):
    """Microseconds per call of fn(s) (s = 0..K-1), K calls captured in one HIP
    graph, after an untimed replay."""
    import torch
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for s in range(K):
            fn(s)
    g.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    g.replay()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) * 1e6 / K


def row_xattn(args):
    """Draft cross-attention into the target's KV cache: the 64 query tokens of
    the QwQ-shaped layer over its 32768-key prefix, no tree part
    (ltree_prefix_attn; split-K partials + merge, the same kernels)."""
    import math

    import torch

    import tree_attention_amd as ta
    from workloads import make_config

    w = make_config(4)
    dev = "cuda:0"
    B, T, Hq, D = w.q.shape
    Hkv = w.k_prefix.shape[1]
    e = w.q.element_size()
    L = sum(w.prefix_lens)
    q, off = w.q.to(dev), w.offsets.to(dev)
    kv_bytes = 2 * w.k_prefix.numel() * e
    n = max(2, math.ceil(512e6 / kv_bytes))
    kp0, vp0 = w.k_prefix.to(dev), w.v_prefix.to(dev)
    kv = [(kp0, vp0)] + [(kp0.clone(), vp0.clone()) for _ in range(n - 1)]
    o = torch.empty((B, T, Hq, D), dtype=torch.float32, device=dev)
    lse = torch.empty((B, Hq, T), dtype=torch.float32, device=dev)
    ws = torch.empty((ta.ltree_attn_workspace_bytes(B, T, Hq, Hkv, D, L),), dtype=torch.uint8,
                     device=dev)

    def call(s):
        kp, vp = kv[s % n]
        return ta.ltree_prefix_attn(q, kp, vp, off, L, o, lse, ws, w.scale)

    for s in range(args.warmup):
        assert call(s) == 0
    torch.cuda.synchronize()
    us = time_graph(call, args.steps)
    assert torch.isfinite(o).all() and torch.isfinite(lse).all()
    flop = 4 * D * Hq * T * L
    bytes_ = 2 * L * Hkv * D * e + B * T * Hq * D * e + B * T * Hq * D * 4 + B * Hq * T * 4
    tflops = flop / (us * 1e-6) / 1e12
    return {
        "metric": "draft cross-attention into the target KV cache, µs/call + TFLOP/s",
        "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(us / 1000, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded N(0,1), 1% of prefix rows x8)",
        "config": {"workload": "draft-xattn-qwq32b-gqa40/8-d128-L32k-T64", "B": B, "T": T,
                   "Hq": Hq, "Hkv": Hkv, "D": D, "prefix_lens": w.prefix_lens,
                   "cache": f"cold ({n} rotating KV copies)"},
        "us_per_call": round(us, 2),
        "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tflops / PEAK_BF16_TFLOPS, 4),
                     "traffic": None,
                     "hbm_frac": round(bytes_ / (us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4)},
    }


def row_shard(args):
    """One GPU's share of the QwQ-shaped layer when the layer is sharded over
    8 GPUs: KV-head (tensor) parallel, one KV head with its 5 query heads over
    the whole 32768-key prefix; context parallel, all heads over the last
    4096 prefix keys with the tree (the shard that holds the tree; the others
    run the same call without it).  Each share is one ltree_attn call on this
    GPU, graph-timed over rotating KV copies; the exchange between GPUs (none
    for KV heads, one all-gather of the partials for the context split) is
    not part of it."""
    import math

    import torch

    import tree_attention_amd as ta
    from workloads import make_config

    w = make_config(4)
    dev = "cuda:0"
    B, T, Hq, D = w.q.shape
    Hkv = w.k_prefix.shape[1]
    G = Hq // Hkv
    e = w.q.element_size()
    mask_all = None
    out = {}
    shares = {
        "kv_head_share": dict(q=w.q[:, :, :G], kp=w.k_prefix[:, :1], vp=w.v_prefix[:, :1],
                              kt=w.k_tree[:, :, :1], vt=w.v_tree[:, :, :1],
                              L=sum(w.prefix_lens)),
        "context_share": dict(q=w.q, kp=w.k_prefix[-4096:], vp=w.v_prefix[-4096:], kt=w.k_tree,
                              vt=w.v_tree, L=4096),
    }
    for name, sh in shares.items():
        q = sh["q"].contiguous().to(dev)
        kt, vt = sh["kt"].contiguous().to(dev), sh["vt"].contiguous().to(dev)
        L = sh["L"]
        hq, hkv = q.shape[2], kt.shape[2]
        off = torch.tensor([0, L], dtype=torch.int32, device=dev)
        kv_bytes = 2 * L * hkv * D * e
        n = max(2, math.ceil(512e6 / kv_bytes))
        kp0, vp0 = sh["kp"].contiguous().to(dev), sh["vp"].contiguous().to(dev)
        kv = [(kp0, vp0)] + [(kp0.clone(), vp0.clone()) for _ in range(n - 1)]
        if mask_all is None:
            mask_all, _ = ta.build_mask(w.parent.to(dev))
        o = torch.empty((B, T, hq, D), dtype=torch.float32, device=dev)
        lse = torch.empty((B, hq, T), dtype=torch.float32, device=dev)
        ws = ta.workspace_for(q, kt, L)

        def call(s):
            kp, vp = kv[s % n]
            return ta.ltree_attn(q, kp, vp, off, L, kt, vt, mask_all, o, lse, ws, w.scale)

        for s in range(args.warmup):
            assert call(s) == 0
        torch.cuda.synchronize()
        us = time_graph(call, args.steps)
        assert torch.isfinite(o).all() and torch.isfinite(lse).all()
        anc = depth_sum(w.parent[0].tolist())
        flop = 4 * D * hq * T * L + 4 * D * hq * anc
        bytes_ = (2 * L * hkv * D * e + B * T * hq * D * e + 2 * B * T * hkv * D * e
                  + B * T * hq * D * 4 + B * hq * T * 4)
        tflops = flop / (us * 1e-6) / 1e12
        out[name] = {"Hq": hq, "Hkv": hkv, "prefix_len": L, "us_per_call": round(us, 2),
                     "tflops": round(tflops, 2), "mfma_frac": round(tflops / PEAK_BF16_TFLOPS, 4),
                     "hbm_frac": round(bytes_ / (us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4),
                     "cache": f"cold ({n} rotating KV copies)"}
    kvs = out["kv_head_share"]
    return {
        "metric": "one GPU's share of the QwQ-shaped layer under 8-way sharding, µs/call + TFLOP/s",
        "value": kvs["tflops"], "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(kvs["us_per_call"] / 1000, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded N(0,1), 1% of prefix rows x8)",
        "config": {"workload": "shard-of-qwq32b-gqa40/8-d128-L32k-T64", "B": B, "T": T, "D": D,
                   "shares": "KV head 0 (value); last 4096 prefix keys"},
        **out,
        "roofline": {"bound": "mfma", "achieved": kvs["tflops"], "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": kvs["mfma_frac"], "traffic": None,
                     "hbm_frac": kvs["hbm_frac"]},
    }


def row_window(args):
    """Draft sliding-window self-attention over the QwQ-shaped 64-node tree:
    window 512 after a 32768-row cache, of which the last 511 rows are visible
    (ltree_window_attn; split-K partials + merge, the same kernels)."""
    import math

    import numpy as np
    import torch

    import tree_attention_amd as ta
    from workloads import make_config

    W = 512
    w = make_config(4)
    dev = "cuda:0"
    B, T, Hq, D = w.q.shape
    Hkv = w.k_prefix.shape[1]
    e = w.q.element_size()
    L = sum(w.prefix_lens)
    q, off = w.q.to(dev), w.offsets.to(dev)
    kt, vt = w.k_tree.to(dev), w.v_tree.to(dev)
    mask, _ = ta.build_mask(w.parent.to(dev))
    # rotating copies of the rows the window reads (the last W - 1 of the
    # cache, as the cache of a sequence of that length) keep every call cold
    kw, vw = w.k_prefix[L - (W - 1):], w.v_prefix[L - (W - 1):]
    offw = torch.tensor([0, W - 1], dtype=torch.int32, device=dev)
    win_bytes = 2 * kw.numel() * e
    n = max(2, math.ceil(512e6 / win_bytes))
    kv = [(kw.to(dev), vw.to(dev)) for _ in range(n)]
    o = torch.empty((B, T, Hq, D), dtype=torch.float32, device=dev)
    lse = torch.empty((B, Hq, T), dtype=torch.float32, device=dev)
    ws = torch.empty((ta.ltree_window_attn_workspace_bytes(B, T, Hq, Hkv, D, W),),
                     dtype=torch.uint8, device=dev)

    def call(s):
        kc, vc = kv[s % n]
        return ta.ltree_window_attn(q, kc, vc, offw, kt, vt, mask, o, lse, ws, w.scale, W)

    for s in range(args.warmup):
        assert call(s) == 0
    torch.cuda.synchronize()
    us = time_graph(call, args.steps)
    # the same result as over the full cache
    assert ta.ltree_window_attn(q, w.k_prefix.to(dev), w.v_prefix.to(dev), off, kt, vt, mask,
                                o, lse, ws, w.scale, W) == 0
    torch.cuda.synchronize()
    assert torch.isfinite(o).all() and torch.isfinite(lse).all()
    # keys seen by node i: min(W, L + depth(i)), depth = popcount of its mask row
    depth = np.array([bin(int(x) & (2**64 - 1)).count("1") for x in mask.cpu().view(-1).tolist()])
    visible = int(np.minimum(W, L + depth).sum())
    flop = 4 * D * Hq * visible
    bytes_ = (win_bytes + B * T * Hq * D * e + 2 * B * T * Hkv * D * e + B * T * 8
              + B * T * Hq * D * 4 + B * Hq * T * 4 + 4 * (B + 1))
    tflops = flop / (us * 1e-6) / 1e12
    gbs = bytes_ / (us * 1e-6) / 1e9
    return {
        "metric": "draft sliding-window self-attention over the tree, µs/call + TFLOP/s",
        "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(us / 1000, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded N(0,1), 1% of cache rows x8)",
        "config": {"workload": "draft-window512-qwq32b-gqa40/8-d128-T64", "B": B, "T": T,
                   "Hq": Hq, "Hkv": Hkv, "D": D, "window": W, "cache_len": L,
                   "cache": f"cold ({n} rotating copies of the window rows)"},
        "us_per_call": round(us, 2),
        "roofline": {"bound": "hbm", "achieved": round(gbs, 2), "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 6), "traffic": None,
                     "note": f"{bytes_ / 1e6:.2f} MB and {flop / 1e9:.3f} GFLOP per call: "
                             "launch- and latency-bound"},
    }


def row_bigtree(args):
    """Verification of a 256-node tree (depth <= 12, branching <= 3; four mask
    words per row) on the QwQ-shaped layer: prefix 32768, 40/8 heads, D 128,
    1% of prefix rows x8 (ltree_attn; the partial kernel's multi-tile tree
    variant, 1280 query rows per KV head in four row blocks)."""
    import math

    import numpy as np
    import torch

    import tree_attention_amd as ta
    from workloads import make_workload

    rng = np.random.default_rng(2024)
    w = make_workload(rng, B=1, T=256, Hq=40, Hkv=8, D=128, prefix_lens=[32768],
                      trees=("bounded", 12, 3), dtype="bf16", outlier_frac=0.01,
                      name="qwq32b-gqa40/8-d128-L32k-T256")
    dev = "cuda:0"
    B, T, Hq, D = w.q.shape
    L = sum(w.prefix_lens)
    q, off = w.q.to(dev), w.offsets.to(dev)
    kt, vt = w.k_tree.to(dev), w.v_tree.to(dev)
    mask, status = ta.build_mask(w.parent.to(dev))
    kv_bytes = 2 * w.k_prefix.numel() * w.q.element_size()
    n = max(2, math.ceil(512e6 / kv_bytes))
    kp0, vp0 = w.k_prefix.to(dev), w.v_prefix.to(dev)
    kv = [(kp0, vp0)] + [(kp0.clone(), vp0.clone()) for _ in range(n - 1)]
    o = torch.empty((B, T, Hq, D), dtype=torch.float32, device=dev)
    lse = torch.empty((B, Hq, T), dtype=torch.float32, device=dev)
    ws = ta.workspace_for(q, kt, L)

    def call(s):
        kp, vp = kv[s % n]
        return ta.ltree_attn(q, kp, vp, off, L, kt, vt, mask, o, lse, ws, w.scale)

    for s in range(args.warmup):
        assert call(s) == 0
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    us = time_graph(call, args.steps)
    assert torch.isfinite(o).all() and torch.isfinite(lse).all()
    flop, bytes_, _ = algorithmic_counts(w)
    tflops = flop / (us * 1e-6) / 1e12
    return {
        "metric": "tree-verify attn with a 256-node tree, µs/call + TFLOP/s",
        "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(us / 1000, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded N(0,1), 1% of prefix rows x8)",
        "config": {"workload": "qwq32b-gqa40/8-d128-L32k-T256", "B": B, "T": T, "Hq": Hq,
                   "Hkv": 8, "D": D, "prefix_lens": w.prefix_lens,
                   "cache": f"cold ({n} rotating KV copies)"},
        "us_per_call": round(us, 2),
        "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tflops / PEAK_BF16_TFLOPS, 4),
                     "traffic": None,
                     "hbm_frac": round(bytes_ / (us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4),
                     "note": "whole call (partial kernel + merge)"},
    }


def row_paged(args):
    """Verification over a paged prefix cache: the QwQ-shaped layer (prefix
    32768, 64-node tree, 40/8 heads, D 128, 1% of prefix rows x8) with its
    prefix cut into 256-key pages placed in shuffled order in the page pool
    (ltree_attn_paged)."""
    import math

    import numpy as np
    import torch

    import tree_attention_amd as ta
    from workloads import make_config

    P = 256
    w = make_config(4)
    dev = "cuda:0"
    B, T, Hq, D = w.q.shape
    Hkv = w.k_prefix.shape[1]
    L = sum(w.prefix_lens)
    npages = L // P
    perm = torch.from_numpy(np.random.default_rng(31).permutation(npages)).long()
    # page perm[j] holds keys j*P .. j*P + P - 1
    kpool = torch.empty((npages, P, Hkv, D), dtype=w.k_prefix.dtype)
    vpool = torch.empty_like(kpool)
    kpool[perm] = w.k_prefix.view(npages, P, Hkv, D)
    vpool[perm] = w.v_prefix.view(npages, P, Hkv, D)
    bt = perm.to(torch.int32).view(1, npages).to(dev)
    lens = torch.tensor([L], dtype=torch.int32, device=dev)
    kv_bytes = 2 * w.k_prefix.numel() * w.q.element_size()
    n = max(2, math.ceil(512e6 / kv_bytes))
    pools = [(kpool.to(dev), vpool.to(dev)) for _ in range(n)]
    q, kt, vt = w.q.to(dev), w.k_tree.to(dev), w.v_tree.to(dev)
    mask, _ = ta.build_mask(w.parent.to(dev))
    o = torch.empty((B, T, Hq, D), dtype=torch.float32, device=dev)
    lse = torch.empty((B, Hq, T), dtype=torch.float32, device=dev)
    ws = torch.empty((ta.ltree_attn_paged_workspace_bytes(B, T, Hq, Hkv, D, L, P),),
                     dtype=torch.uint8, device=dev)

    def call(s):
        kp, vp = pools[s % n]
        return ta.ltree_attn_paged(q, kp, vp, bt, lens, L, kt, vt, mask, o, lse, ws, w.scale)

    for s in range(args.warmup):
        assert call(s) == 0
    torch.cuda.synchronize()
    us = time_graph(call, args.steps)
    assert torch.isfinite(o).all() and torch.isfinite(lse).all()
    flop, bytes_, _ = algorithmic_counts(w)
    bytes_ += B * npages * 4 + B * 4          # block table and lengths
    tflops = flop / (us * 1e-6) / 1e12
    return {
        "metric": "tree-verify attn over a paged KV cache, µs/call + TFLOP/s",
        "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(us / 1000, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded N(0,1), 1% of prefix rows x8)",
        "config": {"workload": "qwq32b-gqa40/8-d128-L32k-T64-paged256", "B": B, "T": T,
                   "Hq": Hq, "Hkv": Hkv, "D": D, "prefix_lens": w.prefix_lens, "page_size": P,
                   "cache": f"cold ({n} rotating page pools)"},
        "us_per_call": round(us, 2),
        "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tflops / PEAK_BF16_TFLOPS, 4),
                     "traffic": None,
                     "hbm_frac": round(bytes_ / (us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4),
                     "note": "whole call (partial kernel + merge)"},
    }


def row_commit(args):
    """KV-cache commit of the accepted branch: 4 accepted tokens (about the
    accepted length the pages report) of the QwQ-shaped 64-node tree appended
    after the 32768-row prefix cache (ltree_commit_kv)."""
    import torch

    import tree_attention_amd as ta
    from workloads import make_config

    w = make_config(4)
    dev = "cuda:0"
    B, T, Hkv, D = w.k_tree.shape
    e = w.k_tree.element_size()
    parent = w.parent[0].tolist()
    node = next(i for i in range(T) if sum(1 for _ in _walk(parent, i)) >= 4)
    path = list(_walk(parent, node))[::-1][:4]
    L = w.k_prefix.shape[0]
    kc = torch.zeros((L + T, Hkv, D), dtype=w.k_tree.dtype, device=dev)
    vc = torch.zeros_like(kc)
    kt, vt = w.k_tree.to(dev), w.v_tree.to(dev)
    acc = torch.zeros((B, T), dtype=torch.int32)
    acc[0, :4] = torch.tensor(path, dtype=torch.int32)
    acc = acc.to(dev)
    n_acc = torch.tensor([4], dtype=torch.int32, device=dev)
    dst = torch.tensor([L], dtype=torch.int32, device=dev)
    status = torch.zeros((1,), dtype=torch.int32, device=dev)

    def call(s):
        return ta.ltree_commit_kv(kt, vt, acc, n_acc, dst, kc, vc, status)

    for s in range(args.warmup):
        assert call(s) == 0
    torch.cuda.synchronize()
    us = time_graph(call, args.steps)
    assert int(status.item()) == 0
    bytes_ = 2 * 2 * 4 * Hkv * D * e          # K and V rows, read and written
    gbs = bytes_ / (us * 1e-6) / 1e9
    return {
        "metric": "KV-cache commit of the accepted branch, µs/call",
        "value": round(us, 3), "unit": "us", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(us / 1000, 6), "higher_is_better": False,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "commit-qwq32b-kv8-d128-T64-accept4", "B": B, "T": T, "Hkv": Hkv,
                   "D": D, "accepted": 4, "cache_rows": L + T},
        "us_per_call": round(us, 3),
        "roofline": {"bound": "hbm", "achieved": round(gbs, 2), "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 6), "traffic": None,
                     "note": "32 KB moved per call: launch-latency bound"},
    }


def _walk(parent, i):
    while i != -1:
        yield i
        i = parent[i]


def row_rope(args):
    """Rotary position embedding of the QwQ-shaped tree's queries and keys at
    their tree positions after the 32768-key prefix (ltree_tree_rope)."""
    import torch

    import tree_attention_amd as ta
    from workloads import make_config

    w = make_config(4)
    dev = "cuda:0"
    B, T, Hq, D = w.q.shape
    Hkv = w.k_tree.shape[2]
    e = w.q.element_size()
    q, kt = w.q.to(dev), w.k_tree.to(dev)
    off = w.offsets.to(dev)
    mask, _ = ta.build_mask(w.parent.to(dev))

    def call(s):
        return ta.ltree_tree_rope(q, kt, mask, off, 1e6)

    for s in range(args.warmup):
        assert call(s) == 0
    torch.cuda.synchronize()
    us = time_graph(call, args.steps)
    bytes_ = 2 * B * T * (Hq + Hkv) * D * e + B * T * 8 + 4 * (B + 1)
    gbs = bytes_ / (us * 1e-6) / 1e9
    return {
        "metric": "tree-position RoPE of tree Q/K, µs/call",
        "value": round(us, 3), "unit": "us", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(us / 1000, 6), "higher_is_better": False,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16 (fp64 arithmetic)",
        "data": "synthetic",
        "config": {"workload": "rope-qwq32b-gqa40/8-d128-T64", "B": B, "T": T, "Hq": Hq,
                   "Hkv": Hkv, "D": D, "rope_base": 1e6},
        "us_per_call": round(us, 3),
        "roofline": {"bound": "hbm", "achieved": round(gbs, 2), "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 6), "traffic": None,
                     "note": "786 KB moved per call: launch-latency bound"},
    }


ROWS = {"xattn": row_xattn, "window": row_window, "bigtree": row_bigtree, "paged": row_paged,
        "commit": row_commit, "rope": row_rope, "shard": row_shard}


def _kernel_kind(name: str):
    if "partial_mfma_kernel" in name or "partial_simple_kernel" in name:
        return "partial"
    if "lse_merge_kernel" in name:
        return "merge"
    return None


def _short_name(name: str) -> str:
    """A kernel's name without namespace, return type and parameter list."""
    name = name.replace("void ", "").replace("ltree::(anonymous namespace)::", "")
    return name.split("(")[0]


def _stats(xs):
    if not xs:
        return "-"
    return f"{statistics.mean(xs):.2f} / {min(xs):.2f} / {max(xs):.2f}"


def trace_summary(path: str, K: int, W: int) -> str:
    """Per-phase durations of the attention kernels in a rocprofv3 kernel trace
    (`--kernel-trace --output-format csv`, the *_kernel_trace.csv file) of
    `bench.py --config k --steps K --warmup W` (neither --hot nor --row).
    main() launches, in this order: W warm-up steps, the step graph (one
    untimed and one timed replay), K eager steps, REPS more replays of the
    step graph, the hot graph over one KV copy (one untimed and REPS timed
    replays) and the graph of the partial kernel alone (one untimed and REPS
    timed replays).  Returns a markdown table."""
    import csv
    rows = []
    with open(path) as f:
        for r in csv.DictReader(f):
            kind = _kernel_kind(r["Kernel_Name"])
            if kind:
                rows.append((int(r["Start_Timestamp"]), int(r["End_Timestamp"]), kind))
    rows.sort()
    per_step = 2 if any(k == "merge" for _, _, k in rows) else 1
    phases = [("warm-up steps, eager", W, "cold"), ("step graph, untimed replay", K, "cold"),
              ("step graph, timed replay (`us_per_call`)", K, "cold"),
              ("eager steps (`us_per_call_eager`)", K, "cold"),
              (f"step graph, {REPS} more replays (`cold_median`)", REPS * K, "cold"),
              ("hot graph, untimed replay", K, "hot"),
              (f"hot graph, {REPS} replays (`hot_median`)", REPS * K, "hot"),
              ("partial kernel graph, untimed replay", K, "cold"),
              (f"partial kernel graph, {REPS} replays (`roofline.kernel_us`)", REPS * K, "cold")]
    lines = ["| phase | cache | steps | partial kernel avg / min / max (us) | merge avg / min / max (us) "
             "| first start to last end, per step (us) |", "|---|---|---:|---:|---:|---:|"]
    pos = 0
    cold = {"partial": [], "merge": []}
    for name, steps, cache in phases:
        n = steps * (1 if name.startswith("partial kernel") else per_step)
        seg = rows[pos:pos + n]
        pos += n
        if len(seg) < n:
            raise SystemExit(f"trace has {len(rows)} attention launches, fewer than the phases need")
        p = [(e - s) / 1000 for s, e, k in seg if k == "partial"]
        m = [(e - s) / 1000 for s, e, k in seg if k == "merge"]
        if cache == "cold" and name != "warm-up steps, eager":
            cold["partial"] += p
            cold["merge"] += m
        span = (seg[-1][1] - seg[0][0]) / 1000 / steps
        lines.append(f"| {name} | {cache} | {steps} | {_stats(p)} | {_stats(m)} | {span:.2f} |")
    if pos != len(rows):
        raise SystemExit(f"trace has {len(rows)} attention launches, the phases account for {pos}")
    lines.append(f"| all cold launches after the warm-up | cold | | {_stats(cold['partial'])} "
                 f"| {_stats(cold['merge'])} | |")
    return "\n".join(lines)


def _counter_means(path: str, counter: str):
    """Per-kernel mean over dispatches of one counter in a rocprofv3
    *_counter_collection.csv (values of one dispatch summed first)."""
    import csv
    per = {}
    with open(path) as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] != counter:
                continue
            key = (r["Kernel_Name"], r["Dispatch_Id"])
            per[key] = per.get(key, 0.0) + float(r["Counter_Value"])
    out = {}
    for (name, _), v in per.items():
        out.setdefault(name, []).append(v)
    return {name: (sum(v) / len(v), len(v)) for name, v in out.items()}


def traffic_summary(config: int, fetch_csv: str, write_csv: str, copy_fetch_csv: str,
                    copy_write_csv: str, copy_mib: int = 256) -> str:
    """HBM bytes per launch from rocprofv3 FETCH_SIZE and WRITE_SIZE runs (KiB
    per dispatch) of `bench.py --config k`, each scaled by what the same counter
    reads for the runtime's copy kernel moving `copy_mib` MiB (`bench.py
    --copy-probe`).  Writes the partial kernel's record (read by the bench
    while the kernel sources hash the same) and returns a markdown table."""
    from workloads import CONFIGS, make_config
    copy_bytes = copy_mib << 20
    cf = _counter_means(copy_fetch_csv, "FETCH_SIZE")
    cw = _counter_means(copy_write_csv, "WRITE_SIZE")
    ck = next(n for n in cf if "copyBuffer" in n)
    fetch_scale = copy_bytes / (cf[ck][0] * 1024)
    write_scale = copy_bytes / (cw[ck][0] * 1024)
    fetch = _counter_means(fetch_csv, "FETCH_SIZE")
    write = _counter_means(write_csv, "WRITE_SIZE")
    w = make_config(config)
    _, bytes_alg, bytes_partials = algorithmic_counts(w)
    lines = [f"Calibration: `__amd_rocclr_copyBuffer` moving {copy_mib} MiB reads FETCH_SIZE = "
             f"{cf[ck][0]:.1f} KiB and WRITE_SIZE = {cw[ck][0]:.1f} KiB per launch: scale "
             f"{fetch_scale:.4f} and {write_scale:.4f}.", "",
             "| kernel | launches | FETCH_SIZE KiB | WRITE_SIZE KiB | read MB | written MB |",
             "|---|---:|---:|---:|---:|---:|"]
    rec = None
    for name in sorted(fetch, key=lambda n: -fetch[n][0]):
        kind = _kernel_kind(name)
        if kind is None:
            continue
        fk, n = fetch[name]
        wk = write.get(name, (0.0, 0))[0]
        rb, wb = fk * 1024 * fetch_scale, wk * 1024 * write_scale
        short = _short_name(name)
        lines.append(f"| `{short}` | {n} | {fk:.1f} | {wk:.1f} | {rb / 1e6:.2f} | {wb / 1e6:.2f} |")
        if kind == "partial" and rec is None:
            rec = {"kernel": short, "config": config, "workload": CONFIGS[config]["name"],
                   "kernel_hash": kernel_hash(), "fetch_kib_raw": round(fk, 3),
                   "write_kib_raw": round(wk, 3), "fetch_scale": round(fetch_scale, 4),
                   "write_scale": round(write_scale, 4), "bytes_per_launch": int(rb + wb),
                   "fetch_bytes": int(rb), "write_bytes": int(wb),
                   "algorithmic_bytes": int(bytes_partials)}
    lines += ["", f"Algorithmic bytes: partial kernel {bytes_partials / 1e6:.2f} MB (prefix K/V, queries, "
              f"tree K/V, mask); whole call {bytes_alg / 1e6:.2f} MB (adds the outputs)."]
    if rec is not None:
        with open(traffic_file(config), "w") as f:
            json.dump(rec, f, indent=1)
        lines.append(f"Partial kernel: {rec['bytes_per_launch'] / 1e6:.2f} MB per launch = "
                     f"{rec['bytes_per_launch'] / bytes_partials:.3f} x its algorithmic bytes.")
    return "\n".join(lines)


def counter_summary(paths) -> str:
    """Per-dispatch means of every counter in rocprofv3 *_counter_collection.csv
    files, for the attention kernels.  Returns a markdown table."""
    import csv
    names, table = [], {}
    for path in paths:
        with open(path) as f:
            counters = sorted({r["Counter_Name"] for r in csv.DictReader(f)})
        for c in counters:
            for kname, (mean, n) in _counter_means(path, c).items():
                if _kernel_kind(kname) is None:
                    continue
                short = _short_name(kname)
                table.setdefault(short, {})[c] = (mean, n)
                if c not in names:
                    names.append(c)
    lines = ["| counter | " + " | ".join(f"`{k}`" for k in table) + " |",
             "|---|" + "---:|" * len(table)]
    for c in names:
        cells = []
        for k in table:
            v = table[k].get(c)
            cells.append(f"{v[0]:.4g} ({v[1]})" if v else "-")
        lines.append(f"| {c} | " + " | ".join(cells) + " |")
    return "\n".join(lines)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=1000)
    ap.add_argument("--config", type=int, default=4)
    ap.add_argument("--hot", action="store_true", help="reuse one KV copy (cache-resident)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="only copy a MIB-MiB buffer 5 times (calibrates HBM byte counters)")
    ap.add_argument("--row", choices=sorted(ROWS), default=None,
                    help="measure one of the steps around the verification path instead")
    ap.add_argument("--trace-summary", metavar="KERNEL_TRACE_CSV", default=None,
                    help="print per-phase kernel durations of a rocprofv3 trace of this bench "
                         "run (same --steps/--warmup) and exit; no GPU needed")
    ap.add_argument("--traffic-summary", nargs=4, default=None,
                    metavar=("FETCH_CSV", "WRITE_CSV", "COPY_FETCH_CSV", "COPY_WRITE_CSV"),
                    help="summarise rocprofv3 FETCH_SIZE/WRITE_SIZE runs of this bench run and "
                         "of --copy-probe 256 (counter_collection.csv files), write the traffic "
                         "record of --config and exit; no GPU needed")
    ap.add_argument("--counter-summary", nargs="+", metavar="COUNTER_CSV", default=None,
                    help="print per-dispatch means of the counters in rocprofv3 "
                         "counter_collection.csv files and exit; no GPU needed")
    args = ap.parse_args()
    if args.counter_summary:
        print(counter_summary(args.counter_summary))
        return
    if args.trace_summary:
        print(trace_summary(args.trace_summary, args.steps, args.warmup))
        return
    if args.traffic_summary:
        print(traffic_summary(args.config, *args.traffic_summary))
        return

    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the work shards by KV head or by sequence with no exchange between GPUs)",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import tree_attention_amd as ta
    from workloads import CONFIGS, make_config

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    dev = "cuda:0"
    if args.copy_probe:
        n = args.copy_probe << 20
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes": n, "launches": 5}), flush=True)
        return
    if args.row:
        print(json.dumps(ROWS[args.row](args)), flush=True)
        return
    spec = CONFIGS[args.config]
    log(f"generating workload {spec['name']}")
    w = make_config(args.config)
    B, T, Hq, D = w.q.shape
    Hkv = w.k_tree.shape[2]
    max_l = max(w.prefix_lens)
    flop, bytes_alg, bytes_partials = algorithmic_counts(w)

    q = w.q.to(dev)
    kt, vt = w.k_tree.to(dev), w.v_tree.to(dev)
    offsets = w.offsets.to(dev)
    parent = w.parent.to(dev)
    kv_bytes = 2 * w.k_prefix.numel() * w.k_prefix.element_size()
    n_copies = 1 if args.hot else max(2, math.ceil(512e6 / max(kv_bytes, 1)))
    kp0, vp0 = w.k_prefix.to(dev), w.v_prefix.to(dev)
    kv = [(kp0, vp0)] + [(kp0.clone(), vp0.clone()) for _ in range(n_copies - 1)]
    log(f"{n_copies} prefix KV copies of {kv_bytes / 1e6:.1f} MB each")

    # mask: built once per verification step, timed on its own.  Its launches
    # are captured in a graph so that the timing sees the GPU, not the
    # launch rate of the host.
    mask = torch.empty((B, T), dtype=torch.int64, device=dev)
    status = torch.empty((1,), dtype=torch.int32, device=dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for _ in range(3):
        assert ta.ltree_build_mask(parent, mask, status) == 0
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for _ in range(20):
            ta.ltree_build_mask(parent, mask, status)
    graph.replay()
    torch.cuda.synchronize()
    e0.record()
    graph.replay()
    e1.record()
    torch.cuda.synchronize()
    mask_us = e0.elapsed_time(e1) * 1000 / 20
    assert int(status.item()) == 0

    ws = ta.workspace_for(q, kt, max_l)
    o = torch.empty((B, T, Hq, D), dtype=torch.float32, device=dev)
    lse = torch.empty((B, Hq, T), dtype=torch.float32, device=dev)

    def partials(s, copies=n_copies):
        kp, vp = kv[s % copies]
        return ta.ltree_attn_partials(q, kp, vp, offsets, max_l, kt, vt, mask, ws, w.scale)

    def step(s, copies=n_copies):
        return partials(s, copies) | ta.ltree_attn_merge(q.dtype, B, T, Hq, Hkv, D, offsets,
                                                         max_l, o, lse, ws)

    def replay_us(g, reps, events=False):
        """Per-launch microseconds of `reps` timed replays of a graph of K
        launches: wall clock around replay + synchronize, or HIP events on
        the launch stream."""
        out = []
        for _ in range(reps):
            if events:
                e0.record()
                g.replay()
                e1.record()
                torch.cuda.synchronize()
                out.append(e0.elapsed_time(e1) * 1000 / K)
            else:
                t0 = time.perf_counter()
                g.replay()
                torch.cuda.synchronize()
                out.append((time.perf_counter() - t0) * 1e6 / K)
        return out

    log(f"warmup {args.warmup} steps")
    for s in range(args.warmup):
        assert step(s) == 0
    torch.cuda.synchronize()

    # the timed region: K whole steps back to back, launched as one HIP graph
    # (a serving loop replays the same launches every verification step), and
    # the same K steps launched one call at a time for comparison
    K = args.steps
    log(f"capturing {K} steps in a graph")
    steps_graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(steps_graph):
        for s in range(K):
            step(s)
    steps_graph.replay()
    torch.cuda.synchronize()
    log(f"timing {K} steps")
    t0 = time.perf_counter()
    steps_graph.replay()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1000 / K
    assert torch.isfinite(o).all() and torch.isfinite(lse).all()
    t0 = time.perf_counter()
    for s in range(K):
        step(s)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step_eager = (t1 - t0) * 1000 / K

    # the spread: the same graph replayed REPS more times (median and minimum
    # per call over the replays), and the same K steps over one KV copy, so
    # that the keys stay in the Infinity Cache (the hot-cache figure)
    cold_us = replay_us(steps_graph, REPS)
    hot_graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(hot_graph):
        for s in range(K):
            step(s, 1)
    hot_graph.replay()
    torch.cuda.synchronize()
    hot_us = replay_us(hot_graph, REPS)
    del hot_graph

    # the dominant kernel alone: K launches of it captured in a graph and
    # replayed between two events on the launch stream (events around every
    # launch would add a cache flush to each; eager launches add the host's
    # launch gaps)
    part_graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(part_graph):
        for s in range(K):
            partials(s)
    part_graph.replay()
    torch.cuda.synchronize()
    part_all = replay_us(part_graph, REPS, events=True)
    part_us = statistics.median(part_all)

    us = ms_per_step * 1000
    tflops = flop / (us * 1e-6) / 1e12
    part_tflops = flop / (part_us * 1e-6) / 1e12
    traffic = None
    tfile = traffic_file(args.config)
    if os.path.exists(tfile):
        rec = json.load(open(tfile))
        if rec.get("kernel_hash") == kernel_hash() and rec.get("config") == args.config:
            traffic = rec.get("bytes_per_launch")

    result = {
        "metric": METRIC,
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1); stands in for the pages' long-context datasets)",
        "config": {
            "workload": spec["name"], "B": B, "T": T, "Hq": Hq, "Hkv": Hkv, "D": D,
            "prefix_lens": w.prefix_lens,
            "cache": "hot (one KV copy)" if args.hot else f"cold ({n_copies} rotating KV copies)",
        },
        "us_per_call": round(us, 2),
        "us_per_call_eager": round(ms_per_step_eager * 1000, 2),
        "us_per_call_spread": {
            "replays": REPS,
            "cold_median": round(statistics.median(cold_us), 2),
            "cold_min": round(min(cold_us), 2),
            "hot_median": round(statistics.median(hot_us), 2),
            "hot_min": round(min(hot_us), 2),
            "hot_tflops": round(flop / (statistics.median(hot_us) * 1e-6) / 1e12, 2),
        },
        "mfma_frac": round(tflops / PEAK_BF16_TFLOPS, 4),
        "hbm_frac": round(bytes_alg / (us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4),
        "mask_build_us": round(mask_us, 2),
        "algorithmic": {"flop": flop, "bytes": bytes_alg},
        "roofline": {
            "kernel": "partial_mfma_kernel (prefix splits + tree part)",
            "bound": "mfma",
            "achieved": round(part_tflops, 2),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(part_tflops / PEAK_BF16_TFLOPS, 4),
            "traffic": traffic,
            "kernel_us": round(part_us, 2),
            "kernel_us_min": round(min(part_all), 2),
            "hbm_frac": round(bytes_partials / (part_us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4),
            # the whole call (partial kernel and merge) against the same peaks
            "call_frac": round(tflops / PEAK_BF16_TFLOPS, 4),
            "call_hbm_frac": round(bytes_alg / (us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4),
        },
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
