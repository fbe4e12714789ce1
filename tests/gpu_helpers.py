"""Shared helpers of the GPU parity tests: move a workload to the device, run
the library through its C ABI, and compare with the fp64 oracle."""

from __future__ import annotations

import sys

import numpy as np
import torch

import oracle

BF16_O_TOL = 2e-2     # max-abs error of o for bf16 inputs, fp32 accumulation
F32_O_TOL = 1e-4      # max-abs error of o for fp32 inputs
LSE_TOL = 1e-3        # max-abs error of lse (natural log)


def say(*a):
    """Name the case before a GPU step, flushed, so a failing run shows it."""
    print("[gpu-case]", *a, file=sys.stderr, flush=True)


def to_device(w, dev="cuda"):
    return dict(q=w.q.to(dev), k_prefix=w.k_prefix.to(dev), v_prefix=w.v_prefix.to(dev),
                offsets=w.offsets.to(dev), k_tree=w.k_tree.to(dev), v_tree=w.v_tree.to(dev),
                parent=w.parent.to(dev))


def run_library(w, d=None):
    """Mask + attention through the C ABI.  Returns (o, lse, mask, status) on
    the host."""
    import tree_attention_amd as ta
    d = d or to_device(w)
    mask, status = ta.build_mask(d["parent"])
    o, lse = ta.attn(d["q"], d["k_prefix"], d["v_prefix"], d["offsets"],
                     max(w.prefix_lens) if w.prefix_lens else 0, d["k_tree"], d["v_tree"],
                     mask, w.scale)
    torch.cuda.synchronize()
    return o.cpu(), lse.cpu(), mask.cpu(), status.cpu()


def oracle_full(w):
    return oracle.oracle_attn(w.q, w.k_prefix, w.v_prefix, w.offsets.numpy(), w.k_tree,
                              w.v_tree, w.parent.numpy(), w.scale)


def mask_words(mask_i64: torch.Tensor) -> np.ndarray:
    return mask_i64.numpy().view(np.uint64)


def check_parity(w, o, lse, o_ref, lse_ref, o_tol=None):
    o_tol = o_tol if o_tol is not None else (BF16_O_TOL if w.dtype == "bf16" else F32_O_TOL)
    o = o.double().numpy()
    lse = lse.double().numpy()
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
    eo = np.max(np.abs(o - o_ref))
    el = np.max(np.abs(lse - lse_ref))
    assert eo <= o_tol, f"o max-abs error {eo:.3e} > {o_tol}"
    assert el <= LSE_TOL, f"lse max-abs error {el:.3e} > {LSE_TOL}"
    return eo, el
