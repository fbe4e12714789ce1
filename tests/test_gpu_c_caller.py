"""The C ABI used from plain C: tests/c_abi/ltree_c_caller (built by
tree_attention_amd/build.py) reads a seeded problem, calls ltree_build_mask
and ltree_attn on hipMalloc'd buffers, then ltree_attn_noalloc and
ltree_attn_strided over an interleaved copy of the prefix cache, and writes
the results, which must match the fp64 oracle (the mask bit-exact, o and lse
within the tolerances) and, for the two other calls, ltree_attn bit for bit
(the same kernels in the same order)."""

import os
import subprocess
import tempfile

import numpy as np
import pytest

import oracle
from gpu_helpers import BF16_O_TOL, F32_O_TOL, LSE_TOL, say
from workloads import make_workload

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CALLER = os.path.join(ROOT, "tests", "c_abi", "ltree_c_caller")


def _raw(t):
    """Element bytes of a CPU tensor (bf16 as its 16-bit pattern)."""
    import torch
    if t.dtype == torch.bfloat16:
        return t.contiguous().view(torch.int16).numpy().tobytes()
    return t.contiguous().numpy().astype(np.float32).tobytes()


@pytest.mark.parametrize("dtype,T,D", [("bf16", 64, 128), ("f32", 20, 64), ("bf16", 100, 128)])
def test_c_caller_matches_oracle(dtype, T, D):
    assert os.path.exists(CALLER), "build the C caller first (tree_attention_amd/build.py)"
    rng = np.random.default_rng(T + D)
    lens = [700, 0, 129]
    w = make_workload(rng, B=3, T=T, Hq=8, Hkv=2, D=D, prefix_lens=lens, trees=("bounded", 9, 3),
                      dtype=dtype)
    B, Hq, Hkv = 3, 8, 2
    with tempfile.TemporaryDirectory() as tmp:
        src, dst = os.path.join(tmp, "in.bin"), os.path.join(tmp, "out.bin")
        with open(src, "wb") as f:
            f.write(np.array([B, T, Hq, Hkv, D, 1 if dtype == "bf16" else 0, max(lens), sum(lens)],
                             dtype=np.int32).tobytes())
            f.write(np.array([w.scale], dtype=np.float32).tobytes())
            f.write(w.parent.numpy().astype(np.int32).tobytes())
            f.write(w.offsets.numpy().astype(np.int32).tobytes())
            for t in (w.q, w.k_prefix, w.v_prefix, w.k_tree, w.v_tree):
                f.write(_raw(t))
        say("C caller", dtype, T, D)
        r = subprocess.run([CALLER, src, dst], capture_output=True, text=True, timeout=120)
        assert r.returncode == 0, r.stdout + r.stderr
        Wd = (T + 63) // 64
        raw = open(dst, "rb").read()
    off = 0
    rc = np.frombuffer(raw, np.int32, 4, off); off += 16
    status = int(np.frombuffer(raw, np.int32, 1, off)[0]); off += 4
    mask = np.frombuffer(raw, np.uint64, B * T * Wd, off).reshape(B, T, Wd); off += 8 * B * T * Wd
    res = []
    for _ in range(3):  # ltree_attn, ltree_attn_noalloc, ltree_attn_strided
        o = np.frombuffer(raw, np.float32, B * T * Hq * D, off).reshape(B, T, Hq, D)
        off += 4 * o.size
        lse = np.frombuffer(raw, np.float32, B * Hq * T, off).reshape(B, Hq, T)
        off += 4 * lse.size
        res.append((o, lse))
    assert off == len(raw)
    assert rc.tolist() == [0, 0, 0, 0] and status == 0
    o, lse = res[0]
    for o2, lse2 in res[1:]:
        assert np.array_equal(o2, o) and np.array_equal(lse2, lse)
    assert np.array_equal(mask, oracle.oracle_mask(w.parent.numpy()))
    o_ref, lse_ref = oracle.oracle_attn(w.q, w.k_prefix, w.v_prefix, w.offsets.numpy(), w.k_tree,
                                        w.v_tree, w.parent.numpy(), w.scale)
    tol = BF16_O_TOL if dtype == "bf16" else F32_O_TOL
    assert np.max(np.abs(o - o_ref)) <= tol
    assert np.max(np.abs(lse - lse_ref)) <= LSE_TOL
