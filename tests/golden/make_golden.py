"""Write the oracle regression fixtures in this folder.

Calls only ``oracle/`` (and the seeded input generator).  The pages print no
worked example of the attention, so these files are not the pages' values:
they pin the oracle against its own past output, so that any later change to
its arithmetic shows up as a diff that must be justified.

Run:  python tests/golden/make_golden.py
"""

import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import oracle  # noqa: E402
from workloads import make_config, make_workload  # noqa: E402


def _write(name, header, rows):
    with open(os.path.join(HERE, name), "w") as f:
        f.write(header)
        for r in rows:
            f.write(" ".join(r) + "\n")


def main():
    # Tiny fp32 workload (batch 1, 4/4 heads, head_dim 64, prefix 512, T = 8).
    w = make_config(1)
    o, lse = oracle.oracle_attn(w.q, w.k_prefix, w.v_prefix, w.offsets.numpy(),
                                w.k_tree, w.v_tree, w.parent.numpy(), w.scale)
    mask = oracle.oracle_mask(w.parent.numpy())
    rows = []
    for h in range(4):
        for i in range(8):
            rows.append([str(h), str(i), repr(float(lse[0, h, i])),
                         repr(float(o[0, i, h, 0])), repr(float(o[0, i, h, 63])),
                         repr(float(o[0, i, h].sum()))])
    _write("tiny_fp32_seed1001.txt",
           "# oracle regression values: tiny fp32 workload, default_rng(1001)\n"
           f"# parent = {w.parent.numpy()[0].tolist()}\n"
           f"# mask words = {[hex(int(x)) for x in mask[0, :, 0]]}\n"
           "# columns: head  node  lse  o[d=0]  o[d=63]  sum_d o\n", rows)

    # Small bf16 ragged case with an empty prefix and a forest.
    rng = np.random.default_rng(77)
    w = make_workload(rng, B=3, T=5, Hq=6, Hkv=2, D=16, prefix_lens=[0, 7, 3],
                      trees=["forest", "chain", ("bounded", 3, 2)], dtype="bf16")
    o, lse = oracle.oracle_attn(w.q, w.k_prefix, w.v_prefix, w.offsets.numpy(),
                                w.k_tree, w.v_tree, w.parent.numpy(), w.scale)
    rows = []
    for b in range(3):
        for h in range(6):
            for i in range(5):
                rows.append([str(b), str(h), str(i), repr(float(lse[b, h, i])),
                             repr(float(o[b, i, h].sum()))])
    _write("ragged_bf16_seed77.txt",
           "# oracle regression values: B=3, T=5, Hq=6, Hkv=2, D=16, prefixes\n"
           "# [0, 7, 3], trees [forest, chain, bounded(3,2)], bf16, default_rng(77)\n"
           f"# parent = {w.parent.numpy().tolist()}\n"
           "# columns: seq  head  node  lse  sum_d o\n", rows)


if __name__ == "__main__":
    main()
