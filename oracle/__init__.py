"""fp64 CPU oracle for hybrid tree-verification attention.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
path (``tree_attention_amd``) and imports nothing from it.

Sources (cited by page title and section; the pages print no code, formula or
worked example):

* gist.science, "LongSpec: Long-Context Lossless Speculative Decoding with
  Efficient Drafting and Verification" (German explainer), section 2
  "Methodik", part C "Schnelle Tree Attention": the attention of the tree
  tokens is split into a cached part (the long KV cache, no mask) and a
  speculative part (the few new draft tokens, tree mask), and the two partial
  results are joined with a log-sum-exp step.
* same page, section 1 "Problemstellung", item "Ineffiziente Verifikation":
  tree attention needs a mask over the draft tokens.
* same page, section 2 "Methodik", part A, item "Cross-Attention mit
  geteiltem KV-Cache": the draft model attends to the target model's KV cache
  directly (the prefix-only attention of ``oracle_prefix_attn``); item
  "Sliding-Window Self-Attention": the draft's own self-attention sees a
  window of recent tokens (``oracle_window_attn``).
* mlsanity.com, "LongSpec: Long-Context Lossless Speculative Decoding with
  Efficient Drafting and Verification", section "Abstract (arXiv)": fast
  prefix computation is combined with standard tree attention.

Every function here is pinned by ``tests/test_oracle_pins.py`` against closed
forms, library routines, invariants and brute force.  No function is
"parity unpinned".
"""

from .tree_attention_oracle import (  # noqa: F401
    ancestor_matrix,
    check_parent,
    gather_paged,
    gather_strided,
    lse_merge,
    oracle_commit_kv,
    oracle_attn,
    oracle_attn_rows,
    oracle_attn_split,
    oracle_mask,
    oracle_prefix_attn,
    oracle_tree_rope,
    oracle_window_attn,
    round_bf16,
    tree_depth,
)
