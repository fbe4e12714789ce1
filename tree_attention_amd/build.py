"""Build libltree.so (the C-ABI library) in-tree with hipcc for gfx950.

    python tree_attention_amd/build.py        # or __graft_entry__.build()

(Run as a file: importing the package loads the library it builds.)
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libltree.so")

SOURCES = ["ltree_api.hip", "ltree_plan.cpp", "mask_build.hip", "attn_partial_mfma.hip",
           "attn_partial_mfma_window.hip", "attn_partial_mfma_paged.hip", "attn_partial_mfma_strided.hip",
           "attn_partial_simple.hip", "lse_merge.hip", "kv_commit.hip",
           "tree_rope.hip"]

# Packed fp32 VALU instructions are switched off: the compiler would otherwise
# form v_pk_* ops from ordinary float code.  The host pass warns that it does
# not know the feature; that warning is harmless.
HIPCC_FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
               "-Wno-unused-command-line-argument"]


# Per-file extras.  The partial-attention kernel never sees a NaN (inputs are
# finite; masked scores are -inf), so NaN-quieting canonicalisation in front of
# every float max can be dropped there.
EXTRA_FLAGS = {name: ["-fno-honor-nans"] for name in
               ("attn_partial_mfma.hip", "attn_partial_mfma_window.hip",
                "attn_partial_mfma_paged.hip", "attn_partial_mfma_strided.hip")}


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def build(verbose: bool = False, jobs: int = 0) -> str:
    """Compile every HIP source (in parallel, `jobs` at a time; 0 = one per
    CPU up to 16) into tree_attention_amd/libltree.so."""
    from concurrent.futures import ThreadPoolExecutor

    def compile_one(src):
        obj = os.path.join(CSRC, "_obj", os.path.splitext(src)[0] + ".o")
        os.makedirs(os.path.dirname(obj), exist_ok=True)
        cmd = [hipcc(), *HIPCC_FLAGS, *EXTRA_FLAGS.get(src, []), "-I", INCLUDE, "-I", CSRC, "-c",
               os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{res.stderr}")
        return obj

    jobs = jobs or min(16, os.cpu_count() or 1)
    with ThreadPoolExecutor(max_workers=jobs) as pool:
        objs = list(pool.map(compile_one, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stderr}")
    os.replace(tmp, LIB)
    return LIB


C_CALLER_SRC = os.path.join(ROOT, "tests", "c_abi", "ltree_c_caller.c")
C_CALLER = os.path.join(ROOT, "tests", "c_abi", "ltree_c_caller")


def build_c_caller(verbose: bool = False) -> str:
    """Compile the plain C test caller of the library (host code only, gcc)
    against include/ltree.h and libltree.so."""
    rocm = os.path.dirname(os.path.dirname(os.path.realpath(hipcc())))
    cmd = ["gcc", "-std=c99", "-O2", "-Wall", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(rocm, "include"), "-I", INCLUDE, C_CALLER_SRC,
           "-L", PKG, "-lltree", "-L", os.path.join(rocm, "lib"), "-lamdhip64",
           "-Wl,-rpath,$ORIGIN/../../tree_attention_amd", "-Wl,-rpath," + os.path.join(rocm, "lib"),
           "-o", C_CALLER]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"gcc failed on the C caller:\n{res.stderr}")
    return C_CALLER


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
    print(build_c_caller(verbose="-v" in sys.argv))
