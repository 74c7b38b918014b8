"""Build the HIP library ``libgpt_attn.so`` in-tree with hipcc for gfx950.

Four translation units hold the C ABI and include the kernel headers:
``csrc/gpt_attn.hip`` (the attention layer, include/gpt_attn.h),
``csrc/gpt_block.hip`` (LayerNorm, the Pre-LN half-block, the MLP;
include/gpt_block.h), ``csrc/gpt_decode.hip`` (one-token decode with a
key/value cache; include/gpt_decode.h) and ``csrc/gpt_noalloc.hip`` (the
allocation-free forward with its static device scratch; include/gpt_attn.h).  Packed-fp32 instructions are disabled for every kernel
(``-target-feature -packed-fp32-ops``); hipcc's host pass warns that it does
not know that feature, which is harmless.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRCS = [os.path.join(HERE, "csrc", n)
        for n in ("gpt_attn.hip", "gpt_block.hip", "gpt_decode.hip", "gpt_noalloc.hip")]
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libgpt_attn.so")
ARCH = os.environ.get("GPT_ATTN_ARCH", "gfx950")


def hipcc() -> str:
    p = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(p):
        raise RuntimeError("hipcc not found; the HIP library cannot be built")
    return p


def build(out: str = LIB, extra=(), verbose: bool = False) -> str:
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-shared", "-fPIC",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-Wno-unused-command-line-argument", "-I", INCLUDE, *extra, *SRCS, "-o", tmp]
    if verbose:
        print(" ".join(cmd), file=sys.stderr)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("hipcc failed building libgpt_attn.so")
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
