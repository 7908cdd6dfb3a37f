"""Build libmla_fp8.so in-tree with hipcc for gfx950.

Usage: ``python -m fp8_mla_context_amd.build`` (or ``__graft_entry__.build()``).
The library lands in ``fp8_mla_context_amd/lib/libmla_fp8.so``.
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
LIB_DIR = os.path.join(PKG, "lib")
LIB_PATH = os.path.join(LIB_DIR, "libmla_fp8.so")

SOURCES = ["abi.hip", "quant_static.hip", "merge_lse.hip", "prefill_fp8.hip", "prefill_bf16.hip",
           "chunked.hip", "kv_producer.hip"]

# Packed-fp32 VALU forms are kept out of the generated code on purpose.
HIP_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def build(verbose: bool = False, extra_flags=(), out_path: str = LIB_PATH) -> str:
    os.makedirs(os.path.dirname(out_path), exist_ok=True)
    tmp = out_path + ".tmp"
    cmd = [hipcc(), *HIP_FLAGS, *extra_flags, "-I", INCLUDE, "-I", CSRC, "-o", tmp]
    cmd += [os.path.join(CSRC, s) for s in SOURCES]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + res.stdout + res.stderr)
    os.replace(tmp, out_path)
    return out_path


if __name__ == "__main__":
    path = build(verbose="-v" in sys.argv)
    print(path)
