"""Build libmla_fp8.so in-tree with hipcc for gfx950.

Usage: ``python -m fp8_mla_context_amd.build`` (or ``__graft_entry__.build()``).
The library lands in ``fp8_mla_context_amd/lib/libmla_fp8.so``. Two build variants of
the FP8 prefill's PV arithmetic land beside it, with the same exports:
``libmla_fp8_pv1.so`` (P rounded once to E4M3, PV on the FP8 MFMA) and
``libmla_fp8_pv2.so`` (P in two E4M3 terms, PV on the FP8 MFMA); the default library
rounds P once to bf16 and runs PV on the bf16 MFMA. The default library also holds the
prefill source built with 4-wave workgroups of 128 rows, for grids too small to fill the
chip (see prefill_launch). Sources compile to objects in parallel; only the prefill source differs
between the variants.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_DIR = os.path.join(PKG, "lib")
LIB_PATH = os.path.join(LIB_DIR, "libmla_fp8.so")
OBJ_DIR = os.path.join(PKG, "_build")

SOURCES = ["abi.hip", "quant_static.hip", "merge_lse.hip", "prefill_fp8.hip", "prefill_bf16.hip",
           "chunked.hip", "kv_producer.hip"]
VARIANT_SOURCE = "prefill_fp8.hip"
# library suffix -> extra flags of the prefill source
VARIANTS = {"": [], "_pv1": ["-DMLA_PV_MODE=1"], "_pv2": ["-DMLA_PV_MODE=2"]}
# the default library also holds the prefill source built with 4-wave workgroups, which
# its launcher uses for grids of at most one workgroup per CU
SMALL_GRID_FLAGS = ["-DMLA_PREFILL_WAVES=4", "-DMLA_PREFILL_SMALL_GRID"]

# Packed-fp32 VALU forms are kept out of the generated code on purpose.
HIP_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def variant_path(suffix: str, out_path: str = LIB_PATH) -> str:
    """Path of the library variant with the given suffix ("", "_pv1", "_pv2")."""
    base, ext = os.path.splitext(out_path)
    return base + suffix + ext


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + " ".join(cmd) + "\n" + res.stdout + res.stderr)


def build(verbose: bool = False, extra_flags=(), out_path: str = LIB_PATH,
          variants: bool = True) -> str:
    """Compile every source and link the library (and, with variants, its PV variants).
    Returns the path of the default library."""
    os.makedirs(os.path.dirname(out_path), exist_ok=True)
    tag = os.path.splitext(os.path.basename(out_path))[0]
    obj_dir = os.path.join(OBJ_DIR, tag)
    os.makedirs(obj_dir, exist_ok=True)
    cc = hipcc()
    base = [cc, *HIP_FLAGS, *extra_flags, "-I", INCLUDE, "-I", CSRC, "-c"]
    wanted = VARIANTS if variants else {"": []}
    jobs = {}  # object path -> command
    for src in SOURCES:
        if src == VARIANT_SOURCE:
            continue
        obj = os.path.join(obj_dir, src.replace(".hip", ".o"))
        jobs[obj] = base + ["-o", obj, os.path.join(CSRC, src)]
    for suffix, flags in wanted.items():
        obj = os.path.join(obj_dir, VARIANT_SOURCE.replace(".hip", suffix + ".o"))
        jobs[obj] = base + flags + ["-o", obj, os.path.join(CSRC, VARIANT_SOURCE)]
    small_obj = os.path.join(obj_dir, VARIANT_SOURCE.replace(".hip", "_4w.o"))
    jobs[small_obj] = base + SMALL_GRID_FLAGS + ["-o", small_obj, os.path.join(CSRC, VARIANT_SOURCE)]
    with ThreadPoolExecutor(max(1, min(len(jobs), os.cpu_count() or 1, 8))) as ex:
        for f in [ex.submit(_run, cmd, verbose) for cmd in jobs.values()]:
            f.result()
    common = [os.path.join(obj_dir, s.replace(".hip", ".o")) for s in SOURCES
              if s != VARIANT_SOURCE]
    for suffix in wanted:
        path = variant_path(suffix, out_path)
        tmp = path + ".tmp"
        objs = common + [os.path.join(obj_dir, VARIANT_SOURCE.replace(".hip", suffix + ".o"))]
        if suffix == "":
            objs.append(small_obj)
        _run([cc, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs], verbose)
        os.replace(tmp, path)
    return out_path


if __name__ == "__main__":
    path = build(verbose="-v" in sys.argv)
    print(path)
