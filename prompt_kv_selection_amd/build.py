"""Builds libkvsel.so in-tree with hipcc for gfx950.

    python -m prompt_kv_selection_amd.build

Every HIP source under csrc/ is compiled to an object and linked into one
shared library next to this file.  Packed fp32 arithmetic is disabled for the
device code (the compiler otherwise forms v_pk_* fp32 instructions on its own).
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libkvsel.so")
DEBUG_LIB = os.path.join(HERE, "libkvsel_debug.so")
ARCH = os.environ.get("KVSEL_ARCH", "gfx950")

SOURCES = ["kvsel_api.hip", "kvsel_score.hip", "kvsel_select.hip", "kvsel_fused.hip", "kvsel_jacap.hip",
           "kvsel_probe.hip"]

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wno-unused-function",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{INCLUDE}",
    f"-I{CSRC}",
]


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found: the HIP toolchain is required to build libkvsel")
    return path


def _run(cmd):
    proc = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # hipcc's host pass does not know the packed-fp32 feature; drop that note.
    out = "\n".join(l for l in proc.stdout.splitlines() if "packed-fp32-ops" not in l)
    if proc.returncode != 0:
        raise RuntimeError(f"command failed ({proc.returncode}): {' '.join(cmd)}\n{out}")
    return out


def build(verbose: bool = False, debug: bool = True) -> str:
    """Build libkvsel.so, and with debug libkvsel_debug.so: the same sources
    with KVSEL_DEBUG defined (device-side index checks that set a flag)."""
    os.makedirs(BUILD, exist_ok=True)
    cc = hipcc()
    variants = [("", [], LIB)] + ([("debug", ["-DKVSEL_DEBUG=1"], DEBUG_LIB)] if debug else [])

    def compile_one(job):
        tag, defs, src = job
        obj_dir = os.path.join(BUILD, tag) if tag else BUILD
        os.makedirs(obj_dir, exist_ok=True)
        obj = os.path.join(obj_dir, os.path.splitext(src)[0] + ".o")
        out = _run([cc, *HIPCC_FLAGS, *defs, "-c", os.path.join(CSRC, src), "-o", obj])
        if verbose and out.strip():
            print(out)
        return obj

    jobs = [(tag, defs, src) for tag, defs, _ in variants for src in SOURCES]
    with ThreadPoolExecutor(max_workers=min(len(jobs), os.cpu_count() or 4)) as ex:
        objs = list(ex.map(compile_one, jobs))
    for i, (tag, _, lib) in enumerate(variants):
        tmp = lib + ".tmp"
        _run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs[i * len(SOURCES):(i + 1) * len(SOURCES)]])
        os.replace(tmp, lib)
        if verbose:
            print(f"built {lib}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
