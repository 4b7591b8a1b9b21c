"""Build libnkv.so in-tree with hipcc for gfx950.

Usage: ``python -m paged_kv_cache_258_amd.build`` (or ``build()`` from Python).
Each HIP source is compiled to an object in parallel, then linked into
``paged_kv_cache_258_amd/libnkv.so`` (replaced atomically).
"""

from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libnkv.so")
SOURCES = ["api.hip", "store.hip", "rope_store.hip", "rmsnorm.hip", "decode.hip", "prefill.hip", "validate.hip",
           "block_manager.cpp"]
ARCH = "gfx950"

FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-fvisibility=hidden",
    # packed fp32 VALU ops are kept out of every kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
    "-Wno-unused-command-line-argument",
]

# Per-source flags.  prefill.hip, decode.hip: keep MFMA accumulators and results in
# VGPRs; with the default heuristic the O^T accumulators live in AGPRs and every loop
# iteration copies all of them between AGPRs (and to VGPRs and back around the rarely
# taken rescale branch).
SOURCE_FLAGS = {
    "prefill.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
    "decode.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
}


# host-only sources
HOST_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-fvisibility=hidden", "-Wall", "-I", os.path.join(ROOT, "include")]


def _cxx() -> str:
    for cand in (os.environ.get("CXX"), shutil.which("g++"), shutil.which("c++")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("no host C++ compiler (g++) found")


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libnkv.so)")


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return r


def build(verbose: bool = False, out: str = LIB, defines=(), build_dir: str = BUILD) -> str:
    """Compile every HIP source and link ``out``; ``defines`` are extra -D flags."""
    hipcc = _hipcc()
    os.makedirs(build_dir, exist_ok=True)
    objs, cmds = [], []
    for src in SOURCES:
        obj = os.path.join(build_dir, os.path.splitext(src)[0] + ".o")
        objs.append(obj)
        if src.endswith(".cpp"):      # host-only C++ (the block manager)
            cmds.append([_cxx(), *HOST_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj])
            continue
        cmds.append([hipcc, *FLAGS, *SOURCE_FLAGS.get(src, []), *[f"-D{d}" for d in defines], "-c",
                     os.path.join(CSRC, src), "-o", obj])
    with cf.ThreadPoolExecutor(max_workers=min(len(cmds), os.cpu_count() or 4)) as ex:
        for r in ex.map(_run, cmds):
            noise = ("packed-fp32-ops", "warning: argument unused")
            msg = "\n".join(l for l in r.stderr.splitlines() if l.strip() and not any(n in l for n in noise))
            if verbose and msg:
                print(msg, file=sys.stderr)
    tmp = out + ".tmp"
    _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp])
    os.replace(tmp, out)
    if verbose:
        print(f"built {out}")
    return out


if __name__ == "__main__":
    build(verbose=True)
