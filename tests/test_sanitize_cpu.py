"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer, on the CPU.

A copy of libnkv.so is built with the sanitizers on the host side of every source (the C
ABI's argument checks, the decode work planning, the launch wrappers, the block manager;
device code is built as usual) and with clang for all of it, so that one sanitizer runtime
serves the whole library.  The ABI tests (every rejection path, run through ctypes with
fake device pointers: nothing is launched) and the block manager tests (hand-worked trace,
random traces checked against the oracle, invariants) are then re-run in a subprocess
that preloads clang's ASan runtime, against that copy.  Any report fails the test.
No GPU is used: all of these calls return before a kernel would be enqueued.
"""

import concurrent.futures as cf
import glob
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "paged_kv_cache_258_amd", "csrc")
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
CLANGXX = shutil.which("amdclang++") or "/opt/rocm/llvm/bin/clang++"
ASAN_RT = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))

pytestmark = pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANGXX) and ASAN_RT),
                                reason="needs hipcc, amdclang++ and clang's ASan runtime")

SAN = ["-fsanitize=address", "-fsanitize=undefined", "-fno-omit-frame-pointer", "-fno-sanitize-recover=all"]
HIP_FLAGS = ["--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", "-fvisibility=hidden",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-I", os.path.join(ROOT, "include"),
             "-Wno-unused-command-line-argument"]


def build_sanitized(out_dir):
    cmds, objs = [], []
    for src in sorted(os.listdir(CSRC)):
        path = os.path.join(CSRC, src)
        obj = os.path.join(out_dir, os.path.splitext(src)[0] + ".o")
        if src.endswith(".hip"):
            host_san = [x for f in SAN for x in ("-Xarch_host", f)]   # host side only
            cmds.append([HIPCC, *HIP_FLAGS, *host_san, "-c", path, "-o", obj])
        elif src.endswith(".cpp"):
            cmds.append([CLANGXX, "-O1", "-g", "-std=c++17", "-fPIC", "-fvisibility=hidden", *SAN,
                         "-I", os.path.join(ROOT, "include"), "-c", path, "-o", obj])
        else:
            continue
        objs.append(obj)

    def run(cmd):
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stderr[-3000:]}"

    with cf.ThreadPoolExecutor(max_workers=min(8, len(cmds))) as ex:
        list(ex.map(run, cmds))
    lib = os.path.join(out_dir, "libnkv_san.so")
    run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", lib])
    return lib


def test_host_code_under_asan_and_ubsan(tmp_path):
    lib = build_sanitized(str(tmp_path))
    env = dict(os.environ)
    env.update(NKV_LIB=lib, LD_PRELOAD=ASAN_RT[-1],
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=0:exitcode=97",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1:exitcode=98",
               PYTHONDONTWRITEBYTECODE="1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-s", "-p", "no:cacheprovider", "-m", "not gpu",
                        os.path.join(ROOT, "tests", "test_abi_cpu.py"),
                        os.path.join(ROOT, "tests", "test_block_manager_cpu.py")],
                       capture_output=True, text=True, env=env, cwd=ROOT, timeout=600)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert " passed" in r.stdout
