"""Build libpkv.so (the HIP library behind include/pkv.h) for gfx950, in-tree.

    python -m paged_kv_cache_434_amd.build

Each csrc/*.hip is compiled separately (in parallel) and linked into one
shared library next to this file.
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
INCLUDE = os.path.join(ROOT, "include")
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libpkv.so")
OBJDIR = os.path.join(ROOT, "_build", "pkv")

ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # keep hipcc from forming packed fp32 instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    "-I", INCLUDE,
]


def _compile(src: str) -> str:
    obj = os.path.join(OBJDIR, os.path.basename(src) + ".o")
    cmd = [HIPCC, *FLAGS, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    """Compile every source and link libpkv.so; returns its path."""
    os.makedirs(OBJDIR, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


SAN_LIB = os.path.join(ROOT, "_build", "asan", "libpkv.so")
# the argument checks (csrc/api.hip) with AddressSanitizer and
# UndefinedBehaviorSanitizer on their host code; device code is not
# instrumented
SAN_SOURCE = "api.hip"
SAN_FLAGS = [
    "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
    "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer",
    "-Xarch_host", "-g",
]


def build_sanitized(verbose: bool = False) -> str:
    """libpkv.so whose argument checks (csrc/api.hip) are built with host
    ASan and UBSan, linked with the kernel sources' regular objects (reused
    from the last build when newer than their sources).  Returns its path."""
    outdir = os.path.dirname(SAN_LIB)
    os.makedirs(outdir, exist_ok=True)
    os.makedirs(OBJDIR, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    headers = glob.glob(os.path.join(CSRC, "*.hpp")) + glob.glob(os.path.join(INCLUDE, "*.h"))
    newest_header = max(os.path.getmtime(h) for h in headers)

    def comp(src):
        if os.path.basename(src) == SAN_SOURCE:
            obj = os.path.join(outdir, SAN_SOURCE + ".o")
            cmd = [HIPCC, *FLAGS, *SAN_FLAGS, "-c", src, "-o", obj]
        else:
            obj = os.path.join(OBJDIR, os.path.basename(src) + ".o")
            if (os.path.exists(obj) and os.path.getmtime(obj) >= os.path.getmtime(src)
                    and os.path.getmtime(obj) >= newest_header):
                return obj
            cmd = [HIPCC, *FLAGS, "-c", src, "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
        return obj

    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(comp, srcs))
    r = subprocess.run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-Xarch_host",
                        "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                        "-shared-libsan", *objs, "-o", SAN_LIB], capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    if verbose:
        print(f"built {SAN_LIB}")
    return SAN_LIB


def sanitizer_runtime() -> str:
    """Path of the compiler's shared ASan runtime (preloaded into a Python
    process that loads the sanitized library)."""
    r = subprocess.run([HIPCC, "-print-file-name=libclang_rt.asan-x86_64.so"],
                       capture_output=True, text=True)
    path = r.stdout.strip()
    if not os.path.isabs(path) or not os.path.exists(path):
        found = glob.glob("/opt/rocm/lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so")
        path = found[0] if found else ""
    return path


def clean() -> None:
    shutil.rmtree(OBJDIR, ignore_errors=True)


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
