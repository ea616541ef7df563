"""Build libgqa.so in-tree with hipcc for gfx950.

    python -m grouped_query_attention_02_amd.build

Every HIP source under csrc/ is compiled to an object in _build/ (in parallel)
and linked into grouped_query_attention_02_amd/libgqa.so; probes/probes.hip (the
microbenchmarks bench.py compares against) becomes libgqa_probes.so. The
packed-fp32 target feature is switched off for all device code.
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
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libgqa.so")
PROBES_SRC = os.path.join(PKG, "probes", "probes.hip")
PROBES_LIB = os.path.join(PKG, "libgqa_probes.so")
ARCH = os.environ.get("GQA_OFFLOAD_ARCH", "gfx950")

HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"

CFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
    "-I", INCLUDE, "-I", CSRC,
]


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src)[:-4] + ".o")
    cmd = [HIPCC, *CFLAGS, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + f".tmp{os.getpid()}"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    ptmp = PROBES_LIB + f".tmp{os.getpid()}"
    cmd = [HIPCC, *CFLAGS, "-shared", PROBES_SRC, "-o", ptmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"probe build failed:\n{r.stdout}\n{r.stderr}")
    os.replace(ptmp, PROBES_LIB)
    if verbose:
        print(f"built {LIB} and {PROBES_LIB}")
    return LIB


# Host-side sanitizers for the library's host code (argument checks, planning, launch
# set-up): each flag sits right after -Xarch_host, so the device code is built as usual.
HOST_SANITIZE = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                 "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host",
                 "-fno-omit-frame-pointer", "-Xarch_host", "-g"]


def clang_asan_runtime():
    """Path of the ASan runtime of the compiler hipcc drives (None if not installed)."""
    r = subprocess.run([HIPCC, "-print-file-name=libclang_rt.asan-x86_64.so"],
                       capture_output=True, text=True)
    path = r.stdout.strip().splitlines()[-1] if r.stdout.strip() else ""
    if os.path.isabs(path) and os.path.exists(path):
        return path
    import glob
    hits = sorted(glob.glob("/opt/rocm*/lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[-1] if hits else None


def build_host_sanitized(path: str) -> str:
    """libgqa.so with ASan + UBSan on its host code, written to `path` (for the CPU tests of
    the C ABI; the process must load the ASan runtime first)."""
    bdir = os.path.join(os.path.dirname(path), "objs")
    os.makedirs(bdir, exist_ok=True)
    objs = []
    for src in sources():
        obj = os.path.join(bdir, os.path.basename(src)[:-4] + ".o")
        r = subprocess.run([HIPCC, *CFLAGS, *HOST_SANITIZE, "-c", src, "-o", obj],
                           capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
        objs.append(obj)
    r = subprocess.run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *HOST_SANITIZE,
                        "-shared-libsan", "-o", path, *objs], capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    return path


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
