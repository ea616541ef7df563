"""Build tests/_build/c_abi_client from tests/c_abi_client.cpp: a C++ program that calls
libgqa.so through include/gqa.h only and checks its results against the fp64 oracle
(liboracle.so). Test infrastructure; run by __graft_entry__.build() after the library and the
oracle are built, and by test_c_client_gpu.py on a GPU."""
import os
import shutil
import subprocess

TESTS = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(TESTS)
SRC = os.path.join(TESTS, "c_abi_client.cpp")
EXE = os.path.join(TESTS, "_build", "c_abi_client")


def build() -> str:
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    os.makedirs(os.path.dirname(EXE), exist_ok=True)
    tmp = EXE + f".tmp{os.getpid()}"
    cmd = [hipcc, "-O2", "-std=c++17", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-Wno-unused-command-line-argument", "-I", os.path.join(ROOT, "include"), SRC,
           "-L", os.path.join(ROOT, "grouped_query_attention_02_amd"), "-lgqa",
           "-L", os.path.join(ROOT, "oracle"), "-loracle",
           "-Wl,-rpath,$ORIGIN/../../grouped_query_attention_02_amd",
           "-Wl,-rpath,$ORIGIN/../../oracle", "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"building the C ABI client failed:\n{r.stderr[-3000:]}")
    os.replace(tmp, EXE)
    return EXE


if __name__ == "__main__":
    print("built", build())
