"""The C ABI from C++: tests/c_abi_client.cpp allocates device memory with the HIP runtime,
calls gqa_prefill (causal, with LSE) and gqa_decode (ragged, 3 splits) through include/gqa.h
and checks both against the fp64 oracle (O within 2e-2, LSE within 1e-3), plus a rejected bad
argument. Built by __graft_entry__.build() (tests/build_c_client.py)."""
import os
import subprocess

import pytest

from build_c_client import EXE

pytestmark = pytest.mark.gpu


def test_c_abi_client(built_lib):
    if not os.path.exists(EXE):
        pytest.fail(f"{EXE} is missing: run __graft_entry__.build() (tests/build_c_client.py)")
    print("case c_abi_client", flush=True)
    r = subprocess.run([EXE], capture_output=True, text=True, timeout=120)
    print(r.stdout, r.stderr, flush=True)
    assert r.returncode == 0 and r.stdout.strip().endswith("OK"), r.stdout + r.stderr
