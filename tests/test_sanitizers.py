"""Host sanitizer builds, run on the CPU.

* The oracle (oracle/oracle.c) built with AddressSanitizer + UndefinedBehaviorSanitizer runs
  the oracle pin suites; any out-of-bounds access, use of freed memory or undefined behaviour
  (signed overflow, shift, misaligned access, ...) aborts the run.
* The library's host code (argument checks and launch planning of libgqa.so, clang's ASan +
  UBSan on the host side only; device code is built as usual) runs the C-ABI checks, which
  drive every invalid-argument path and the planning queries without a GPU.
Each suite runs in a subprocess whose LD_PRELOAD starts with the matching sanitizer runtime.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

pytestmark = pytest.mark.timeout(900)


def _run_suite(env_extra, runtime, tests, tmp_path):
    env = dict(os.environ)
    env.update(env_extra)
    prev = env.get("LD_PRELOAD", "")
    env["LD_PRELOAD"] = runtime + (":" + prev if prev else "")
    # reports go to files: pytest's capture of the subprocess's stderr is lost when a
    # sanitizer stops the process
    logs = tmp_path / "san"
    env["ASAN_OPTIONS"] = f"detect_leaks=0:halt_on_error=1:log_path={logs}"
    env["UBSAN_OPTIONS"] = f"halt_on_error=1:print_stacktrace=1:log_path={logs}"
    env["PYTHONDONTWRITEBYTECODE"] = "1"
    cmd = [sys.executable, "-m", "pytest", "-q", "-x", "-s", "-m", "not gpu", "-p", "no:cacheprovider",
           *tests]
    r = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=850)
    out = r.stdout + r.stderr
    for f in sorted(tmp_path.glob("san*")):
        out += f"\n--- {f.name}\n" + f.read_text()
    assert "AddressSanitizer" not in out, out[-4000:]
    assert "runtime error" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert " passed" in out


def _gcc_runtime(name):
    p = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True)
    path = p.stdout.strip()
    if not os.path.isabs(path) or not os.path.exists(path):
        pytest.skip(f"gcc's {name} is not installed")
    return path


def test_oracle_pins_under_asan_ubsan(tmp_path):
    import oracle
    lib = oracle.build_sanitized(str(tmp_path / "liboracle_san.so"))
    _run_suite({oracle.SANITIZED_ENV: lib}, _gcc_runtime("libasan.so"),
               ["tests/test_oracle_pins.py", "tests/test_oracle_pins_ext.py"], tmp_path)


def test_abi_host_code_under_asan_ubsan(tmp_path):
    from grouped_query_attention_02_amd import build as gbuild
    runtime = gbuild.clang_asan_runtime()
    if runtime is None:
        pytest.skip("clang's ASan runtime is not installed")
    lib = gbuild.build_host_sanitized(str(tmp_path / "libgqa_san.so"))
    _run_suite({"GQA_LIBRARY_PATH": lib}, runtime, ["tests/test_abi_cpu.py"], tmp_path)
