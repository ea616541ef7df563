"""Calls from several host threads at once, each on its own stream, in a fresh process.

The library keeps per-device state that is filled in on first use (compute-unit count,
workgroups per CU and LDS attribute per kernel); those caches are written with atomic
stores of values every thread computes alike, and everything else a call needs arrives in
its arguments. The script below starts five threads together (a barrier), so that their
first calls into the library overlap, each thread running one kind of call 30 times on its
own default-priority stream (ctypes releases the GIL around foreign calls, so the calls
and their launches interleave). Afterwards the same calls run one at a time on the default
stream. The kernels are deterministic, so every output must match bit for bit.
"""
import os
import subprocess
import sys
import textwrap

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

SCRIPT = textwrap.dedent("""
    import sys, threading
    import torch
    import grouped_query_attention_02_amd as gqa

    dev = torch.device("cuda:0")
    g = torch.Generator(device="cpu").manual_seed(7)

    def rnd(*shape, dtype=torch.bfloat16):
        return torch.randn(*shape, generator=g).to(dtype).to(dev)

    def lens(b, hi, lo=1):
        return torch.randint(lo, hi + 1, (b,), generator=g, dtype=torch.int32).to(dev)

    q0, k0, v0 = rnd(2, 300, 8, 64), rnd(2, 300, 2, 64), rnd(2, 300, 2, 64)
    l0 = lens(2, 300)
    q1, k1, v1 = rnd(1, 513, 8, 128), rnd(1, 513, 2, 128), rnd(1, 513, 2, 128)
    q2, kc2, vc2 = rnd(5, 16, 128), rnd(5, 2, 700, 128), rnd(5, 2, 700, 128)
    l2 = lens(5, 700, 0)
    q3, kc3, vc3 = rnd(3, 8, 64), rnd(3, 8, 300, 64), rnd(3, 8, 300, 64)
    l3 = lens(3, 300)
    q4, k4, v4 = (rnd(1, 64, 4, 32, dtype=torch.float32), rnd(1, 64, 2, 32, dtype=torch.float32),
                  rnd(1, 64, 2, 32, dtype=torch.float32))
    torch.cuda.synchronize()

    calls = [
        lambda: gqa.prefill(q0, k0, v0, seqlens=l0, return_lse=True),
        lambda: gqa.prefill(q1, k1, v1, causal=True),
        lambda: gqa.decode(q2, kc2, vc2, l2, num_splits=3, return_lse=True),
        lambda: gqa.decode(q3, kc3, vc3, l3),
        lambda: gqa.prefill(q4, k4, v4),
    ]

    def flat(r):
        return [t.clone() for t in (r if isinstance(r, tuple) else (r,))]

    results, errors = [None] * len(calls), []
    start = threading.Barrier(len(calls))

    def worker(i):
        try:
            s = torch.cuda.Stream(device=dev)
            s.wait_stream(torch.cuda.default_stream(dev))
            start.wait()
            with torch.cuda.stream(s):
                for _ in range(30):
                    r = calls[i]()
                results[i] = flat(r)
            s.synchronize()
        except BaseException as e:
            errors.append(f"thread {i}: {e!r}")

    ts = [threading.Thread(target=worker, args=(i,)) for i in range(len(calls))]
    for t in ts: t.start()
    for t in ts: t.join()
    if errors:
        print("\\n".join(errors)); sys.exit(1)
    torch.cuda.synchronize()
    bad = 0
    for i, c in enumerate(calls):
        ref = flat(c())
        torch.cuda.synchronize()
        for a, b in zip(results[i], ref):
            same = torch.equal(a, b)
            print(f"call {i}: shape {tuple(a.shape)} bitwise equal: {same}", flush=True)
            bad += not same
    print("OK" if bad == 0 else "MISMATCH", flush=True)
    sys.exit(1 if bad else 0)
""")


@pytest.mark.gpu
def test_concurrent_calls_from_threads_match_serial_calls():
    r = subprocess.run([sys.executable, "-c", SCRIPT], cwd=ROOT, capture_output=True, text=True,
                       timeout=150, env={**os.environ, "PYTHONPATH": ROOT})
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-3000:]
    assert r.stdout.strip().splitlines()[-1] == "OK", out[-3000:]
