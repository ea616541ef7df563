"""Every entry point under HIP graph capture: the library allocates nothing, never
synchronises and enqueues only kernel launches on the caller's stream, so a whole step
(prefill and decode calls, the workspace decode and the allocation-free decode) can be
captured once and replayed. Each replay runs on new inputs copied into the captured
buffers, with eager calls and synchronisations between replays, and must give outputs
bitwise equal to eager calls on the same inputs (the kernels are deterministic). A
fresh process whose first library calls happen under capture replays them correctly too."""
import sys

import pytest
import torch

import grouped_query_attention_02_amd as gqa

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu(built_lib):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    gqa.load()


def _fill(bufs, seed):
    """New seeded inputs, copied into the existing device buffers."""
    g = torch.Generator().manual_seed(seed)
    for t in bufs:
        t.copy_(torch.randn(t.shape, generator=g).to(t.dtype))


class Step:
    """Five calls over fixed device buffers: bf16 causal d=128 and ragged bidirectional d=64
    prefills, an fp32 prefill, a ragged multi-query decode with a caller workspace (split
    partials and the merge kernel) and the same decode through the allocation-free entry."""

    def __init__(self, dev):
        bf, f32 = torch.bfloat16, torch.float32
        self.pc = [torch.empty((2, 320, 8, 128), dtype=bf, device=dev),
                   torch.empty((2, 320, 2, 128), dtype=bf, device=dev),
                   torch.empty((2, 320, 2, 128), dtype=bf, device=dev)]
        self.pb = [torch.empty((3, 200, 12, 64), dtype=bf, device=dev),
                   torch.empty((3, 200, 3, 64), dtype=bf, device=dev),
                   torch.empty((3, 200, 3, 64), dtype=bf, device=dev)]
        self.pf = [torch.empty((1, 64, 4, 32), dtype=f32, device=dev),
                   torch.empty((1, 64, 2, 32), dtype=f32, device=dev),
                   torch.empty((1, 64, 2, 32), dtype=f32, device=dev)]
        self.dc = [torch.empty((5, 32, 128), dtype=bf, device=dev),
                   torch.empty((5, 1, 3000, 128), dtype=bf, device=dev),
                   torch.empty((5, 1, 3000, 128), dtype=bf, device=dev)]
        self.pc_lens = torch.tensor([320, 257], dtype=torch.int32, device=dev)
        self.pb_lens = torch.tensor([200, 7, 130], dtype=torch.int32, device=dev)
        self.dc_lens = torch.tensor([3000, 1, 1777, 640, 2048], dtype=torch.int32, device=dev)
        need = gqa.decode_workspace_bytes(5, 32, 1, 128, 3000, 0)
        self.ws = torch.empty(need, dtype=torch.uint8, device=dev)
        self.outs = [torch.empty_like(self.pc[0]), torch.empty_like(self.pb[0]),
                     torch.empty_like(self.pf[0]), torch.empty_like(self.dc[0]),
                     torch.empty_like(self.dc[0])]
        self.lses = [torch.empty((2, 8, 320), dtype=f32, device=dev),
                     torch.empty((5, 32), dtype=f32, device=dev),
                     torch.empty((5, 32), dtype=f32, device=dev)]

    def inputs(self):
        return self.pc + self.pb + self.pf + self.dc

    def run(self):
        o, l = self.outs, self.lses
        gqa.prefill(*self.pc, causal=True, seqlens=self.pc_lens, return_lse=True, out=o[0],
                    lse_out=l[0])
        gqa.prefill(*self.pb, causal=False, seqlens=self.pb_lens, out=o[1])
        gqa.prefill(*self.pf, causal=False, out=o[2])
        gqa.decode(*self.dc, self.dc_lens, workspace=self.ws, return_lse=True, out=o[3],
                   lse_out=l[1])
        gqa.decode_noalloc(*self.dc, self.dc_lens, o[4], lse_out=l[2])

    def results(self):
        return [t.clone() for t in self.outs + self.lses]


def test_step_replays_match_eager_calls():
    dev = torch.device("cuda:0")
    step = Step(dev)
    _fill(step.inputs(), 11)
    # warm-up on a side stream (first calls set up the library's per-device state)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step.run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step.run()
    torch.cuda.synchronize()

    other = Step(dev)  # eager work between replays, on buffers of its own
    for rep, seed in enumerate((21, 22, 23, 24)):
        _fill(step.inputs(), seed)
        step.run()                       # eager reference on these inputs
        torch.cuda.synchronize()
        want = step.results()
        for t in step.outs + step.lses:  # poison, so a replay that writes nothing fails
            t.fill_(float("nan"))
        _fill(other.inputs(), 100 + seed)
        other.run()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = step.results()
        same = [torch.equal(a, b) for a, b in zip(got, want)]
        _say(f"  replay {rep}: outputs bitwise equal to eager calls: {same}")
        assert all(same)


_COLD_CAPTURE = r'''
import sys
import torch
import grouped_query_attention_02_amd as gqa
dev = torch.device("cuda:0")
g = torch.Generator().manual_seed(5)
def rnd(shape):
    return torch.randn(shape, generator=g).to(torch.bfloat16).to(dev)
q, k, v = rnd((2, 200, 8, 128)), rnd((2, 200, 2, 128)), rnd((2, 200, 2, 128))
dq, kc, vc = rnd((3, 16, 128)), rnd((3, 2, 900, 128)), rnd((3, 2, 900, 128))
lens = torch.tensor([900, 5, 444], dtype=torch.int32, device=dev)
o1, o2, o3 = torch.empty_like(q), torch.empty_like(dq), torch.empty_like(dq)
ws = torch.empty(gqa.decode_workspace_bytes(3, 16, 2, 128, 900, 0), dtype=torch.uint8,
                 device=dev)
torch.cuda.synchronize()
graph = torch.cuda.CUDAGraph()
with torch.cuda.graph(graph):   # the library's first calls in this process
    gqa.prefill(q, k, v, causal=True, out=o1)
    gqa.decode(dq, kc, vc, lens, workspace=ws, out=o2)
    gqa.decode_noalloc(dq, kc, vc, lens, o3)
graph.replay()
torch.cuda.synchronize()
r1, r2 = gqa.prefill(q, k, v, causal=True), gqa.decode(dq, kc, vc, lens)
torch.cuda.synchronize()
ok = torch.equal(o1, r1) and torch.equal(o2, r2) and torch.equal(o3, r2)
print("cold capture replay equals eager:", ok, flush=True)
sys.exit(0 if ok else 1)
'''


def test_first_calls_captured_in_fresh_process():
    """The per-device set-up done on a device's first call (CU count, kernel attributes,
    occupancy, the scratch address) is allowed under stream capture: a fresh process whose
    first library calls are inside a graph capture replays them correctly."""
    import os
    import subprocess
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    env = dict(os.environ, PYTHONPATH=root + os.pathsep + os.environ.get("PYTHONPATH", ""))
    r = subprocess.run([sys.executable, "-c", _COLD_CAPTURE], cwd=root, env=env,
                       capture_output=True, text=True, timeout=110)
    _say(r.stdout.strip())
    assert r.returncode == 0, r.stderr[-2000:]
