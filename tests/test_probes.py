"""The microbenchmarks bench.py compares its rates with (libgqa_probes.so): the library
exports its five functions, the FLOP count is the stated formula, and on a GPU the read
probe folds every 16-byte chunk exactly once (checked bit for bit against the CPU)."""
import ctypes
import os

import numpy as np
import pytest

from grouped_query_attention_02_amd import build as gbuild


@pytest.fixture(scope="module")
def probes(built_lib):
    if not os.path.exists(gbuild.PROBES_LIB):
        gbuild.build()
    import torch  # noqa: F401  (torch's HIP runtime first; see _lib.load)
    lib = ctypes.CDLL(gbuild.PROBES_LIB, mode=ctypes.RTLD_LOCAL)
    lib.gqa_probe_mfma_flops.argtypes = [ctypes.c_int, ctypes.c_int]
    lib.gqa_probe_mfma_flops.restype = ctypes.c_double
    lib.gqa_probe_mfma_bf16.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                        ctypes.c_void_p]
    lib.gqa_probe_mfma_bf16_rand.argtypes = lib.gqa_probe_mfma_bf16.argtypes
    lib.gqa_probe_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p,
                                   ctypes.c_int, ctypes.c_void_p]
    lib.gqa_probe_read_nt.argtypes = lib.gqa_probe_read.argtypes
    return lib


def test_probe_exports_and_flop_count(probes):
    for n in ("gqa_probe_mfma_bf16", "gqa_probe_mfma_bf16_rand", "gqa_probe_read",
              "gqa_probe_read_nt", "gqa_probe_mfma_flops"):
        assert getattr(probes, n) is not None
    # blocks x 4 waves x iters x 4 chains x (2 x 32 x 32 x 16)
    assert probes.gqa_probe_mfma_flops(3, 5) == 3 * 4 * 5 * 4 * 2 * 32 * 32 * 16
    # invalid arguments are refused before any launch
    assert probes.gqa_probe_mfma_bf16(0, 1, None, None) != 0
    assert probes.gqa_probe_mfma_bf16_rand(1, 6, None, None) != 0   # iters not a multiple of 4
    assert probes.gqa_probe_read(None, 16, None, 1, None) != 0
    assert probes.gqa_probe_read_nt(None, 16, None, 1, None) != 0


@pytest.mark.gpu
def test_read_probe_folds_every_chunk(probes):
    import torch
    rng = np.random.default_rng(5)
    n16, blocks = 100003, 7
    host = rng.integers(0, 2**32, size=(n16, 4), dtype=np.uint64).astype(np.uint32)
    buf = torch.from_numpy(host.view(np.int32)).cuda()
    out = torch.zeros(blocks * 256, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    want = np.bitwise_xor.reduce(host.reshape(-1))
    for fn in (probes.gqa_probe_read, probes.gqa_probe_read_nt):
        out.zero_()
        assert fn(buf.data_ptr(), n16, out.data_ptr(), blocks, stream) == 0
        torch.cuda.synchronize()
        got = np.bitwise_xor.reduce(out.cpu().numpy().view(np.uint32))
        assert got == want


@pytest.mark.gpu
def test_mfma_probe_runs(probes):
    import torch
    out = torch.full((2 * 256,), float("nan"), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    assert probes.gqa_probe_mfma_bf16(2, 10, out.data_ptr(), stream) == 0
    torch.cuda.synchronize()
    assert torch.isfinite(out).all()


@pytest.mark.gpu
def test_mfma_probe_random_operands_runs(probes):
    import torch
    out = torch.full((2 * 256,), float("nan"), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    assert probes.gqa_probe_mfma_bf16_rand(2, 8, out.data_ptr(), stream) == 0
    torch.cuda.synchronize()
    assert torch.isfinite(out).all() and (out != 0).any()
