"""ctypes loader for libgqa.so (argument marshalling only)."""
from __future__ import annotations

import ctypes
import os
import re
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libgqa.so")
HEADER = os.path.join(os.path.dirname(PKG), "include", "gqa.h")

GQA_OK = 0
GQA_ERR_INVALID_ARG = 1
GQA_ERR_UNSUPPORTED = 2
GQA_ERR_WORKSPACE = 3
GQA_ERR_HIP = 4
GQA_DTYPE_F32 = 0
GQA_DTYPE_BF16 = 1

_lib = None


class GQAError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {status_string(status)} (status {status})")


def header_functions():
    """Names of every function the public header declares."""
    with open(HEADER) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gqa_[a-z0-9_]+)\s*\(", text)))


# Another build of the library to load instead of the in-tree libgqa.so (the CPU tests use it
# for a build whose host code runs under sanitizers).
LIBRARY_ENV = "GQA_LIBRARY_PATH"


def _torch_runtime_first():
    """torch ships its own HIP runtime under the soname this library links
    (libamdhip64.so.7), and whichever copy a process loads first serves every library in it.
    When torch is installed it is imported before the library, so that torch's own libraries
    find the runtime they were built with (loaded the other way round, torch's first device
    allocation and the library's launches fail with no-device and out-of-memory errors)."""
    if "torch" in sys.modules:
        return
    import importlib.util
    if importlib.util.find_spec("torch") is not None:
        import torch  # noqa: F401


def load():
    """Load libgqa.so from the package directory; raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    path = os.environ.get(LIBRARY_ENV) or LIB_PATH
    _torch_runtime_first()
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is missing: build it with `python -m grouped_query_attention_02_amd.build` "
            "(there is no fallback path)")
    lib = ctypes.CDLL(path)
    vp, i32, f32, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    lib.gqa_version.argtypes = []
    lib.gqa_version.restype = i32
    lib.gqa_status_string.argtypes = [i32]
    lib.gqa_status_string.restype = ctypes.c_char_p
    lib.gqa_prefill.argtypes = [i32, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, f32, i32, vp]
    lib.gqa_prefill.restype = i32
    lib.gqa_decode_workspace_bytes.argtypes = [i32, i32, i32, i32, i32, i32]
    lib.gqa_decode_workspace_bytes.restype = sz
    lib.gqa_decode_num_workgroups.argtypes = [i32, i32, i32, i32, i32]
    lib.gqa_decode_num_workgroups.restype = i32
    lib.gqa_decode.argtypes = [i32, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, f32, i32,
                               vp, sz, vp]
    lib.gqa_decode.restype = i32
    lib.gqa_prefill_ex.argtypes = [i32, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, f32,
                                   i32, i32, vp, vp]
    lib.gqa_prefill_ex.restype = i32
    lib.gqa_decode_ex.argtypes = [i32, vp, vp, vp, vp, vp, i32, i32, i32, vp, vp, i32, i32, i32,
                                  i32, i32, f32, i32, vp, i32, vp, sz, vp]
    lib.gqa_decode_ex.restype = i32
    lib.gqa_decode_noalloc.argtypes = [i32, vp, vp, vp, vp, vp, i32, i32, i32, vp, vp, i32, i32,
                                       i32, i32, i32, f32, i32, vp, i32, vp]
    lib.gqa_decode_noalloc.restype = i32
    lib.gqa_mean_pool_heads.argtypes = [i32, vp, i32, i32, ctypes.c_int64, vp, vp]
    lib.gqa_mean_pool_heads.restype = i32
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load().gqa_status_string(int(status)).decode()
