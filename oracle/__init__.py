"""fp64 CPU oracle for grouped-query attention.

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
``cpu_baseline`` leg are the only callers. The product path (the HIP library
and its binding) never imports this package, and this package never imports
the product path.

The arithmetic lives in ``oracle.c`` (plain C, IEEE double, OpenMP over rows);
this module only compiles it with gcc, marshals numpy/torch CPU arrays into it
and returns float64 numpy arrays. See the header of ``oracle.c`` for what is
computed and which passage of the pages each step follows.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

F64, F32, BF16 = 0, 1, 2

_lib = None


# A sanitizer build of oracle.c (see build_sanitized) is loaded instead of liboracle.so when
# this environment variable names it; the process must then have the matching runtime
# (gcc's libasan) loaded first, e.g. through LD_PRELOAD.
SANITIZED_ENV = "ORACLE_SANITIZED_LIB"

SANITIZE_FLAGS = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
                  "-fno-sanitize-recover=all"]


def build_sanitized(path: str) -> str:
    """Compile oracle.c with AddressSanitizer and UndefinedBehaviorSanitizer into `path`
    (host code only; the same arithmetic flags as build())."""
    cmd = ["gcc", *SANITIZE_FLAGS, "-fopenmp", "-fPIC", "-shared", "-std=c11",
           "-fno-fast-math", "-ffp-contract=off", _SRC, "-o", path, "-lm"]
    subprocess.run(cmd, check=True)
    return path


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so with gcc (-O2, OpenMP, no fast-math)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + f".tmp{os.getpid()}"
        cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11",
               "-fno-fast-math", "-ffp-contract=off", _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        path = os.environ.get(SANITIZED_ENV)
        if not path:
            path = _LIB
            if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
                build(force=True)
        lib = ctypes.CDLL(path)
        vp, i32, i64, dbl = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_double
        lib.oracle_prefill_rows.argtypes = [i32, vp, vp, vp, vp, i32, i32, i32, i32, i32,
                                            dbl, i32, vp, i64, vp, vp, vp, i32]
        lib.oracle_prefill.argtypes = [i32, vp, vp, vp, vp, i32, i32, i32, i32, i32,
                                       dbl, i32, vp, vp, i32]
        lib.oracle_decode_pairs.argtypes = [i32, vp, vp, vp, vp, i32, i32, i32, i32, i32,
                                            dbl, i32, i32, vp, i64, vp, vp, i32]
        lib.oracle_decode.argtypes = [i32, vp, vp, vp, vp, i32, i32, i32, i32, i32,
                                      dbl, vp, vp, i32]
        lib.oracle_prefill_rows_ex.argtypes = [i32, vp, vp, vp, vp, i32, i32, i32, i32, i32,
                                               dbl, i32, i32, vp, vp, i64, vp, vp, vp, i32]
        lib.oracle_prefill_ex.argtypes = [i32, vp, vp, vp, vp, i32, i32, i32, i32, i32,
                                          dbl, i32, i32, vp, vp, vp, i32]
        lib.oracle_decode_pairs_ex.argtypes = [i32, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32,
                                               i32, i32, i32, dbl, i32, vp, i32, i32, vp, i64,
                                               vp, vp, i32]
        lib.oracle_decode_ex.argtypes = [i32, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32,
                                         i32, i32, dbl, i32, vp, vp, vp, i32]
        lib.oracle_mean_pool_heads.argtypes = [i32, vp, i32, i32, i64, vp]
        lib.oracle_max_threads.argtypes = []
        for f in (lib.oracle_prefill_rows, lib.oracle_prefill, lib.oracle_decode_pairs,
                  lib.oracle_decode, lib.oracle_prefill_rows_ex, lib.oracle_prefill_ex,
                  lib.oracle_decode_pairs_ex, lib.oracle_decode_ex, lib.oracle_mean_pool_heads,
                  lib.oracle_max_threads):
            f.restype = ctypes.c_int
        _lib = lib
    return _lib


def max_threads() -> int:
    return int(_load().oracle_max_threads())


def _as_host(x):
    """Return (contiguous CPU buffer object, dtype code). Accepts numpy or torch CPU tensors.

    bf16 is passed as its raw 16-bit pattern; the C side decodes it exactly.
    """
    try:
        import torch
    except ImportError:  # pragma: no cover
        torch = None
    if torch is not None and isinstance(x, torch.Tensor):
        if x.device.type != "cpu":
            raise ValueError("the oracle takes host tensors only")
        x = x.contiguous()
        if x.dtype == torch.bfloat16:
            return x.view(torch.int16).numpy(), BF16
        if x.dtype == torch.float32:
            return x.numpy(), F32
        if x.dtype == torch.float64:
            return x.numpy(), F64
        raise TypeError(f"unsupported dtype {x.dtype}")
    x = np.ascontiguousarray(x)
    if x.dtype == np.float64:
        return x, F64
    if x.dtype == np.float32:
        return x, F32
    raise TypeError(f"unsupported dtype {x.dtype}")


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _lens(lens):
    if lens is None:
        return None
    try:
        import torch
        if isinstance(lens, torch.Tensor):
            lens = lens.cpu().numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.ascontiguousarray(np.asarray(lens, dtype=np.int32))


def _slopes(alibi_slopes, Hq):
    if alibi_slopes is None:
        return None
    try:
        import torch
        if isinstance(alibi_slopes, torch.Tensor):
            alibi_slopes = alibi_slopes.detach().cpu().double().numpy()
    except ImportError:  # pragma: no cover
        pass
    a = np.ascontiguousarray(np.asarray(alibi_slopes, dtype=np.float64).reshape(-1))
    if a.shape != (Hq,):
        raise ValueError(f"alibi_slopes must have {Hq} entries")
    return a


def _table(block_table):
    if block_table is None:
        return None
    try:
        import torch
        if isinstance(block_table, torch.Tensor):
            block_table = block_table.cpu().numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.ascontiguousarray(np.asarray(block_table, dtype=np.int32))


def prefill(q, k, v, *, scale: float, causal: bool = False, seqlens=None, window: int = 0,
            alibi_slopes=None, n_threads: int = 0):
    """Whole prefill. q [B,S,Hq,d], k/v [B,S,Hkv,d] -> (o [B,S,Hq,d] f64, lse [B,Hq,S] f64).

    window > 0 keeps keys j > i - window; alibi_slopes [Hq] adds -slope_h * |i - j|.
    """
    qa, qt = _as_host(q)
    ka, kt = _as_host(k)
    va, vt = _as_host(v)
    if not (qt == kt == vt):
        raise TypeError("q, k, v must share a dtype")
    B, S, Hq, d = qa.shape
    Hkv = ka.shape[2]
    if ka.shape != (B, S, Hkv, d) or va.shape != ka.shape:
        raise ValueError("shape mismatch")
    sl = _lens(seqlens)
    sa = _slopes(alibi_slopes, Hq)
    o = np.empty((B, S, Hq, d), np.float64)
    lse = np.empty((B, Hq, S), np.float64)
    rc = _load().oracle_prefill_ex(qt, _ptr(qa), _ptr(ka), _ptr(va), _ptr(sl), B, S, Hq, Hkv, d,
                                   float(scale), int(bool(causal)), int(window), _ptr(sa),
                                   _ptr(o), _ptr(lse), int(n_threads))
    if rc != 0:
        raise ValueError(f"oracle_prefill rejected the arguments (rc={rc})")
    return o, lse


def prefill_rows(q, k, v, rows, *, scale: float, causal: bool = False, seqlens=None,
                 window: int = 0, alibi_slopes=None, want_probs: bool = False,
                 n_threads: int = 0):
    """Selected rows. rows: int array [n, 3] of (b, h, i). Returns o [n,d], lse [n] (, p [n,S])."""
    qa, qt = _as_host(q)
    ka, _ = _as_host(k)
    va, _ = _as_host(v)
    B, S, Hq, d = qa.shape
    Hkv = ka.shape[2]
    r = np.ascontiguousarray(np.asarray(rows, dtype=np.int64).reshape(-1, 3))
    n = r.shape[0]
    o = np.empty((n, d), np.float64)
    lse = np.empty((n,), np.float64)
    p = np.empty((n, S), np.float64) if want_probs else None
    sl = _lens(seqlens)
    sa = _slopes(alibi_slopes, Hq)
    rc = _load().oracle_prefill_rows_ex(qt, _ptr(qa), _ptr(ka), _ptr(va), _ptr(sl), B, S, Hq,
                                        Hkv, d, float(scale), int(bool(causal)), int(window),
                                        _ptr(sa), _ptr(r), n, _ptr(o), _ptr(lse), _ptr(p),
                                        int(n_threads))
    if rc != 0:
        raise ValueError(f"oracle_prefill_rows rejected the arguments (rc={rc})")
    return (o, lse, p) if want_probs else (o, lse)


def _decode_shapes(qa, ka, block_table, page_size):
    B, Hq, d = qa.shape
    Hkv = ka.shape[1]
    bt = _table(block_table)
    if bt is None:
        return B, Hq, d, Hkv, ka.shape[2], None, 0, 0, 0
    if ka.shape[2] != page_size or bt.ndim != 2 or bt.shape[0] != B:
        raise ValueError("paged cache: pools [num_pages, Hkv, page_size, d], table [B, blocks]")
    return B, Hq, d, Hkv, bt.shape[1] * page_size, bt, page_size, bt.shape[1], ka.shape[0]


def decode(q, k_cache, v_cache, *, scale: float, lens=None, window: int = 0, alibi_slopes=None,
           block_table=None, page_size: int = 0, n_threads: int = 0):
    """Whole decode. q [B,Hq,d], caches [B,Hkv,max_len,d] -> (o [B,Hq,d], lse [B,Hq]).

    With block_table [B, blocks] the caches are page pools [num_pages, Hkv, page_size, d].
    """
    qa, qt = _as_host(q)
    ka, _ = _as_host(k_cache)
    va, _ = _as_host(v_cache)
    B, Hq, d, Hkv, max_len, bt, P, MB, NP = _decode_shapes(qa, ka, block_table, page_size)
    sl = _lens(lens)
    sa = _slopes(alibi_slopes, Hq)
    o = np.empty((B, Hq, d), np.float64)
    lse = np.empty((B, Hq), np.float64)
    rc = _load().oracle_decode_ex(qt, _ptr(qa), _ptr(ka), _ptr(va), _ptr(sl), _ptr(bt), P, MB, NP,
                                  B, Hq, Hkv, d, max_len, float(scale), int(window), _ptr(sa),
                                  _ptr(o), _ptr(lse), int(n_threads))
    if rc != 0:
        raise ValueError(f"oracle_decode rejected the arguments (rc={rc})")
    return o, lse


def decode_pairs(q, k_cache, v_cache, pairs, *, scale: float, lens=None, key_range=None,
                 window: int = 0, alibi_slopes=None, block_table=None, page_size: int = 0,
                 n_threads: int = 0):
    """Selected (b, h) pairs, optionally restricted to keys in [lo, hi)."""
    qa, qt = _as_host(q)
    ka, _ = _as_host(k_cache)
    va, _ = _as_host(v_cache)
    B, Hq, d, Hkv, max_len, bt, P, MB, NP = _decode_shapes(qa, ka, block_table, page_size)
    lo, hi = (0, max_len) if key_range is None else key_range
    pr = np.ascontiguousarray(np.asarray(pairs, dtype=np.int64).reshape(-1, 2))
    n = pr.shape[0]
    o = np.empty((n, d), np.float64)
    lse = np.empty((n,), np.float64)
    sl = _lens(lens)
    sa = _slopes(alibi_slopes, Hq)
    rc = _load().oracle_decode_pairs_ex(qt, _ptr(qa), _ptr(ka), _ptr(va), _ptr(sl), _ptr(bt), P,
                                        MB, NP, B, Hq, Hkv, d, max_len, float(scale),
                                        int(window), _ptr(sa), int(lo), int(hi), _ptr(pr), n,
                                        _ptr(o), _ptr(lse), int(n_threads))
    if rc != 0:
        raise ValueError(f"oracle_decode_pairs rejected the arguments (rc={rc})")
    return o, lse


def mean_pool_heads(w, num_groups: int):
    """[H, ...] per-head projection weights -> [G, ...] group means (contiguous groups)."""
    wa, wt = _as_host(w)
    H = wa.shape[0]
    per_head = int(np.prod(wa.shape[1:])) if wa.ndim > 1 else 1
    out = np.empty((num_groups,) + tuple(wa.shape[1:]), np.float64)
    rc = _load().oracle_mean_pool_heads(wt, _ptr(wa), H, int(num_groups), per_head, _ptr(out))
    if rc != 0:
        raise ValueError(f"oracle_mean_pool_heads rejected the arguments (rc={rc})")
    return out
