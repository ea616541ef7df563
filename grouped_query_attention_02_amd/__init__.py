"""Grouped-query attention forward pass for MI355X (gfx950): Python binding of libgqa.so.

The binding only checks tensors and passes pointers, sizes and the current HIP
stream to the C ABI declared in include/gqa.h; every step of the computation
runs in the library's HIP kernels. There is no fallback: if libgqa.so is not
built, every call raises.

    import grouped_query_attention_02_amd as gqa
    o = gqa.prefill(q, k, v, causal=False, seqlens=lens)          # q [B,S,Hq,d]
    o = gqa.decode(q, k_cache, v_cache, cache_lens=lens)           # q [B,Hq,d]
"""
from __future__ import annotations

import math
from typing import Optional

from ._lib import (GQA_DTYPE_BF16, GQA_DTYPE_F32, GQA_OK, GQAError, header_functions, load,
                   status_string)

__all__ = ["prefill", "decode", "decode_noalloc", "decode_workspace_bytes", "decode_num_workgroups",
           "mean_pool_heads", "version", "status_string", "GQAError", "load", "header_functions"]


def version() -> int:
    return int(load().gqa_version())


def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return GQA_DTYPE_BF16
    if t.dtype == torch.float32:
        return GQA_DTYPE_F32
    raise TypeError(f"unsupported dtype {t.dtype}; use bfloat16 or float32")


def _check(t, name, ndim, dtype=None):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dimensions, got shape {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")


def _check_buffer(t, name, shape, dtype, device):
    """A caller-provided output buffer: the kernels write every element of `shape`
    unconditionally, so anything smaller, of another type or elsewhere is rejected before
    any launch."""
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if not t.is_cuda or t.device != device:
        raise ValueError(f"{name} must be on {device}, got {t.device}")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _check_workspace(ws, need, device):
    torch = _torch()
    if not isinstance(ws, torch.Tensor):
        raise TypeError("workspace must be a torch tensor")
    if not ws.is_cuda or ws.device != device:
        raise ValueError(f"workspace must be on {device}, got {ws.device}")
    if ws.dtype != torch.uint8 or ws.dim() != 1 or not ws.is_contiguous():
        raise ValueError("workspace must be a contiguous 1-D uint8 tensor")
    if ws.numel() < need:
        raise ValueError(f"workspace holds {ws.numel()} bytes; this call needs {need}")


def _lens_arg(x, B, device, name):
    torch = _torch()
    if x is None:
        return None, 0
    if not isinstance(x, torch.Tensor):
        x = torch.as_tensor(x, dtype=torch.int32)
    if x.device != device:
        x = x.to(device)
    if x.dtype != torch.int32:
        x = x.to(torch.int32)
    x = x.contiguous()
    if x.shape != (B,):
        raise ValueError(f"{name} must have shape ({B},)")
    return x, x.data_ptr()


def _slopes_arg(x, Hq, device):
    """ALiBi slopes as a contiguous fp32 [Hq] device tensor (or None)."""
    torch = _torch()
    if x is None:
        return None, 0
    if not isinstance(x, torch.Tensor):
        x = torch.as_tensor(x, dtype=torch.float32)
    x = x.to(device=device, dtype=torch.float32).contiguous()
    if x.shape != (Hq,):
        raise ValueError(f"alibi_slopes must have shape ({Hq},)")
    return x, x.data_ptr()


def _stream_ptr(device) -> int:
    torch = _torch()
    return torch.cuda.current_stream(device).cuda_stream


def prefill(q, k, v, *, causal: bool = False, softmax_scale: Optional[float] = None,
            seqlens=None, window: int = 0, alibi_slopes=None, return_lse: bool = False,
            out=None, lse_out=None):
    """Attention of every query row over the valid keys of its sequence.

    q [B, S, Hq, d], k/v [B, S, Hkv, d] (contiguous, same dtype: bfloat16 or float32,
    on the GPU), seqlens int32 [B] valid key lengths or None. window > 0 (causal
    only) keeps keys j > i - window; alibi_slopes [Hq] subtracts slope_h * |i - j|
    from the scaled scores. Returns o [B, S, Hq, d] (and lse [B, Hq, S] float32 when
    return_lse).
    """
    torch = _torch()
    _check(q, "q", 4)
    _check(k, "k", 4, q.dtype)
    _check(v, "v", 4, q.dtype)
    if k.device != q.device or v.device != q.device:
        raise ValueError("q, k and v must be on the same device")
    B, S, Hq, d = q.shape
    Hkv = k.shape[2]
    if tuple(k.shape) != (B, S, Hkv, d) or tuple(v.shape) != tuple(k.shape):
        raise ValueError(f"k and v must be [B, S, Hkv, d] = [{B}, {S}, Hkv, {d}]")
    if Hkv <= 0 or Hq % Hkv != 0:
        raise ValueError(f"num_heads_q ({Hq}) must be divisible by num_heads_kv ({Hkv})")
    scale = 1.0 / math.sqrt(d) if softmax_scale is None else float(softmax_scale)
    if out is None:
        out = torch.empty_like(q)
    else:
        _check_buffer(out, "out", q.shape, q.dtype, q.device)
    lse_ptr = 0
    if return_lse:
        if lse_out is None:
            lse_out = torch.empty((B, Hq, S), dtype=torch.float32, device=q.device)
        else:
            _check_buffer(lse_out, "lse_out", (B, Hq, S), torch.float32, q.device)
        lse_ptr = lse_out.data_ptr()
    elif lse_out is not None:
        raise ValueError("lse_out is given but return_lse is False")
    lens, lens_ptr = _lens_arg(seqlens, B, q.device, "seqlens")
    slopes, slopes_ptr = _slopes_arg(alibi_slopes, Hq, q.device)
    st = load().gqa_prefill_ex(_dtype_code(q), q.data_ptr(), k.data_ptr(), v.data_ptr(),
                               out.data_ptr(), lse_ptr or None, lens_ptr or None, B, S, Hq, Hkv,
                               d, scale, int(bool(causal)), int(window), slopes_ptr or None,
                               _stream_ptr(q.device))
    if st != GQA_OK:
        raise GQAError(st, "gqa_prefill_ex")
    return (out, lse_out) if return_lse else out


def decode_workspace_bytes(B: int, Hq: int, Hkv: int, d: int, max_len: int,
                           num_splits: int = 0) -> int:
    return int(load().gqa_decode_workspace_bytes(B, Hq, Hkv, d, max_len, num_splits))


def decode_num_workgroups(B: int, Hq: int, Hkv: int, max_len: int, num_splits: int = 0) -> int:
    return int(load().gqa_decode_num_workgroups(B, Hq, Hkv, max_len, num_splits))


def decode(q, k_cache, v_cache, cache_lens=None, *, softmax_scale: Optional[float] = None,
           num_splits: int = 0, window: int = 0, alibi_slopes=None, block_table=None,
           page_size: int = 0, return_lse: bool = False, workspace=None, out=None,
           lse_out=None):
    """One query token per sequence over its KV cache.

    q [B, Hq, d], k_cache/v_cache [B, Hkv, max_len, d] (bfloat16, contiguous, on the
    GPU), cache_lens int32 [B] or None (= max_len). With block_table (int32
    [B, max_blocks]) the caches are page pools [num_pages, Hkv, page_size, d] and
    key j of sequence b is row j % page_size of page block_table[b, j // page_size].
    window > 0 keeps only each sequence's last `window` keys; alibi_slopes [Hq]
    subtracts slope_h * (L_b - 1 - j). Returns o [B, Hq, d] (and lse [B, Hq] float32
    when return_lse). `workspace` (uint8 GPU tensor) is allocated when not given.
    """
    torch = _torch()
    _check(q, "q", 3)
    _check(k_cache, "k_cache", 4, q.dtype)
    _check(v_cache, "v_cache", 4, q.dtype)
    if k_cache.device != q.device or v_cache.device != q.device:
        raise ValueError("q, k_cache and v_cache must be on the same device")
    B, Hq, d = q.shape
    Hkv = k_cache.shape[1]
    if tuple(v_cache.shape) != tuple(k_cache.shape) or k_cache.shape[3] != d:
        raise ValueError("k_cache and v_cache must have the same shape, last dim d")
    table, table_ptr, max_blocks, num_pages = None, 0, 0, 0
    if block_table is None:
        max_len = k_cache.shape[2]
        if k_cache.shape[0] != B:
            raise ValueError("k_cache and v_cache must be [B, Hkv, max_len, d]")
    else:
        _check(block_table, "block_table", 2, torch.int32)
        if block_table.device != q.device:
            raise ValueError("block_table must be on q's device")
        if block_table.shape[0] != B or k_cache.shape[2] != page_size:
            raise ValueError("paged cache: pools [num_pages, Hkv, page_size, d], "
                             "block_table [B, max_blocks]")
        table, table_ptr = block_table, block_table.data_ptr()
        max_blocks, num_pages = block_table.shape[1], k_cache.shape[0]
        max_len = max_blocks * page_size
    if Hkv <= 0 or Hq % Hkv != 0:
        raise ValueError(f"num_heads_q ({Hq}) must be divisible by num_heads_kv ({Hkv})")
    scale = 1.0 / math.sqrt(d) if softmax_scale is None else float(softmax_scale)
    need = decode_workspace_bytes(B, Hq, Hkv, d, max_len, num_splits)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    else:
        _check_workspace(workspace, need, q.device)
    if out is None:
        out = torch.empty_like(q)
    else:
        _check_buffer(out, "out", q.shape, q.dtype, q.device)
    lse_ptr = 0
    if return_lse:
        if lse_out is None:
            lse_out = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
        else:
            _check_buffer(lse_out, "lse_out", (B, Hq), torch.float32, q.device)
        lse_ptr = lse_out.data_ptr()
    elif lse_out is not None:
        raise ValueError("lse_out is given but return_lse is False")
    lens, lens_ptr = _lens_arg(cache_lens, B, q.device, "cache_lens")
    slopes, slopes_ptr = _slopes_arg(alibi_slopes, Hq, q.device)
    st = load().gqa_decode_ex(_dtype_code(q), q.data_ptr(), k_cache.data_ptr(),
                              v_cache.data_ptr(), lens_ptr or None, table_ptr or None,
                              int(page_size) if table is not None else 0, max_blocks, num_pages,
                              out.data_ptr(), lse_ptr or None, B, Hq, Hkv, d, max_len, scale,
                              int(window), slopes_ptr or None, int(num_splits),
                              workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                              _stream_ptr(q.device))
    if st != GQA_OK:
        raise GQAError(st, "gqa_decode_ex")
    return (out, lse_out) if return_lse else out


DECODE_SCRATCH_BYTES = 32 << 20  # GQA_DECODE_SCRATCH_BYTES of include/gqa.h


def decode_noalloc(q, k_cache, v_cache, cache_lens, out, *, lse_out=None,
                   softmax_scale: Optional[float] = None, num_splits: int = 0, window: int = 0,
                   alibi_slopes=None, block_table=None, page_size: int = 0):
    """gqa_decode_noalloc: decode() with the library's static device scratch in place of a
    workspace. Nothing is allocated: `out` ([B, Hq, d], q's dtype) and, when wanted, `lse_out`
    ([B, Hq] float32) are the caller's; cache_lens and alibi_slopes must already be device
    tensors of the right dtype (int32 / float32) when given. Calls that overlap in time on one
    GPU share its scratch and must not be issued concurrently. Returns out (and lse_out)."""
    torch = _torch()
    _check(q, "q", 3)
    _check(k_cache, "k_cache", 4, q.dtype)
    _check(v_cache, "v_cache", 4, q.dtype)
    if k_cache.device != q.device or v_cache.device != q.device:
        raise ValueError("q, k_cache and v_cache must be on the same device")
    B, Hq, d = q.shape
    Hkv = k_cache.shape[1]
    if tuple(v_cache.shape) != tuple(k_cache.shape) or k_cache.shape[3] != d:
        raise ValueError("k_cache and v_cache must have the same shape, last dim d")
    table_ptr, max_blocks, num_pages = 0, 0, 0
    if block_table is None:
        max_len = k_cache.shape[2]
        if k_cache.shape[0] != B:
            raise ValueError("k_cache and v_cache must be [B, Hkv, max_len, d]")
    else:
        _check(block_table, "block_table", 2, torch.int32)
        if block_table.device != q.device or block_table.shape[0] != B \
                or k_cache.shape[2] != page_size:
            raise ValueError("paged cache: pools [num_pages, Hkv, page_size, d], "
                             "block_table [B, max_blocks] on q's device")
        table_ptr = block_table.data_ptr()
        max_blocks, num_pages = block_table.shape[1], k_cache.shape[0]
        max_len = max_blocks * page_size
    if Hkv <= 0 or Hq % Hkv != 0:
        raise ValueError(f"num_heads_q ({Hq}) must be divisible by num_heads_kv ({Hkv})")
    _check_buffer(out, "out", q.shape, q.dtype, q.device)
    if lse_out is not None:
        _check_buffer(lse_out, "lse_out", (B, Hq), torch.float32, q.device)
    lens_ptr = 0
    if cache_lens is not None:
        _check_buffer(cache_lens, "cache_lens", (B,), torch.int32, q.device)
        lens_ptr = cache_lens.data_ptr()
    slopes_ptr = 0
    if alibi_slopes is not None:
        _check_buffer(alibi_slopes, "alibi_slopes", (Hq,), torch.float32, q.device)
        slopes_ptr = alibi_slopes.data_ptr()
    scale = 1.0 / math.sqrt(d) if softmax_scale is None else float(softmax_scale)
    st = load().gqa_decode_noalloc(_dtype_code(q), q.data_ptr(), k_cache.data_ptr(),
                                   v_cache.data_ptr(), lens_ptr or None, table_ptr or None,
                                   int(page_size) if table_ptr else 0, max_blocks, num_pages,
                                   out.data_ptr(),
                                   lse_out.data_ptr() if lse_out is not None else None,
                                   B, Hq, Hkv, d, max_len, scale, int(window), slopes_ptr or None,
                                   int(num_splits), _stream_ptr(q.device))
    if st != GQA_OK:
        raise GQAError(st, "gqa_decode_noalloc")
    return (out, lse_out) if lse_out is not None else out


def mean_pool_heads(w, num_groups: int, *, out=None):
    """MHA -> GQA conversion: [H, ...] per-head weights (GPU, bfloat16 or float32,
    contiguous) -> [num_groups, ...], each group the mean of its H/num_groups
    consecutive heads."""
    torch = _torch()
    if not w.is_cuda or not w.is_contiguous():
        raise ValueError("w must be a contiguous GPU tensor")
    H = w.shape[0]
    per_head = w.numel() // H if H else 0
    if out is None:
        out = torch.empty((num_groups,) + tuple(w.shape[1:]), dtype=w.dtype, device=w.device)
    else:
        _check_buffer(out, "out", (num_groups,) + tuple(w.shape[1:]), w.dtype, w.device)
    st = load().gqa_mean_pool_heads(_dtype_code(w), w.data_ptr(), H, int(num_groups), per_head,
                                    out.data_ptr(), _stream_ptr(w.device))
    if st != GQA_OK:
        raise GQAError(st, "gqa_mean_pool_heads")
    return out
