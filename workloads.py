"""Seeded synthetic inputs for grouped-query attention workloads.

This module is shared by the tests, the benchmark and the smoke check. It
holds shapes, seeds and random draws only, none of the attention arithmetic:
both the oracle and the HIP library receive exactly the tensors built here.

Recipe (fixed draw order per workload: lengths, then Q, then K, then V):
  * a ``torch.Generator`` seeded with the workload's seed (CPU by default; the
    benchmark may pass ``device="cuda"`` to draw the same distributions on the
    GPU, which gives different numbers from the same seed);
  * lengths: ``torch.randint(lo, hi + 1)`` (inclusive range), int32;
  * values: ``torch.randn`` in float32, drawn one leading-index slice at a time
    (one batch entry per call), multiplied by the workload's value scale
    (0.5 is exact in binary), then rounded to the storage dtype (bf16 rounds to
    nearest even);
  * decode cache rows at or past a sequence's length hold zeros, or NaN when
    ``poison=True`` (nothing past the length may reach the output);
  * prefill K/V rows at or past a sequence's key length are ordinary draws,
    or NaN when ``poison=True``.

The workloads mirror the pages' settings: a BERT-base-shaped bidirectional
prefill (12 query heads over 3 K/V heads, head size 64, sequence 1024, batch
32), a Llama-style causal prefill, a decode over a uniform 8k cache with 64
query heads over 8 K/V heads, and a multi-query decode over ragged caches.
No dataset items are used.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field, replace
from typing import Optional, Tuple

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    kind: str                 # "prefill" or "decode"
    dtype: str                # "f32" or "bf16"
    B: int
    Hq: int
    Hkv: int
    d: int
    S: int = 0                # prefill sequence length
    max_len: int = 0          # decode cache capacity
    causal: bool = False
    lens: Optional[Tuple[int, int]] = None   # inclusive uniform range of valid lengths
    value_scale: float = 1.0
    seed: int = 0
    description: str = ""

    @property
    def g(self) -> int:
        return self.Hq // self.Hkv

    @property
    def softmax_scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == "f32" else torch.bfloat16

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


WORKLOADS = {
    "tiny_f32_prefill": Workload(
        name="tiny_f32_prefill", kind="prefill", dtype="f32", B=1, S=64, Hq=4, Hkv=2, d=32,
        causal=False, lens=None, seed=101,
        description="fp32 non-causal prefill, batch 1, seq 64, 4 query heads over 2 K/V heads, d 32"),
    "bert_base_prefill": Workload(
        name="bert_base_prefill", kind="prefill", dtype="bf16", B=32, S=1024, Hq=12, Hkv=3, d=64,
        causal=False, lens=(512, 1024), seed=102,
        description="bf16 bidirectional prefill, batch 32, seq 1024, 12 query heads over 3 K/V "
                    "heads, d 64, key lengths uniform in [512, 1024]"),
    "llama_causal_prefill": Workload(
        name="llama_causal_prefill", kind="prefill", dtype="bf16", B=4, S=4096, Hq=32, Hkv=8,
        d=128, causal=True, lens=None, value_scale=0.5, seed=103,
        description="bf16 causal prefill, batch 4, seq 4096, 32 query heads over 8 K/V heads, "
                    "d 128, values N(0,1) x 0.5"),
    "gqa_decode_8k": Workload(
        name="gqa_decode_8k", kind="decode", dtype="bf16", B=64, Hq=64, Hkv=8, d=128,
        max_len=8192, lens=(8192, 8192), seed=104,
        description="bf16 decode, 64 sequences, 64 query heads over 8 K/V heads, d 128, "
                    "every cache 8192 long"),
    "mqa_ragged_decode": Workload(
        name="mqa_ragged_decode", kind="decode", dtype="bf16", B=32, Hq=32, Hkv=1, d=128,
        max_len=32768, lens=(1024, 32768), seed=105,
        description="bf16 multi-query decode, 32 sequences, 32 query heads over 1 K/V head, "
                    "d 128, cache lengths uniform in [1024, 32768]"),
}

ORDER = ["tiny_f32_prefill", "bert_base_prefill", "llama_causal_prefill",
         "gqa_decode_8k", "mqa_ragged_decode"]


def _gen(seed: int, device: str) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def _draw(shape, gen, device, dtype, value_scale):
    """randn in float32, one leading-index slice per call, scaled, rounded to dtype."""
    out = torch.empty(shape, dtype=dtype, device=device)
    for i in range(shape[0]):
        x = torch.randn(shape[1:], generator=gen, dtype=torch.float32, device=device)
        if value_scale != 1.0:
            x.mul_(value_scale)
        out[i].copy_(x)
    return out


def _lengths(w: Workload, gen, device) -> Optional[torch.Tensor]:
    if w.lens is None:
        return None
    lo, hi = w.lens
    return torch.randint(lo, hi + 1, (w.B,), generator=gen, dtype=torch.int32, device=device)


def make_prefill(w: Workload, seed: Optional[int] = None, *, device: str = "cpu",
                 poison: bool = False):
    """Returns dict(q, k, v, seqlens) with q [B,S,Hq,d], k/v [B,S,Hkv,d], seqlens int32 [B] or None."""
    assert w.kind == "prefill"
    gen = _gen(w.seed if seed is None else seed, device)
    seqlens = _lengths(w, gen, device)
    dt = w.torch_dtype
    q = _draw((w.B, w.S, w.Hq, w.d), gen, device, dt, w.value_scale)
    k = _draw((w.B, w.S, w.Hkv, w.d), gen, device, dt, w.value_scale)
    v = _draw((w.B, w.S, w.Hkv, w.d), gen, device, dt, w.value_scale)
    if poison and seqlens is not None:
        for b in range(w.B):
            L = int(seqlens[b])
            k[b, L:] = float("nan")
            v[b, L:] = float("nan")
    return dict(q=q, k=k, v=v, seqlens=seqlens)


def make_decode(w: Workload, seed: Optional[int] = None, *, device: str = "cpu",
                poison: bool = False):
    """Returns dict(q, k_cache, v_cache, lens): q [B,Hq,d], caches [B,Hkv,max_len,d], lens int32 [B]."""
    assert w.kind == "decode"
    gen = _gen(w.seed if seed is None else seed, device)
    lens = _lengths(w, gen, device)
    if lens is None:
        lens = torch.full((w.B,), w.max_len, dtype=torch.int32, device=device)
    dt = w.torch_dtype
    q = _draw((w.B, w.Hq, w.d), gen, device, dt, w.value_scale)
    kc = _draw((w.B, w.Hkv, w.max_len, w.d), gen, device, dt, w.value_scale)
    vc = _draw((w.B, w.Hkv, w.max_len, w.d), gen, device, dt, w.value_scale)
    fill = float("nan") if poison else 0.0
    lens_host = lens.cpu()
    for b in range(w.B):
        L = int(lens_host[b])
        if L < w.max_len:
            kc[b, :, L:] = fill
            vc[b, :, L:] = fill
    return dict(q=q, k_cache=kc, v_cache=vc, lens=lens)
