"""CPU-only checks of the C ABI: the library loads, exports every declared symbol, and
rejects invalid arguments on the host before any HIP call (no kernel is launched here)."""
import ctypes
import math

import pytest

import grouped_query_attention_02_amd as gqa
from grouped_query_attention_02_amd import _lib

F32, BF16 = _lib.GQA_DTYPE_F32, _lib.GQA_DTYPE_BF16
INV, UNS, WS = _lib.GQA_ERR_INVALID_ARG, _lib.GQA_ERR_UNSUPPORTED, _lib.GQA_ERR_WORKSPACE

# Fake, 16-byte aligned addresses: every call below fails validation before any use.
P = 0x10000


@pytest.fixture(scope="module")
def lib(built_lib):
    return _lib.load()


def test_header_symbols_exported(lib):
    names = _lib.header_functions()
    assert set(names) >= {"gqa_prefill", "gqa_decode", "gqa_decode_workspace_bytes",
                          "gqa_decode_num_workgroups", "gqa_status_string", "gqa_version"}
    for n in names:
        assert getattr(lib, n) is not None
        ctypes.cast(getattr(lib, n), ctypes.c_void_p)


def test_version_and_status_strings(lib):
    assert gqa.version() == 10000
    assert gqa.status_string(0) == "ok"
    for s in (1, 2, 3, 4):
        assert gqa.status_string(s) not in ("ok", "unknown status")
    assert gqa.status_string(99) == "unknown status"


def _prefill(lib, dtype=BF16, q=P, k=P, v=P, o=P, lse=None, lens=None, B=2, S=64, Hq=8, Hkv=2,
             d=64, scale=0.125, causal=0):
    return lib.gqa_prefill(dtype, q, k, v, o, lse, lens, B, S, Hq, Hkv, d, scale, causal, None)


@pytest.mark.parametrize("kw,code", [
    (dict(Hq=6, Hkv=4), INV),            # heads not divisible (the pages' assertion)
    (dict(Hkv=0), INV),
    (dict(B=0), INV),
    (dict(S=0), INV),
    (dict(Hq=-4), INV),
    (dict(q=None), INV),
    (dict(o=None), INV),
    (dict(q=P + 2), INV),                # misaligned base
    (dict(v=P + 8), INV),
    (dict(lse=P + 2), INV),
    (dict(lens=P + 1), INV),
    (dict(causal=2), INV),
    (dict(scale=math.inf), INV),
    (dict(scale=math.nan), INV),
    (dict(d=48), UNS),
    (dict(d=256), UNS),
    (dict(dtype=7), UNS),
    (dict(dtype=F32, d=96), UNS),
])
def test_prefill_rejects(lib, kw, code):
    assert _prefill(lib, **kw) == code


def _decode(lib, dtype=BF16, q=P, k=P, v=P, lens=None, o=P, lse=None, B=4, Hq=32, Hkv=1, d=128,
            max_len=1000, scale=0.1, splits=0, ws=P, ws_bytes=None):
    if ws_bytes is None:
        ws_bytes = lib.gqa_decode_workspace_bytes(B, Hq, Hkv, d, max_len, splits)
    return lib.gqa_decode(dtype, q, k, v, lens, o, lse, B, Hq, Hkv, d, max_len, scale, splits,
                          ws, ws_bytes, None)


@pytest.mark.parametrize("kw,code", [
    (dict(Hq=12, Hkv=5), INV),
    (dict(B=0), INV),
    (dict(max_len=0), INV),
    (dict(splits=-1), INV),
    (dict(q=None), INV),
    (dict(k=P + 4), INV),
    (dict(scale=-math.inf), INV),
    (dict(dtype=F32), UNS),
    (dict(d=32), UNS),
    (dict(ws=None), WS),
    (dict(ws_bytes=16), WS),
    (dict(ws=P + 4), WS),
])
def test_decode_rejects(lib, kw, code):
    assert _decode(lib, **kw) == code


def test_decode_plan_rule(lib):
    """Auto rule: max(units, 256) shares, capped at one share per 32-key tile; n splits: n*units."""
    def units(B, Hq, Hkv):
        return B * Hkv * -(-(Hq // Hkv) // 32)
    # 32 sequences x 1 K/V head, 32 heads: 32 units -> 256 shares
    assert gqa.decode_num_workgroups(32, 32, 1, 32768, 0) == 256
    # 64 x 8 units (uniform 8k caches): one share per unit
    assert gqa.decode_num_workgroups(64, 64, 8, 8192, 0) == 512
    # tiny caches cap the shares at the tile count
    assert gqa.decode_num_workgroups(2, 8, 2, 40, 0) == units(2, 8, 2) * 2
    assert gqa.decode_num_workgroups(4, 8, 2, 4096, 3) == 3 * units(4, 8, 2)
    # 64 query heads over 1 K/V head: two blocks of 32 heads per sequence
    assert units(3, 64, 1) == 6
    assert gqa.decode_num_workgroups(3, 64, 1, 64, 0) == 6 * 2
    # workspace = (shares + units) slots x 32 heads x (d + 1) floats
    W, U = 256, 32
    assert gqa.decode_workspace_bytes(32, 32, 1, 128, 32768, 0) == (W + U) * 32 * 129 * 4
    assert gqa.decode_workspace_bytes(32, 32, 1, 128, 0, 0) == 0
    assert gqa.decode_workspace_bytes(32, 30, 4, 128, 100, 0) == 0


def _prefill_ex(lib, window=0, slopes=None, causal=1, **kw):
    a = dict(dtype=BF16, q=P, k=P, v=P, o=P, lse=None, lens=None, B=2, S=64, Hq=8, Hkv=2, d=64,
             scale=0.125)
    a.update(kw)
    return lib.gqa_prefill_ex(a["dtype"], a["q"], a["k"], a["v"], a["o"], a["lse"], a["lens"],
                              a["B"], a["S"], a["Hq"], a["Hkv"], a["d"], a["scale"], causal,
                              window, slopes, None)


@pytest.mark.parametrize("kw,code", [
    (dict(window=-1), INV),
    (dict(slopes=P + 2), INV),            # misaligned slope array
    (dict(window=8, causal=0), UNS),      # the window is the causal (sliding) form only
    (dict(window=4, Hq=6, Hkv=4), INV),   # the ordinary checks still apply
    (dict(window=4, d=48), UNS),
])
def test_prefill_ex_rejects(lib, kw, code):
    assert _prefill_ex(lib, **kw) == code


def _decode_ex(lib, table=None, page=0, blocks=0, pages=0, window=0, slopes=None, max_len=1024,
               ws_bytes=None, **kw):
    a = dict(dtype=BF16, q=P, k=P, v=P, lens=None, o=P, lse=None, B=4, Hq=32, Hkv=1, d=128,
             scale=0.1, splits=0, ws=P)
    a.update(kw)
    if ws_bytes is None:
        ws_bytes = lib.gqa_decode_workspace_bytes(a["B"], a["Hq"], a["Hkv"], a["d"], max_len,
                                                  a["splits"])
    return lib.gqa_decode_ex(a["dtype"], a["q"], a["k"], a["v"], a["lens"], table, page, blocks,
                             pages, a["o"], a["lse"], a["B"], a["Hq"], a["Hkv"], a["d"], max_len,
                             a["scale"], window, slopes, a["splits"], a["ws"], ws_bytes, None)


@pytest.mark.parametrize("kw,code", [
    (dict(window=-3), INV),
    (dict(slopes=P + 1), INV),
    (dict(table=P + 2, page=64, blocks=16, pages=100), INV),  # misaligned table
    (dict(table=P, page=48, blocks=16, pages=100, max_len=768), INV),  # page not a multiple of 32
    (dict(table=P, page=64, blocks=16, pages=100, max_len=1000), INV),  # max_len != blocks * page
    (dict(table=P, page=64, blocks=16, pages=0), INV),
    (dict(table=P, page=0, blocks=16, pages=10), INV),
    (dict(table=P, page=64, blocks=16, pages=10, dtype=F32), UNS),
    (dict(table=P, page=64, blocks=16, pages=10, ws=None), WS),
])
def test_decode_ex_rejects(lib, kw, code):
    assert _decode_ex(lib, **kw) == code


@pytest.mark.parametrize("kw,code", [
    (dict(H=12, G=5), INV),
    (dict(G=0), INV),
    (dict(per_head=12), INV),           # not a multiple of 8
    (dict(per_head=0), INV),
    (dict(w=None), INV),
    (dict(w=P + 4), INV),
    (dict(out=P + 8), INV),
    (dict(dtype=5), UNS),
])
def test_mean_pool_rejects(lib, kw, code):
    a = dict(dtype=BF16, w=P, H=12, G=3, per_head=64, out=P)
    a.update(kw)
    assert lib.gqa_mean_pool_heads(a["dtype"], a["w"], a["H"], a["G"], a["per_head"], a["out"],
                                   None) == code


def test_decode_noalloc_rejects_on_host(lib):
    """gqa_decode_noalloc checks every argument like gqa_decode_ex and refuses calls that need
    more than its static scratch, all before any HIP call (fake pointers are never used)."""
    def call(**kw):
        a = dict(dtype=BF16, q=P, k=P, v=P, lens=None, table=None, page=0, mb=0, np_=0, o=P,
                 lse=None, B=2, Hq=8, Hkv=1, d=128, L=64, scale=0.1, window=0, alibi=None,
                 splits=0)
        a.update(kw)
        return lib.gqa_decode_noalloc(a["dtype"], a["q"], a["k"], a["v"], a["lens"], a["table"],
                                      a["page"], a["mb"], a["np_"], a["o"], a["lse"], a["B"],
                                      a["Hq"], a["Hkv"], a["d"], a["L"], a["scale"], a["window"],
                                      a["alibi"], a["splits"], None)
    assert call(Hq=6, Hkv=4) == INV
    assert call(q=None) == INV
    assert call(k=P + 2) == INV
    assert call(scale=math.nan) == INV
    assert call(window=-1) == INV
    assert call(table=P, page=48, mb=2, np_=4, L=96) == INV       # page not a multiple of 32
    assert call(d=96) == UNS
    assert call(dtype=F32) == UNS
    # 4096 sequences x 8 K/V heads of 8192 keys need far more than the 32 MiB scratch
    assert call(B=4096, Hq=64, Hkv=8, L=8192) == WS
    assert gqa.decode_workspace_bytes(4096, 64, 8, 128, 8192) > gqa.DECODE_SCRATCH_BYTES
