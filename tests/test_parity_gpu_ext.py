"""GPU parity of the optional score modifiers and the paged cache, through the C ABI
(gqa_prefill_ex / gqa_decode_ex), against the fp64 oracle.

Tolerances are those of test_parity_gpu.py: outputs 1e-5 (fp32) and 2e-2 (bf16);
LSE 1e-4 (fp32) and 1e-3 (bf16: with an LSE output the weights are summed in fp32), in
prefill each beyond 2 fp32 ulps of the LSE's own value (its storage precision). The one
exception is the steep-ALiBi stress test, whose q and k are 3x the unit-variance inputs the
fp32 tolerance is stated for: its logits, and the fp32 rounding error they carry, are 9x
larger, and so is its fp32 output tolerance.
"""
import math
import sys

import numpy as np
import pytest
import torch

import grouped_query_attention_02_amd as gqa
import workloads as W

pytestmark = pytest.mark.gpu

TOL = {torch.float32: 1e-5, torch.bfloat16: 2e-2}
LSE_TOL = {torch.float32: 1e-4, torch.bfloat16: 1e-3}
DEC_LSE_TOL = 1e-3


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu(built_lib):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    gqa.load()


def _rand(shape, seed, dtype, scale=1.0):
    g = torch.Generator().manual_seed(seed)
    return (torch.randn(shape, generator=g) * scale).to(dtype)


def _errs(o, lse, ref_o, ref_l):
    a = o.detach().double().cpu().numpy()
    assert not np.isnan(a).any(), "NaN in GPU output"
    e = float(np.abs(a - ref_o).max())
    b = lse.detach().double().cpu().numpy()
    fin = np.isfinite(ref_l)
    assert np.array_equal(np.isfinite(b), fin), "LSE finiteness differs"
    # LSE error beyond 2 fp32 ulps of the value: an LSE of a few thousand (a strong ALiBi
    # bias on a row far past its last key) is stored no closer than ~1e-4 whatever the kernel.
    le = float((np.abs(b[fin] - ref_l[fin]) - 2.0 ** -22 * np.abs(ref_l[fin])).max()) \
        if fin.any() else 0.0
    return e, le


def alibi_slopes(H):
    """The usual geometric ALiBi slopes 2^(-8 k / H), k = 1..H."""
    return [2.0 ** (-8.0 * (k + 1) / H) for k in range(H)]


PREFILL_CASES = []
for dtype in (torch.bfloat16, torch.float32):
    for d in (32, 64, 128):
        for (window, alibi, causal) in ((1, False, True), (17, False, True), (64, False, True),
                                        (100, True, True), (0, True, True), (0, True, False)):
            PREFILL_CASES.append((dtype, d, window, alibi, causal))


@pytest.mark.parametrize("dtype,d,window,alibi,causal", PREFILL_CASES)
def test_prefill_window_alibi(oracle_mod, dtype, d, window, alibi, causal):
    B, S, Hq, Hkv = 3, 150, 8, 2
    seed = 2000 + d + window + 7 * int(alibi) + int(causal)
    _say(f"case prefill_ex {dtype} d={d} window={window} alibi={alibi} causal={causal}")
    q, k, v = _rand((B, S, Hq, d), seed, dtype), _rand((B, S, Hkv, d), seed + 1, dtype), \
        _rand((B, S, Hkv, d), seed + 2, dtype)
    slopes = alibi_slopes(Hq) if alibi else None
    scale = 1 / math.sqrt(d)
    for lens in (None, [150, 3, 77]):
        ld = None if lens is None else torch.tensor(lens, dtype=torch.int32, device="cuda")
        o_plain = gqa.prefill(q.cuda(), k.cuda(), v.cuda(), causal=causal, softmax_scale=scale,
                              seqlens=ld, window=window, alibi_slopes=slopes)
        o, lse = gqa.prefill(q.cuda(), k.cuda(), v.cuda(), causal=causal, softmax_scale=scale,
                             seqlens=ld, window=window, alibi_slopes=slopes, return_lse=True)
        torch.cuda.synchronize()
        ro, rl = oracle_mod.prefill(q, k, v, scale=scale, causal=causal, seqlens=lens,
                                    window=window, alibi_slopes=slopes)
        e_plain, _ = _errs(o_plain, lse, ro, rl)
        e, le = _errs(o, lse, ro, rl)
        _say(f"  lens={lens} max_abs_err={e_plain:.3e} (with LSE {e:.3e}) lse_err={le:.3e}")
        assert e_plain <= TOL[dtype] and e <= TOL[dtype] and le <= LSE_TOL[dtype]


NEG_CASES = [(dtype, d, w, a, c) for dtype in (torch.bfloat16, torch.float32)
             for d in (32, 64, 128)
             for (w, a, c) in ((0, False, False), (0, False, True), (40, True, True),
                               (0, True, False))]


@pytest.mark.parametrize("dtype,d,window,alibi,causal", NEG_CASES)
def test_prefill_negative_scale(oracle_mod, dtype, d, window, alibi, causal):
    """A negative softmax scale (the weights favour small dot products) with every option:
    masked keys must still get weight 0 whatever the sign."""
    B, S, Hq, Hkv = 2, 100, 4, 2
    seed = 2600 + d + window + 7 * int(alibi) + int(causal)
    _say(f"case prefill_ex negative scale {dtype} d={d} window={window} alibi={alibi} "
         f"causal={causal}")
    q, k, v = _rand((B, S, Hq, d), seed, dtype), _rand((B, S, Hkv, d), seed + 1, dtype), \
        _rand((B, S, Hkv, d), seed + 2, dtype)
    slopes = alibi_slopes(Hq) if alibi else None
    scale = -0.7 / math.sqrt(d)
    lens = [100, 37]
    ld = torch.tensor(lens, dtype=torch.int32, device="cuda")
    o, lse = gqa.prefill(q.cuda(), k.cuda(), v.cuda(), causal=causal, softmax_scale=scale,
                         seqlens=ld, window=window, alibi_slopes=slopes, return_lse=True)
    torch.cuda.synchronize()
    ro, rl = oracle_mod.prefill(q, k, v, scale=scale, causal=causal, seqlens=lens,
                                window=window, alibi_slopes=slopes)
    e, le = _errs(o, lse, ro, rl)
    _say(f"  max_abs_err={e:.3e} lse_err={le:.3e}")
    assert e <= TOL[dtype] and le <= LSE_TOL[dtype]


STEEP_CASES = [(dtype, d, Hkv, causal) for dtype in (torch.bfloat16, torch.float32)
               for d in (64, 128) for Hkv in (4, 1) for causal in (True, False)]


@pytest.mark.parametrize("dtype,d,Hkv,causal", STEEP_CASES)
def test_prefill_alibi_steep_long(oracle_mod, dtype, d, Hkv, causal):
    """ALiBi with slopes from 8 down to 2^-8 over long rows and widely spread scores, for MHA
    (one query head per K/V head) and MQA: the bias changes the row max by many exp2 units
    from one key tile to the next, which moves the kernel's exponent offset."""
    B, S, Hq = 2, 700, 4
    seed = 2800 + d + Hkv + int(causal)
    _say(f"case prefill_ex steep alibi {dtype} d={d} Hkv={Hkv} causal={causal}")
    q, k, v = _rand((B, S, Hq, d), seed, dtype, 3.0), _rand((B, S, Hkv, d), seed + 1, dtype, 3.0), \
        _rand((B, S, Hkv, d), seed + 2, dtype)
    slopes = [8.0, 1.0, 2.0 ** -3, 2.0 ** -8]
    scale = 1 / math.sqrt(d)
    lens = [700, 333]
    ld = torch.tensor(lens, dtype=torch.int32, device="cuda")
    o, lse = gqa.prefill(q.cuda(), k.cuda(), v.cuda(), causal=causal, softmax_scale=scale,
                         seqlens=ld, alibi_slopes=slopes, return_lse=True)
    torch.cuda.synchronize()
    ro, rl = oracle_mod.prefill(q, k, v, scale=scale, causal=causal, seqlens=lens,
                                alibi_slopes=slopes)
    e, le = _errs(o, lse, ro, rl)
    _say(f"  max_abs_err={e:.3e} lse_err={le:.3e}")
    # q and k are 3x the unit-variance inputs the fp32 tolerance is set for: the rounding
    # error of each dot product, and so of each weight, grows with |q| |k| (x9).
    tol = TOL[dtype] * (9.0 if dtype == torch.float32 else 1.0)
    assert e <= tol and le <= LSE_TOL[dtype]


@pytest.mark.parametrize("dtype,d", [(torch.bfloat16, 64), (torch.bfloat16, 128),
                                     (torch.float32, 64)])
def test_prefill_negative_alibi_slopes(oracle_mod, dtype, d):
    """Negative slopes (the bias grows with distance, up to +110 nats here, more than fp32's
    exponent range in exp2 units): far keys can outweigh near ones, so every change of the
    kernels' exponent offset goes the other way."""
    B, S, Hq, Hkv = 2, 1100, 4, 2
    _say(f"case prefill_ex negative alibi slopes {dtype} d={d}")
    q, k, v = _rand((B, S, Hq, d), 2980 + d, dtype), _rand((B, S, Hkv, d), 2981 + d, dtype), \
        _rand((B, S, Hkv, d), 2982 + d, dtype)
    slopes = [-0.1, -0.01, 0.05, -2.0 ** -8]
    lens = [1100, 333]
    ld = torch.tensor(lens, dtype=torch.int32, device="cuda")
    for causal in (True, False):
        o, lse = gqa.prefill(q.cuda(), k.cuda(), v.cuda(), causal=causal,
                             softmax_scale=1 / math.sqrt(d), seqlens=ld, alibi_slopes=slopes,
                             return_lse=True)
        torch.cuda.synchronize()
        ro, rl = oracle_mod.prefill(q, k, v, scale=1 / math.sqrt(d), causal=causal,
                                    seqlens=lens, alibi_slopes=slopes)
        e, le = _errs(o, lse, ro, rl)
        _say(f"  causal={causal} max_abs_err={e:.3e} lse_err={le:.3e}")
        assert e <= TOL[dtype] and le <= LSE_TOL[dtype]


@pytest.mark.parametrize("dtype,d", [(torch.bfloat16, 64), (torch.bfloat16, 128),
                                     (torch.float32, 64)])
def test_prefill_zero_scale_with_alibi(oracle_mod, dtype, d):
    """softmax_scale = 0 with ALiBi: the weights depend on the bias alone, which the kernels
    carry in raw-score units (slope / exponent factor per key); O and the LSE must still
    equal the oracle's, with rows past a short key length included."""
    B, S, Hq, Hkv = 2, 200, 4, 2
    _say(f"case prefill_ex zero scale + alibi {dtype} d={d}")
    q, k, v = _rand((B, S, Hq, d), 2900 + d, dtype), _rand((B, S, Hkv, d), 2901 + d, dtype), \
        _rand((B, S, Hkv, d), 2902 + d, dtype)
    slopes = [0.5, 0.1, 2.0 ** -5, 2.0 ** -8]
    lens = [200, 70]
    ld = torch.tensor(lens, dtype=torch.int32, device="cuda")
    for causal in (True, False):
        o, lse = gqa.prefill(q.cuda(), k.cuda(), v.cuda(), causal=causal, softmax_scale=0.0,
                             seqlens=ld, alibi_slopes=slopes, return_lse=True)
        torch.cuda.synchronize()
        ro, rl = oracle_mod.prefill(q, k, v, scale=0.0, causal=causal, seqlens=lens,
                                    alibi_slopes=slopes)
        e, le = _errs(o, lse, ro, rl)
        _say(f"  causal={causal} max_abs_err={e:.3e} lse_err={le:.3e}")
        assert e <= TOL[dtype] and le <= LSE_TOL[dtype]


def test_decode_negative_alibi_slopes(oracle_mod):
    """Negative slopes in the split-KV decode: the oldest keys carry the largest bias."""
    B, Hq, Hkv, d, max_len = 3, 8, 2, 64, 900
    _say("case decode_ex negative alibi slopes")
    q = _rand((B, Hq, d), 2990, torch.bfloat16)
    kc = _rand((B, Hkv, max_len, d), 2991, torch.bfloat16)
    vc = _rand((B, Hkv, max_len, d), 2992, torch.bfloat16)
    lens = [900, 400, 17]
    slopes = [-0.05, -0.01, 0.02, -2.0 ** -8, 0.0, -0.002, 0.1, -0.03]
    ref_o, ref_l = oracle_mod.decode(q, kc, vc, scale=0.125, lens=lens, alibi_slopes=slopes)
    for splits in (0, 1, 4):
        o, lse = gqa.decode(q.cuda(), kc.cuda(), vc.cuda(),
                            torch.tensor(lens, dtype=torch.int32).cuda(), softmax_scale=0.125,
                            num_splits=splits, alibi_slopes=slopes, return_lse=True)
        torch.cuda.synchronize()
        e, le = _errs(o, lse, ref_o, ref_l)
        _say(f"  splits={splits} max_abs_err={e:.3e} lse_err={le:.3e}")
        assert e <= 2e-2 and le <= DEC_LSE_TOL


def test_decode_zero_scale_with_alibi(oracle_mod):
    """softmax_scale = 0 with ALiBi in the split-KV decode: a share that does not hold the
    query's own key has its row max far below the other shares', and the merge weights the
    shares by their LSEs, so a wrong LSE would show in O."""
    B, Hq, Hkv, d, max_len = 3, 16, 2, 128, 1500
    _say("case decode_ex zero scale + alibi")
    q = _rand((B, Hq, d), 2950, torch.bfloat16)
    kc = _rand((B, Hkv, max_len, d), 2951, torch.bfloat16)
    vc = _rand((B, Hkv, max_len, d), 2952, torch.bfloat16)
    lens = [1500, 700, 33]
    slopes = [2.0 ** (-k / 2) for k in range(Hq)]
    ref_o, ref_l = oracle_mod.decode(q, kc, vc, scale=0.0, lens=lens, alibi_slopes=slopes)
    for splits in (0, 1, 5):
        o, lse = gqa.decode(q.cuda(), kc.cuda(), vc.cuda(),
                            torch.tensor(lens, dtype=torch.int32).cuda(), softmax_scale=0.0,
                            num_splits=splits, alibi_slopes=slopes, return_lse=True)
        torch.cuda.synchronize()
        e, le = _errs(o, lse, ref_o, ref_l)
        _say(f"  splits={splits} max_abs_err={e:.3e} lse_err={le:.3e}")
        assert e <= 2e-2 and le <= DEC_LSE_TOL


def test_prefill_window_full_size_sampled(oracle_mod):
    """Causal Llama-shaped prefill (B=4, S=4096, 32/8 heads, d=128) with a 1000-key window and
    ALiBi, in the launch configuration the benchmark uses; 300 sampled rows."""
    w = W.WORKLOADS["llama_causal_prefill"]
    x = W.make_prefill(w)
    slopes = alibi_slopes(w.Hq)
    _say("case llama_causal_prefill window=1000 + alibi (full size)")
    o, lse = gqa.prefill(x["q"].cuda(), x["k"].cuda(), x["v"].cuda(), causal=True,
                         softmax_scale=w.softmax_scale, window=1000, alibi_slopes=slopes,
                         return_lse=True)
    torch.cuda.synchronize()
    rng = np.random.default_rng(9)
    rows = [(int(rng.integers(w.B)), int(rng.integers(w.Hq)), int(rng.integers(w.S)))
            for _ in range(296)] + [(0, 0, 0), (1, 5, 999), (2, 31, 1000), (3, 17, w.S - 1)]
    ro, rl = oracle_mod.prefill_rows(x["q"], x["k"], x["v"], rows, scale=w.softmax_scale,
                                     causal=True, window=1000, alibi_slopes=slopes)
    oc, lc = o.cpu(), lse.cpu()
    got = torch.stack([oc[b, i, h] for b, h, i in rows])
    got_l = torch.tensor([float(lc[b, h, i]) for b, h, i in rows], dtype=torch.float64)
    e, le = _errs(got, got_l, ro, rl)
    _say(f"  rows={len(rows)} max_abs_err={e:.3e} lse_err={le:.3e}")
    assert e <= 2e-2 and le <= LSE_TOL[torch.bfloat16]


def _paged(kc, vc, page_size, seed, extra=5, poison=True):
    """Scatter [B, Hkv, max_len, d] caches into NaN-filled page pools with a random table."""
    B, Hkv, max_len, d = kc.shape
    mb = max_len // page_size
    n = B * mb + extra
    order = np.random.default_rng(seed).permutation(n)
    table = torch.tensor(order[: B * mb].reshape(B, mb), dtype=torch.int32)
    fill = float("nan") if poison else 0.0
    kp = torch.full((n, Hkv, page_size, d), fill, dtype=kc.dtype)
    vp = torch.full((n, Hkv, page_size, d), fill, dtype=vc.dtype)
    for b in range(B):
        for i in range(mb):
            kp[table[b, i]] = kc[b, :, i * page_size:(i + 1) * page_size]
            vp[table[b, i]] = vc[b, :, i * page_size:(i + 1) * page_size]
    return kp, vp, table


DECODE_CASES = []
for d in (64, 128):
    for (Hq, Hkv) in ((32, 1), (16, 2), (8, 8), (64, 2)):
        for (window, alibi, page) in ((0, False, 32), (0, True, 0), (100, False, 0),
                                      (33, True, 64), (0, False, 256), (257, True, 128)):
            DECODE_CASES.append((d, Hq, Hkv, window, alibi, page))


@pytest.mark.parametrize("d,Hq,Hkv,window,alibi,page", DECODE_CASES)
def test_decode_window_alibi_paged(oracle_mod, d, Hq, Hkv, window, alibi, page):
    B, max_len = 5, 768
    seed = 3000 + d + Hq + Hkv + window + page + int(alibi)
    _say(f"case decode_ex d={d} Hq={Hq} Hkv={Hkv} window={window} alibi={alibi} page={page}")
    q = _rand((B, Hq, d), seed, torch.bfloat16)
    kc = _rand((B, Hkv, max_len, d), seed + 1, torch.bfloat16)
    vc = _rand((B, Hkv, max_len, d), seed + 2, torch.bfloat16)
    lens = [768, 1, 0, 300, 513]
    slopes = alibi_slopes(Hq) if alibi else None
    if page:
        kp, vp, table = _paged(kc, vc, page, seed)
        args = dict(block_table=table.cuda(), page_size=page)
        kd, vd = kp.cuda(), vp.cuda()
    else:
        args, kd, vd, table = {}, kc.cuda(), vc.cuda(), None
    ref_o, ref_l = oracle_mod.decode(q, kc, vc, scale=0.09, lens=lens, window=window,
                                     alibi_slopes=slopes)
    outs = []
    for splits in (0, 1, 3):
        o, lse = gqa.decode(q.cuda(), kd, vd, torch.tensor(lens, dtype=torch.int32).cuda(),
                            softmax_scale=0.09, num_splits=splits, window=window,
                            alibi_slopes=slopes, return_lse=True, **args)
        torch.cuda.synchronize()
        e, le = _errs(o, lse, ref_o, ref_l)
        _say(f"  splits={splits} max_abs_err={e:.3e} lse_err={le:.3e}")
        assert e <= 2e-2 and le <= DEC_LSE_TOL
        outs.append(o.float())
    for o in outs[1:]:
        assert (o - outs[0]).abs().max().item() <= 2e-2


def test_paged_decode_matches_contiguous_bitwise():
    """The paged kernel only changes where rows are read from: with the same split plan its
    output equals the contiguous kernel's bit for bit."""
    B, Hq, Hkv, d, max_len, page = 6, 32, 4, 128, 1024, 64
    q = _rand((B, Hq, d), 41, torch.bfloat16)
    kc = _rand((B, Hkv, max_len, d), 42, torch.bfloat16)
    vc = _rand((B, Hkv, max_len, d), 43, torch.bfloat16)
    lens = torch.tensor([1024, 5, 700, 64, 0, 999], dtype=torch.int32).cuda()
    kp, vp, table = _paged(kc, vc, page, 44)
    for window, slopes in ((0, None), (200, alibi_slopes(Hq))):
        a = gqa.decode(q.cuda(), kc.cuda(), vc.cuda(), lens, window=window, alibi_slopes=slopes)
        b = gqa.decode(q.cuda(), kp.cuda(), vp.cuda(), lens, window=window, alibi_slopes=slopes,
                       block_table=table.cuda(), page_size=page)
        torch.cuda.synchronize()
        assert torch.equal(a, b)


@pytest.mark.parametrize("use_alibi", [False, True])
def test_paged_decode_full_size_sampled(oracle_mod, use_alibi):
    """MQA ragged decode (B=32, 32/1 heads, d=128, caches up to 32768) from a paged cache with
    256-key pages scattered over the pool, in the benchmark's launch configuration."""
    w = W.WORKLOADS["mqa_ragged_decode"]
    x = W.make_decode(w)
    page = 256
    mb = w.max_len // page
    n_pages = w.B * mb + 7
    perm = np.random.default_rng(12).permutation(n_pages)
    table = torch.tensor(perm[: w.B * mb].reshape(w.B, mb), dtype=torch.int32)
    kc, vc = x["k_cache"], x["v_cache"]
    kp = torch.zeros((n_pages, w.Hkv, page, w.d), dtype=kc.dtype)
    vp = torch.zeros((n_pages, w.Hkv, page, w.d), dtype=vc.dtype)
    kp[table.view(-1).long()] = kc.view(w.B, w.Hkv, mb, page, w.d).permute(0, 2, 1, 3, 4) \
        .reshape(w.B * mb, w.Hkv, page, w.d)
    vp[table.view(-1).long()] = vc.view(w.B, w.Hkv, mb, page, w.d).permute(0, 2, 1, 3, 4) \
        .reshape(w.B * mb, w.Hkv, page, w.d)
    slopes = alibi_slopes(w.Hq) if use_alibi else None
    _say(f"case mqa_ragged_decode paged page={page} alibi={use_alibi} (full size)")
    o, lse = gqa.decode(x["q"].cuda(), kp.cuda(), vp.cuda(), x["lens"].cuda(),
                        softmax_scale=w.softmax_scale, alibi_slopes=slopes,
                        block_table=table.cuda(), page_size=page, return_lse=True)
    torch.cuda.synchronize()
    pairs = [(b, h) for b in range(w.B) for h in (0, 13, 31)]
    ro, rl = oracle_mod.decode_pairs(x["q"], kc, vc, pairs, scale=w.softmax_scale,
                                     lens=x["lens"], alibi_slopes=slopes)
    oc, lc = o.cpu(), lse.cpu()
    got = torch.stack([oc[b, h] for b, h in pairs])
    got_l = torch.tensor([float(lc[b, h]) for b, h in pairs], dtype=torch.float64)
    e, le = _errs(got, got_l, ro, rl)
    _say(f"  pairs={len(pairs)} max_abs_err={e:.3e} lse_err={le:.3e}")
    assert e <= 2e-2 and le <= DEC_LSE_TOL


def test_bad_page_ids_read_as_zeros():
    """A page id outside the pool must not fault: its rows read as zeros (equal to a cache
    whose rows there are zero)."""
    B, Hq, Hkv, d, page, mb = 2, 8, 1, 64, 32, 4
    q = _rand((B, Hq, d), 51, torch.bfloat16)
    kc = _rand((B, Hkv, page * mb, d), 52, torch.bfloat16)
    vc = _rand((B, Hkv, page * mb, d), 53, torch.bfloat16)
    kp, vp, table = _paged(kc, vc, page, 54, poison=False)
    bad = table.clone()
    bad[1, 2] = 10_000       # far outside the pool
    bad[0, 1] = -3
    lens = torch.tensor([128, 128], dtype=torch.int32).cuda()
    o = gqa.decode(q.cuda(), kp.cuda(), vp.cuda(), lens, block_table=bad.cuda(), page_size=page)
    kz, vz = kc.clone(), vc.clone()
    kz[1, :, 2 * page:3 * page] = 0
    vz[1, :, 2 * page:3 * page] = 0
    kz[0, :, page:2 * page] = 0
    vz[0, :, page:2 * page] = 0
    ref = gqa.decode(q.cuda(), kz.cuda(), vz.cuda(), lens)
    torch.cuda.synchronize()
    assert torch.isfinite(o.float()).all()
    assert (o.float() - ref.float()).abs().max().item() <= 2e-2


def _random_prefill_case(rng):
    d = int(rng.choice([32, 64, 128]))
    g = int(rng.choice([1, 2, 4, 8, 32]))
    Hkv = int(rng.integers(1, 4)) if g < 32 else 1
    S = int(rng.integers(1, 260 if g < 32 else 140))
    B = int(rng.integers(1, 6))
    causal = bool(rng.integers(2))
    lens = [int(x) for x in rng.integers(0, S + 3, size=B)] if rng.integers(3) else None
    window = int(rng.integers(1, S + 2)) if causal and rng.integers(2) else 0
    slopes = list(rng.uniform(0.0, 0.5, size=g * Hkv)) if rng.integers(2) else None
    dtype = torch.float32 if rng.integers(4) == 0 else torch.bfloat16
    scale = float(rng.choice([1 / math.sqrt(d), 0.3, -0.2]))
    return dict(d=d, Hq=g * Hkv, Hkv=Hkv, S=S, B=B, causal=causal, lens=lens, window=window,
                slopes=slopes, dtype=dtype, scale=scale)


@pytest.mark.parametrize("case_seed", range(80))
def test_prefill_random_shapes(oracle_mod, case_seed):
    """Seeded random configurations across head size, group size (1-32), length (from 1),
    batch, key lengths (with zeros and clamped values), causal, window, ALiBi, dtype and scale."""
    c = _random_prefill_case(np.random.default_rng(7000 + case_seed))
    _say(f"case prefill random #{case_seed}: {c}")
    B, S, Hq, Hkv, d = c["B"], c["S"], c["Hq"], c["Hkv"], c["d"]
    q = _rand((B, S, Hq, d), 7100 + case_seed, c["dtype"])
    k = _rand((B, S, Hkv, d), 7200 + case_seed, c["dtype"])
    v = _rand((B, S, Hkv, d), 7300 + case_seed, c["dtype"])
    ld = None if c["lens"] is None else torch.tensor(c["lens"], dtype=torch.int32, device="cuda")
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    # Without an LSE output the kernels are the plain instantiations (those the benchmark
    # times); with one they also sum the fp32 weights.
    o_plain = gqa.prefill(qd, kd, vd, causal=c["causal"], softmax_scale=c["scale"], seqlens=ld,
                          window=c["window"], alibi_slopes=c["slopes"])
    o, lse = gqa.prefill(qd, kd, vd, causal=c["causal"], softmax_scale=c["scale"], seqlens=ld,
                         window=c["window"], alibi_slopes=c["slopes"], return_lse=True)
    torch.cuda.synchronize()
    ro, rl = oracle_mod.prefill(q, k, v, scale=c["scale"], causal=c["causal"], seqlens=c["lens"],
                                window=c["window"], alibi_slopes=c["slopes"])
    e_plain, _ = _errs(o_plain, lse, ro, rl)
    e, le = _errs(o, lse, ro, rl)
    _say(f"  max_abs_err={e_plain:.3e} (with LSE {e:.3e}) lse_err={le:.3e}")
    assert e_plain <= TOL[c["dtype"]] and e <= TOL[c["dtype"]] and le <= LSE_TOL[c["dtype"]]


@pytest.mark.parametrize("case_seed", range(50))
def test_decode_random_shapes(oracle_mod, case_seed):
    """Seeded random decode configurations: head size, group size (1-64), cache length,
    batch, lengths (with zeros), window, ALiBi, paged or contiguous, split count and scale."""
    rng = np.random.default_rng(8000 + case_seed)
    d = int(rng.choice([64, 128]))
    g = int(rng.choice([1, 2, 4, 8, 32, 40, 64]))
    Hkv = int(rng.integers(1, 4))
    page = int(rng.choice([0, 32, 64, 256]))
    max_len = int(rng.integers(1, 900))
    if page:
        max_len = -(-max_len // page) * page
    B = int(rng.integers(1, 7))
    lens = [int(x) for x in rng.integers(0, max_len + 1, size=B)]
    window = int(rng.integers(1, max_len + 2)) if rng.integers(2) else 0
    slopes = list(rng.uniform(0.0, 0.5, size=g * Hkv)) if rng.integers(2) else None
    splits = int(rng.choice([0, 1, 2, 7]))
    scale = float(rng.choice([1 / math.sqrt(d), 0.25, -0.1]))
    Hq = g * Hkv
    _say(f"case decode random #{case_seed}: d={d} Hq={Hq} Hkv={Hkv} max_len={max_len} B={B} "
         f"lens={lens} window={window} alibi={slopes is not None} page={page} splits={splits} "
         f"scale={scale:.3f}")
    q = _rand((B, Hq, d), 8100 + case_seed, torch.bfloat16)
    kc = _rand((B, Hkv, max_len, d), 8200 + case_seed, torch.bfloat16)
    vc = _rand((B, Hkv, max_len, d), 8300 + case_seed, torch.bfloat16)
    if page:
        kp, vp, table = _paged(kc, vc, page, 8400 + case_seed)
        kd, vd, args = kp.cuda(), vp.cuda(), dict(block_table=table.cuda(), page_size=page)
    else:
        kd, vd, args = kc.cuda(), vc.cuda(), {}
    o, lse = gqa.decode(q.cuda(), kd, vd, torch.tensor(lens, dtype=torch.int32).cuda(),
                        softmax_scale=scale, num_splits=splits, window=window,
                        alibi_slopes=slopes, return_lse=True, **args)
    torch.cuda.synchronize()
    ro, rl = oracle_mod.decode(q, kc, vc, scale=scale, lens=lens, window=window,
                               alibi_slopes=slopes)
    e, le = _errs(o, lse, ro, rl)
    _say(f"  max_abs_err={e:.3e} lse_err={le:.3e}")
    assert e <= 2e-2 and le <= DEC_LSE_TOL
