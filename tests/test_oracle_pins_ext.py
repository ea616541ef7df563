"""Pins for the oracle's sliding-window, ALiBi and paged-cache options.

Readings (stated in the oracle's header): a window w > 0 keeps keys j > i - w;
ALiBi adds -slope_h * |i - j| to the scaled score before the softmax; the decode
query sits at position L_b - 1; a paged cache stores key j of sequence b as row
j % page_size of page block_table[b][j / page_size] of a pool
[num_pages, H_kv, page_size, d].

Independent anchors:
  * torch's float64 scaled_dot_product_attention with an explicit boolean mask
    (window) or an additive float mask (ALiBi), K/V heads expanded explicitly;
  * closed forms: window 1 (and a huge ALiBi slope) leaves only the diagonal key,
    so O_i = V_i; past a key length L a huge slope leaves only key L - 1, whose biased
    score is then the LSE; zero slopes and windows >= S change nothing;
  * gathering: a paged pool with the identity table, and with pages scattered
    by a random permutation, both equal the contiguous cache;
  * the sampled entry points (prefill_rows, decode_pairs) that the full-size GPU
    tests use equal the whole computation at the same rows and pairs.
A wrong window bound (off by one), a bias sign or scale error, a wrong bias
position for decode, or a wrong page/row split fails at least one test.
"""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F


def _rand(shape, seed, dtype=torch.float64):
    g = torch.Generator().manual_seed(seed)
    return torch.randn(shape, generator=g, dtype=torch.float64).to(dtype)


def _sdpa(q, k, v, scale, causal, seqlens, window=0, slopes=None):
    """fp64 SDPA on [B,S,H,d]; boolean validity and the ALiBi bias as one float mask."""
    B, S, Hq, d = q.shape
    g = Hq // k.shape[2]
    qt = q.double().permute(0, 2, 1, 3)
    kt = k.double().repeat_interleave(g, dim=2).permute(0, 2, 1, 3)
    vt = v.double().repeat_interleave(g, dim=2).permute(0, 2, 1, 3)
    i = torch.arange(S).view(S, 1)
    j = torch.arange(S).view(1, S)
    valid = torch.ones(B, 1, S, S, dtype=torch.bool)
    if seqlens is not None:
        valid &= (j < torch.as_tensor(seqlens).view(B, 1, 1, 1))
    if causal:
        valid &= (j <= i)
    if window:
        valid &= (j > i - window)
    bias = torch.zeros(B, Hq, S, S, dtype=torch.float64)
    if slopes is not None:
        bias = bias - torch.as_tensor(slopes, dtype=torch.float64).view(1, Hq, 1, 1) * \
            (i - j).abs().double()
    mask = torch.where(valid, bias, torch.tensor(-math.inf, dtype=torch.float64))
    out = F.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask, scale=scale)
    return out.permute(0, 2, 1, 3).numpy()


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("window", [1, 2, 5, 9])
def test_window_matches_sdpa(oracle_mod, causal, window):
    B, S, Hq, Hkv, d = 2, 13, 4, 2, 8
    q, k, v = _rand((B, S, Hq, d), 11), _rand((B, S, Hkv, d), 12), _rand((B, S, Hkv, d), 13)
    lens = np.array([13, 7], np.int32)
    o, _ = oracle_mod.prefill(q, k, v, scale=0.3, causal=causal, seqlens=lens, window=window)
    ref = _sdpa(q, k, v, 0.3, causal, lens, window=window)
    ok = ~np.isnan(ref)  # SDPA gives NaN for rows with no valid key; the oracle gives 0
    np.testing.assert_allclose(o[ok], ref[ok], rtol=0, atol=1e-12)
    assert np.all(o[~ok] == 0.0)


def test_window_one_keeps_only_the_diagonal(oracle_mod):
    B, S, Hq, Hkv, d = 1, 9, 3, 1, 4
    q, k, v = _rand((B, S, Hq, d), 21), _rand((B, S, Hkv, d), 22), _rand((B, S, Hkv, d), 23)
    o, lse = oracle_mod.prefill(q, k, v, scale=0.5, causal=True, window=1)
    for i in range(S):
        for h in range(Hq):
            np.testing.assert_allclose(o[0, i, h], v[0, i, 0].numpy(), rtol=0, atol=1e-15)
            s = 0.5 * float(q[0, i, h] @ k[0, i, 0])
            assert abs(lse[0, h, i] - s) < 1e-12  # a single term: lse = its score


def test_window_wider_than_sequence_changes_nothing(oracle_mod):
    B, S, Hq, Hkv, d = 2, 10, 4, 1, 8
    q, k, v = _rand((B, S, Hq, d), 31), _rand((B, S, Hkv, d), 32), _rand((B, S, Hkv, d), 33)
    a, la = oracle_mod.prefill(q, k, v, scale=0.2, causal=True)
    b, lb = oracle_mod.prefill(q, k, v, scale=0.2, causal=True, window=S)
    np.testing.assert_array_equal(a, b)
    np.testing.assert_array_equal(la, lb)


@pytest.mark.parametrize("causal", [False, True])
def test_alibi_matches_sdpa(oracle_mod, causal):
    B, S, Hq, Hkv, d = 2, 11, 4, 2, 8
    q, k, v = _rand((B, S, Hq, d), 41), _rand((B, S, Hkv, d), 42), _rand((B, S, Hkv, d), 43)
    slopes = np.array([0.5, 0.25, 0.125, 1.5])
    lens = np.array([11, 6], np.int32)
    o, _ = oracle_mod.prefill(q, k, v, scale=0.35, causal=causal, seqlens=lens,
                              alibi_slopes=slopes)
    ref = _sdpa(q, k, v, 0.35, causal, lens, slopes=slopes)
    np.testing.assert_allclose(o, ref, rtol=0, atol=1e-12)


def test_alibi_zero_slopes_change_nothing(oracle_mod):
    B, S, Hq, Hkv, d = 1, 12, 4, 2, 8
    q, k, v = _rand((B, S, Hq, d), 51), _rand((B, S, Hkv, d), 52), _rand((B, S, Hkv, d), 53)
    a, la = oracle_mod.prefill(q, k, v, scale=0.3, causal=False)
    b, lb = oracle_mod.prefill(q, k, v, scale=0.3, causal=False, alibi_slopes=np.zeros(Hq))
    np.testing.assert_array_equal(a, b)
    np.testing.assert_array_equal(la, lb)


@pytest.mark.parametrize("causal", [False, True])
def test_alibi_huge_slope_keeps_the_diagonal(oracle_mod, causal):
    B, S, Hq, Hkv, d = 1, 8, 2, 1, 4
    q, k, v = _rand((B, S, Hq, d), 61), _rand((B, S, Hkv, d), 62), _rand((B, S, Hkv, d), 63)
    o, _ = oracle_mod.prefill(q, k, v, scale=0.1, causal=causal, alibi_slopes=[2000.0, 2000.0])
    for i in range(S):
        for h in range(Hq):
            np.testing.assert_allclose(o[0, i, h], v[0, i, 0].numpy(), rtol=0, atol=1e-12)


def test_alibi_huge_slope_lse_past_the_keys(oracle_mod):
    """Rows at or past a short key length L with a huge slope: only the visible key nearest the
    query survives, j* = min(i, L - 1), so O = v_j* and LSE = scale <q_i, k_j*> - slope |i - j*|
    (the bias of every other key is smaller by at least the slope, e^-2000 of the total)."""
    B, S, Hq, Hkv, d, L, slope, scale = 1, 10, 2, 1, 4, 4, 2000.0, 0.3
    q, k, v = _rand((B, S, Hq, d), 71), _rand((B, S, Hkv, d), 72), _rand((B, S, Hkv, d), 73)
    for causal in (False, True):
        o, lse = oracle_mod.prefill(q, k, v, scale=scale, causal=causal, seqlens=[L],
                                    alibi_slopes=[slope, slope])
        for i in range(S):
            js = min(i, L - 1)
            for h in range(Hq):
                s = scale * float(q[0, i, h] @ k[0, js, 0]) - slope * abs(i - js)
                assert abs(lse[0, h, i] - s) < 1e-9 * max(1.0, abs(s))
                np.testing.assert_allclose(o[0, i, h], v[0, js, 0].numpy(), rtol=0, atol=1e-12)


def _decode_sdpa(q, kc, vc, lens, scale, window=0, slopes=None):
    """fp64 SDPA per (b, h): one query over the sequence's valid keys."""
    B, Hq, d = q.shape
    g = Hq // kc.shape[1]
    out = np.zeros((B, Hq, d))
    for b in range(B):
        L = int(lens[b])
        lo = max(0, L - window) if window else 0
        for h in range(Hq):
            kk = kc[b, h // g, lo:L].double()
            vv = vc[b, h // g, lo:L].double()
            bias = torch.zeros(1, L - lo, dtype=torch.float64)
            if slopes is not None:
                bias -= slopes[h] * (L - 1 - torch.arange(lo, L)).double()
            r = F.scaled_dot_product_attention(q[b, h].double().view(1, 1, d), kk.view(1, -1, d),
                                               vv.view(1, -1, d), attn_mask=bias.view(1, 1, -1),
                                               scale=scale)
            out[b, h] = r.view(d).numpy()
    return out


@pytest.mark.parametrize("window", [0, 1, 3, 40])
@pytest.mark.parametrize("with_alibi", [False, True])
def test_decode_window_and_alibi_match_sdpa(oracle_mod, window, with_alibi):
    B, Hq, Hkv, d, max_len = 3, 4, 2, 8, 30
    q, kc, vc = _rand((B, Hq, d), 71), _rand((B, Hkv, max_len, d), 72), _rand((B, Hkv, max_len, d), 73)
    lens = np.array([30, 17, 2], np.int32)
    slopes = np.array([0.3, 0.1, 0.7, 0.05]) if with_alibi else None
    o, _ = oracle_mod.decode(q, kc, vc, scale=0.4, lens=lens, window=window, alibi_slopes=slopes)
    ref = _decode_sdpa(q, kc, vc, lens, 0.4, window, slopes)
    np.testing.assert_allclose(o, ref, rtol=0, atol=1e-12)


def test_decode_alibi_equals_last_causal_row(oracle_mod):
    B, S, Hq, Hkv, d = 2, 9, 4, 2, 8
    q, k, v = _rand((B, S, Hq, d), 81), _rand((B, S, Hkv, d), 82), _rand((B, S, Hkv, d), 83)
    slopes = np.array([0.2, 0.4, 0.8, 1.6])
    po, pl = oracle_mod.prefill(q, k, v, scale=0.3, causal=True, alibi_slopes=slopes, window=4)
    kc = k.permute(0, 2, 1, 3).contiguous()
    vc = v.permute(0, 2, 1, 3).contiguous()
    do, dl = oracle_mod.decode(q[:, S - 1].contiguous(), kc, vc, scale=0.3, alibi_slopes=slopes,
                               window=4)
    np.testing.assert_allclose(do, po[:, S - 1], rtol=0, atol=1e-13)
    np.testing.assert_allclose(dl, pl[:, :, S - 1], rtol=0, atol=1e-13)


def _paged(kc, vc, page_size, perm_seed=None, extra_pages=3):
    """Scatter a contiguous cache [B, Hkv, max_len, d] into a page pool and a table."""
    B, Hkv, max_len, d = kc.shape
    mb = max_len // page_size
    n = B * mb + extra_pages
    order = np.arange(n) if perm_seed is None else np.random.default_rng(perm_seed).permutation(n)
    table = order[: B * mb].reshape(B, mb).astype(np.int32)
    kp = torch.full((n, Hkv, page_size, d), float("nan"), dtype=kc.dtype)
    vp = torch.full((n, Hkv, page_size, d), float("nan"), dtype=vc.dtype)
    for b in range(B):
        for i in range(mb):
            kp[table[b, i]] = kc[b, :, i * page_size:(i + 1) * page_size]
            vp[table[b, i]] = vc[b, :, i * page_size:(i + 1) * page_size]
    return kp, vp, table


@pytest.mark.parametrize("perm_seed", [None, 5, 6])
@pytest.mark.parametrize("dtype", [torch.float64, torch.bfloat16])
def test_paged_cache_equals_contiguous(oracle_mod, perm_seed, dtype):
    B, Hq, Hkv, d, P, mb = 3, 4, 2, 8, 4, 6
    q = _rand((B, Hq, d), 91, dtype)
    kc = _rand((B, Hkv, P * mb, d), 92, dtype)
    vc = _rand((B, Hkv, P * mb, d), 93, dtype)
    lens = np.array([24, 9, 1], np.int32)
    kp, vp, table = _paged(kc, vc, P, perm_seed)
    a, la = oracle_mod.decode(q, kc, vc, scale=0.3, lens=lens, alibi_slopes=[0.1, 0.2, 0.3, 0.4])
    b, lb = oracle_mod.decode(q, kp, vp, scale=0.3, lens=lens, block_table=table, page_size=P,
                              alibi_slopes=[0.1, 0.2, 0.3, 0.4])
    np.testing.assert_allclose(b, a, rtol=0, atol=1e-14)
    np.testing.assert_allclose(lb, la, rtol=0, atol=1e-14)
    assert np.isfinite(b).all()  # the NaN filler pages are never read


def test_paged_cache_rejects_a_bad_page(oracle_mod):
    B, Hq, Hkv, d, P, mb = 1, 2, 1, 4, 4, 2
    q = _rand((B, Hq, d), 1)
    kc = _rand((B, Hkv, P * mb, d), 2)
    kp, vp, table = _paged(kc, kc, P)
    table[0, 1] = kp.shape[0]  # one past the pool
    with pytest.raises(ValueError):
        oracle_mod.decode(q, kp, vp, scale=1.0, lens=[8], block_table=table, page_size=P)
    # a bad entry past the sequence's length is never looked at
    oracle_mod.decode(q, kp, vp, scale=1.0, lens=[4], block_table=table, page_size=P)


@pytest.mark.parametrize("causal,window,with_alibi", [(False, 0, False), (True, 0, False),
                                                      (True, 5, True), (False, 0, True)])
def test_sampled_rows_equal_the_whole_prefill(oracle_mod, causal, window, with_alibi):
    """prefill_rows (the full-size GPU tests' reference) gives, row for row, what the whole
    prefill gives: same indexing of (b, h, i), same masks and bias."""
    B, S, Hq, Hkv, d = 2, 13, 6, 2, 8
    q, k, v = _rand((B, S, Hq, d), 81), _rand((B, S, Hkv, d), 82), _rand((B, S, Hkv, d), 83)
    lens = [13, 7]
    slopes = [0.3, 0.1, 0.05, 0.7, 0.0, 1.2] if with_alibi else None
    o, lse = oracle_mod.prefill(q, k, v, scale=0.4, causal=causal, seqlens=lens, window=window,
                                alibi_slopes=slopes)
    rng = np.random.default_rng(5)
    rows = np.stack([rng.integers(B, size=40), rng.integers(Hq, size=40),
                     rng.integers(S, size=40)], 1)
    ro, rl = oracle_mod.prefill_rows(q, k, v, rows, scale=0.4, causal=causal, seqlens=lens,
                                     window=window, alibi_slopes=slopes)
    for r, (b, h, i) in enumerate(rows):
        np.testing.assert_allclose(ro[r], o[b, i, h], rtol=0, atol=1e-13)
        if np.isfinite(lse[b, h, i]):
            assert abs(rl[r] - lse[b, h, i]) < 1e-13
        else:
            assert rl[r] == lse[b, h, i]


@pytest.mark.parametrize("window,with_alibi", [(0, False), (4, True)])
def test_sampled_pairs_equal_the_whole_decode(oracle_mod, window, with_alibi):
    """decode_pairs gives, pair for pair, what the whole decode gives."""
    B, Hq, Hkv, d, max_len = 3, 6, 3, 8, 20
    q = _rand((B, Hq, d), 91)
    kc, vc = _rand((B, Hkv, max_len, d), 92), _rand((B, Hkv, max_len, d), 93)
    lens = [20, 1, 9]
    slopes = [0.2, 0.0, 0.6, 0.1, 1.0, 0.03] if with_alibi else None
    o, lse = oracle_mod.decode(q, kc, vc, scale=0.3, lens=lens, window=window,
                               alibi_slopes=slopes)
    pairs = [(b, h) for b in range(B) for h in range(Hq)]
    po, pl = oracle_mod.decode_pairs(q, kc, vc, pairs, scale=0.3, lens=lens, window=window,
                                     alibi_slopes=slopes)
    for r, (b, h) in enumerate(pairs):
        np.testing.assert_allclose(po[r], o[b, h], rtol=0, atol=1e-13)
        assert abs(pl[r] - lse[b, h]) < 1e-13
