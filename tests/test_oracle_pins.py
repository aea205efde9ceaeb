"""Pins for the fp64 oracle: each test checks it against something other than itself.

* brute force at 50 digits with mpmath, with the mask built from key ranges and
  the softmax taken without the max shift;
* torch's float64 scaled_dot_product_attention on the CPU (a library routine);
* closed forms: zero queries give plain means of V over the visible keys;
  constant V gives a constant output; V = identity returns the softmax rows;
* the printed GQA example of the CTE page;
* the CTE page's affine-select construction of the causal and window masks;
* needles: a key aligned with one query dominates that row exactly;
* the online-softmax recurrence of the pages (one tile and many tiles) and the
  log-sum-exp merge of key-split partials, written here as separate models.
"""
import json
import math
import os

import mpmath
import numpy as np
import pytest
import torch

import oracle
from flash_attention_forward_amd import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


# ----------------------------------------------------------------------------- brute force
def brute_row(q, k, v, b, i, h, scale, causal, window):
    """mpmath, 50 digits. Visible keys from explicit ranges; softmax without max shift."""
    mpmath.mp.dps = 50
    B, Sq, Hq, D = q.shape
    Skv, Hkv = k.shape[1], k.shape[2]
    hk = h // (Hq // Hkv)
    qpos = i + Skv - Sq
    hi = min(Skv, qpos + 1) if causal else Skv
    lo = max(0, qpos - window + 1) if window > 0 else 0
    keys = list(range(lo, hi))
    if not keys:
        return [mpmath.mpf(0)] * D, -mpmath.inf
    e = []
    for j in keys:
        s = mpmath.mpf(scale) * mpmath.fsum(mpmath.mpf(q[b, i, h, d]) * mpmath.mpf(k[b, j, hk, d]) for d in range(D))
        e.append(mpmath.exp(s))
    Z = mpmath.fsum(e)
    o = [mpmath.fsum(e[t] * mpmath.mpf(v[b, j, hk, d]) for t, j in enumerate(keys)) / Z for d in range(D)]
    return o, mpmath.log(Z)


CASES = [
    # B, Hq, Hkv, Sq, Skv, D, causal, window
    (1, 1, 1, 5, 5, 3, False, 0),
    (2, 4, 2, 7, 7, 4, True, 0),
    (1, 3, 1, 6, 11, 5, True, 0),  # Sq < Skv: bottom-right alignment
    (1, 2, 2, 9, 9, 8, True, 3),
    (2, 6, 2, 8, 13, 4, True, 4),
    (1, 2, 1, 12, 12, 2, True, 1),  # window 1: each row sees only itself
    (1, 1, 1, 4, 24, 6, False, 0),
]


@pytest.mark.parametrize("case", CASES)
def test_bruteforce_mpmath(case):
    B, Hq, Hkv, Sq, Skv, D, causal, window = case
    seed = 11 + sum(case[:6])
    q, k, v = rand((B, Sq, Hq, D), seed), rand((B, Skv, Hkv, D), seed + 1), rand((B, Skv, Hkv, D), seed + 2)
    scale = 0.7
    o, lse = oracle.attention(q, k, v, scale, causal, window, return_lse=True)
    for b in range(B):
        for i in range(Sq):
            for h in range(Hq):
                ref, ref_lse = brute_row(q, k, v, b, i, h, scale, causal, window)
                ref = np.array([float(x) for x in ref])
                assert np.allclose(o[b, i, h], ref, rtol=1e-13, atol=1e-13)
                if ref_lse == -mpmath.inf:
                    assert lse[b, i, h] == -np.inf
                else:
                    assert abs(lse[b, i, h] - float(ref_lse)) <= 1e-13 * max(1.0, abs(float(ref_lse)))


# ----------------------------------------------------------------------------- library cross-check
@pytest.mark.parametrize("causal,window,Hq,Hkv", [(False, 0, 4, 4), (True, 0, 6, 2), (True, 5, 4, 1), (True, 16, 8, 2)])
def test_torch_sdpa_float64(causal, window, Hq, Hkv):
    B, S, D = 2, 37, 16
    q, k, v = rand((B, S, Hq, D), 1), rand((B, S, Hkv, D), 2), rand((B, S, Hkv, D), 3)
    scale = 1.0 / math.sqrt(D)
    o = oracle.attention(q, k, v, scale, causal, window)
    tq, tk, tv = (torch.from_numpy(x).permute(0, 2, 1, 3) for x in (q, k, v))
    if window > 0:
        band = torch.ones(S, S, dtype=torch.bool).tril(0).triu(-(window - 1))
        ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=band, scale=scale, enable_gqa=True)
    else:
        ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=causal, scale=scale, enable_gqa=True)
    ref = ref.permute(0, 2, 1, 3).numpy()
    np.testing.assert_allclose(o, ref, rtol=1e-12, atol=1e-12)


# ----------------------------------------------------------------------------- closed forms
@pytest.mark.parametrize("Sq,Skv,causal,window", [(20, 20, False, 0), (20, 20, True, 0), (13, 29, True, 0), (30, 30, True, 7), (9, 40, True, 12)])
def test_zero_query_gives_window_means(Sq, Skv, causal, window):
    """scale*q.k = 0 for every key, so each row is the plain mean of V over its visible keys."""
    D = 5
    q = np.zeros((1, Sq, 2, D))
    k, v = rand((1, Skv, 1, D), 4), rand((1, Skv, 1, D), 5)
    o = oracle.attention(q, k, v, 0.3, causal, window)
    cs = np.concatenate([np.zeros((1, D)), np.cumsum(v[0, :, 0], axis=0)])  # cs[n] = sum of first n rows
    for i in range(Sq):
        qpos = i + Skv - Sq
        hi = min(Skv, qpos + 1) if causal else Skv
        lo = max(0, qpos - window + 1) if window > 0 else 0
        mean = (cs[hi] - cs[lo]) / (hi - lo)
        np.testing.assert_allclose(o[0, i, 0], mean, rtol=1e-13, atol=1e-14)
        np.testing.assert_array_equal(o[0, i, 0], o[0, i, 1])


def test_constant_v_gives_constant_output():
    q, k = rand((2, 17, 4, 8), 6), rand((2, 17, 2, 8), 7)
    v = np.full((2, 17, 2, 8), -1.375)
    o = oracle.attention(q, k, v, 0.5, True, 5)
    np.testing.assert_allclose(o, -1.375, rtol=4e-16 * 17, atol=0)


def test_identity_v_returns_softmax_rows():
    """V = I (D = Skv) makes each output row the probability row: sums to 1, exact zeros where masked."""
    Sq = Skv = 24
    q, k = rand((1, Sq, 1, 6), 8), rand((1, Skv, 1, 6), 9)
    kpad = np.zeros((1, Skv, 1, Skv))
    kpad[..., :6] = k
    qpad = np.zeros((1, Sq, 1, Skv))
    qpad[..., :6] = q
    v = np.eye(Skv)[None, :, None, :]
    for causal, window in [(False, 0), (True, 0), (True, 6)]:
        p = oracle.attention(qpad, kpad, v, 0.9, causal, window)[0, :, 0, :]
        np.testing.assert_allclose(p.sum(axis=1), 1.0, rtol=0, atol=1e-15)
        vis = oracle.visible_mask(Sq, Skv, causal, window)
        assert (p[~vis] == 0).all() and (p[vis] > 0).all()
        s = 0.9 * (q[0, :, 0] @ k[0, :, 0].T)
        for i in range(Sq):
            e = np.exp(s[i, vis[i]] - s[i, vis[i]].max())
            np.testing.assert_allclose(p[i, vis[i]], e / e.sum(), rtol=1e-14)


# ----------------------------------------------------------------------------- printed values
def test_gqa_printed_example():
    """6 query heads over 2 kv heads map {0,1,2 -> 0; 3,4,5 -> 1}."""
    g = json.load(open(os.path.join(GOLDEN, "gqa_map_bs6_bskv2.json")))
    Hq, Hkv, D = g["bs"], g["bs_kv"], 4
    q, k = rand((1, 3, Hq, D), 10), rand((1, 3, Hkv, D), 11)
    v = np.zeros((1, 3, Hkv, D))
    for kv in range(Hkv):
        v[:, :, kv, :] = 10.0 * (kv + 1)
    o = oracle.attention(q, k, v, 1.0, False)
    got = [int(round(o[0, 0, h, 0] / 10.0)) - 1 for h in range(Hq)]
    assert got == g["kv_of_q"]


def test_gqa_equals_replicated_kv_bitwise():
    q, k, v = rand((2, 19, 8, 8), 12), rand((2, 19, 2, 8), 13), rand((2, 19, 2, 8), 14)
    a = oracle.attention(q, k, v, 0.4, True, 6)
    b = oracle.attention(q, np.repeat(k, 4, axis=2), np.repeat(v, 4, axis=2), 0.4, True, 6)
    assert np.array_equal(a, b)


def affine_select_mask(S, causal, window, qgrp=128, ktile=512):
    """Causal/window mask assembled the way the CTE page describes it: tile skip,
    then per-tile affine predicates  1*p - 1*f + (g*qgrp - k0) >= 0  and, for the
    window, -1*p + 1*f + (k0 + w - 1 - g*qgrp) >= 0."""
    m = np.zeros((S, S), dtype=bool)
    for g in range(-(-S // qgrp)):
        for k0 in range(0, S, ktile):
            max_q, min_q = g * qgrp + qgrp - 1, g * qgrp
            if causal and not (max_q >= k0):
                continue
            if window > 0 and not (min_q < k0 + ktile - 1 + window):
                continue
            for p in range(min(qgrp, S - g * qgrp)):
                for f in range(min(ktile, S - k0)):
                    keep = True
                    if causal:
                        keep &= 1 * p + (-1) * f + (g * qgrp - k0) >= 0
                    if window > 0:
                        keep &= (-1) * p + 1 * f + (k0 + window - 1 - g * qgrp) >= 0
                    m[g * qgrp + p, k0 + f] = keep
    return m


@pytest.mark.parametrize("causal,window", [(True, 0), (True, 200), (True, 513), (True, 1)])
def test_mask_matches_affine_select_construction(causal, window):
    S = 1100
    assert np.array_equal(oracle.visible_mask(S, S, causal, window), affine_select_mask(S, causal, window))


def test_decode_mask_is_index_below_cache_len():
    """One query token at the end of the cache sees exactly the keys with index < cache_len."""
    for L in (1, 7, 16, 33):
        m = oracle.visible_mask(1, L, True, 0)[0]
        assert np.array_equal(m, np.arange(L) < L)
        # and a padded cache: keys at or beyond cache_len never count
        full = np.arange(64) < L
        assert full[:L].all() and not full[L:].any()


def test_mask_sentinel_is_float32_min():
    g = json.load(open(os.path.join(GOLDEN, "mask_sentinel.json")))
    assert g["float32_min"] == float(np.finfo(np.float32).min)


# ----------------------------------------------------------------------------- needles and poison
@pytest.mark.parametrize("causal,window", [(True, 0), (True, 5), (False, 0)])
def test_needles(causal, window):
    """Key j* = 60*q_i/|q_i|^2 gives row i a score gap >= ~50 over all others, so
    o_i == v[j*] bit-exactly when j* is visible, and o_i is untouched by it otherwise."""
    Sq = Skv = 16
    D = 8
    q = rand((1, Sq, 1, D), 15)
    base_k = 0.05 * rand((1, Skv, 1, D), 16)
    v = rand((1, Skv, 1, D), 17)
    vis = oracle.visible_mask(Sq, Skv, causal, window)
    for i in (0, 5, 15):
        for jstar in range(Skv):
            k = base_k.copy()
            k[0, jstar, 0] = 60.0 * q[0, i, 0] / (q[0, i, 0] @ q[0, i, 0])
            o = oracle.attention(q, k, v, 1.0, causal, window)
            if vis[i, jstar]:
                assert np.array_equal(o[0, i, 0], v[0, jstar, 0])
            else:
                ref = oracle.attention(q, base_k, v, 1.0, causal, window)
                assert np.array_equal(o[0, i, 0], ref[0, i, 0])


def test_masked_keys_cannot_leak():
    Sq, Skv = 10, 14
    q, k, v = rand((1, Sq, 2, 4), 18), rand((1, Skv, 1, 4), 19), rand((1, Skv, 1, 4), 20)
    for causal, window in [(True, 0), (True, 3)]:
        ref = oracle.attention(q, k, v, 0.8, causal, window)
        vis = oracle.visible_mask(Sq, Skv, causal, window)
        for i in range(Sq):
            kp, vp = k.copy(), v.copy()
            kp[0, ~vis[i]] = np.nan
            vp[0, ~vis[i]] = np.inf
            o = oracle.attention(q, kp, vp, 0.8, causal, window)
            assert np.array_equal(o[0, i], ref[0, i])


def test_empty_rows_and_sizes():
    q = rand((1, 3, 1, 4), 21)
    k = np.zeros((1, 0, 1, 4))
    o, lse = oracle.attention(q, k, k, 1.0, False, return_lse=True)
    assert (o == 0).all() and (lse == -np.inf).all()
    o = oracle.attention(np.zeros((1, 0, 1, 4)), rand((1, 5, 1, 4), 22), rand((1, 5, 1, 4), 23), 1.0, True)
    assert o.shape == (1, 0, 1, 4)
    # window reaching before the first key, Sq > Skv: early rows see nothing
    q, k, v = rand((1, 6, 1, 4), 24), rand((1, 3, 1, 4), 25), rand((1, 3, 1, 4), 26)
    o, lse = oracle.attention(q, k, v, 1.0, True, 0, return_lse=True)
    assert (o[0, :3] == 0).all() and (lse[0, :3] == -np.inf).all() and (lse[0, 3:] > -np.inf).all()


# ----------------------------------------------------------------------------- recurrence models
def seqdot(a, b):
    acc = 0.0
    for x, y in zip(a.tolist(), b.tolist()):
        acc += x * y
    return acc


def online_softmax_model(q, k, v, scale, vis, tile):
    """The pages' online softmax for one (batch, head): per key tile, m_new = max(m, tile max),
    alpha = exp(m - m_new), l = alpha*l + sum p, O = alpha*O + P V; finally O / l.
    Sequential sums in key order (same order as a row-at-a-time two-pass softmax)."""
    Sq, D = q.shape
    Skv = k.shape[0]
    out = np.zeros((Sq, D))
    for i in range(Sq):
        m, l, acc = -math.inf, 0.0, np.zeros(D)
        for t0 in range(0, Skv, tile):
            js = [j for j in range(t0, min(Skv, t0 + tile)) if vis[i, j]]
            if not js:
                continue
            s = {j: scale * seqdot(q[i], k[j]) for j in js}
            m_new = max(m, max(s.values()))
            alpha = math.exp(m - m_new) if m != -math.inf else 0.0
            l *= alpha
            acc = acc * alpha
            for j in js:
                p = math.exp(s[j] - m_new)
                l += p
                acc = acc + p * v[j]
            m = m_new
        out[i] = acc / l if l > 0 else 0.0
    return out


@pytest.mark.parametrize("tile", [64, 8, 3])
def test_online_recurrence_matches(tile):
    Sq = Skv = 40
    q, k, v = rand((1, Sq, 1, 6), 27), rand((1, Skv, 1, 6), 28), rand((1, Skv, 1, 6), 29)
    k[0, [7, 23, 31]] *= 3.0  # late maxima force alpha < 1
    for causal, window in [(False, 0), (True, 0), (True, 9)]:
        o = oracle.attention(q, k, v, 0.6, causal, window)[0, :, 0]
        vis = oracle.visible_mask(Sq, Skv, causal, window)
        m = online_softmax_model(q[0, :, 0], k[0, :, 0], v[0, :, 0], 0.6, vis, tile)
        if tile >= Skv:  # one tile: the recurrence is the two-pass softmax, same sum order
            assert np.array_equal(m, o)
        else:
            np.testing.assert_allclose(m, o, rtol=1e-13, atol=1e-14)


@pytest.mark.parametrize("splits", [[0, 40], [0, 16, 32, 40], [0, 1, 2, 39, 40]])
def test_split_lse_merge(splits):
    """Attention over key chunks, merged by their log-sum-exp, equals attention over all keys."""
    Sq, Skv, D = 5, 40, 7
    q, k, v = rand((1, Sq, 3, D), 30), rand((1, Skv, 1, D), 31), rand((1, Skv, 1, D), 32)
    full_o, full_lse = oracle.attention(q, k, v, 0.7, False, return_lse=True)
    parts = [oracle.attention(q, np.ascontiguousarray(k[:, a:b]), np.ascontiguousarray(v[:, a:b]), 0.7, False, return_lse=True)
             for a, b in zip(splits[:-1], splits[1:])]
    lses = np.stack([p[1] for p in parts])
    M = lses.max(axis=0)
    w = np.exp(lses - M)
    merged = sum(w[c][..., None] * parts[c][0] for c in range(len(parts))) / w.sum(axis=0)[..., None]
    np.testing.assert_allclose(merged, full_o, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(M + np.log(w.sum(axis=0)), full_lse, rtol=1e-14, atol=1e-14)


# ----------------------------------------------------------------------------- paged decode
def small_decode(seed=40, **kw):
    spec = W.DecodeSpec(batch=5, s_active=1, n_q_heads=8, n_kv_heads=2, head_dim=16, dtype="bf16",
                        page_size=4, len_lo=1, len_hi=23, **kw)
    return W.make_decode(spec, seed)


def test_decode_matches_flat_sdpa():
    d = small_decode()
    s = d.spec
    f64 = lambda a: W.as_f64(a, "bf16")
    o = oracle.decode(f64(d.q), d.k_pool, d.v_pool, d.block_table, d.cache_len, s.scale_f32, to_f64=f64)
    # flat padded cache built by page-by-page copies, then a length mask
    maxlen = s.max_pages_per_seq * s.page_size
    kf = np.zeros((s.batch, maxlen, s.n_kv_heads, s.head_dim))
    vf = np.zeros_like(kf)
    for b in range(s.batch):
        for p in range(s.max_pages_per_seq):
            kf[b, p * s.page_size:(p + 1) * s.page_size] = f64(d.k_pool[d.block_table[b, p]])
            vf[b, p * s.page_size:(p + 1) * s.page_size] = f64(d.v_pool[d.block_table[b, p]])
    for b in range(s.batch):
        mask = torch.from_numpy(np.arange(maxlen) < d.cache_len[b])[None, None, None, :]
        tq = torch.from_numpy(f64(d.q[b:b + 1])).permute(0, 2, 1, 3)
        tk = torch.from_numpy(kf[b:b + 1]).permute(0, 2, 1, 3)
        tv = torch.from_numpy(vf[b:b + 1]).permute(0, 2, 1, 3)
        ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask, scale=s.scale_f32, enable_gqa=True)
        np.testing.assert_allclose(o[b], ref.permute(0, 2, 1, 3).numpy()[0], rtol=1e-12, atol=1e-12)


def test_decode_page_permutation_bitwise():
    """Identity page table over pages laid out in order == the random permutation."""
    d = small_decode(41)
    f64 = lambda a: W.as_f64(a, "bf16")
    o = oracle.decode(f64(d.q), d.k_pool, d.v_pool, d.block_table, d.cache_len, d.spec.scale_f32, to_f64=f64)
    B, maxp = d.block_table.shape
    ident = np.arange(B * maxp, dtype=np.uint32).reshape(B, maxp)
    kp = d.k_pool[d.block_table.reshape(-1)]
    vp = d.v_pool[d.block_table.reshape(-1)]
    o2 = oracle.decode(f64(d.q), kp, vp, ident, d.cache_len, d.spec.scale_f32, to_f64=f64)
    assert np.array_equal(o, o2)


def test_decode_tail_and_unreferenced_pages_cannot_leak():
    d = small_decode(42, extra_pages=3)
    s = d.spec
    f64 = lambda a: W.as_f64(a, "bf16")
    o = oracle.decode(f64(d.q), d.k_pool, d.v_pool, d.block_table, d.cache_len, s.scale_f32, to_f64=f64)
    kp, vp = f64(d.k_pool), f64(d.v_pool)
    used = np.zeros(kp.shape[:2], dtype=bool)
    for b in range(s.batch):
        for t in range(d.cache_len[b]):
            used[d.block_table[b, t // s.page_size], t % s.page_size] = True
    kp[~used] = np.nan
    vp[~used] = np.nan
    o2 = oracle.decode(f64(d.q), kp, vp, d.block_table, d.cache_len, s.scale_f32)
    assert np.array_equal(o, o2)


def test_decode_needles_follow_page_table():
    """A needle key at logical position t of sequence b returns that slot's V exactly;
    V encodes (page, slot), so the output names the physical slot the gather used."""
    d = small_decode(43)
    s = d.spec
    kp = np.zeros(d.k_pool.shape)
    vp = np.zeros(d.v_pool.shape)
    for pg in range(kp.shape[0]):
        for sl in range(s.page_size):
            vp[pg, sl, :, 0] = pg + 1  # nonzero codes: the needle's tiny neighbours round away
            vp[pg, sl, :, 1] = sl + 1
    q = W.as_f64(d.q, "bf16")
    for b in range(s.batch):
        for t in sorted({0, int(d.cache_len[b]) - 1, int(d.cache_len[b]) // 2}):
            k2 = kp.copy()
            pg, sl = d.block_table[b, t // s.page_size], t % s.page_size
            for h in range(s.n_kv_heads):
                qh = q[b, 0, h * (s.n_q_heads // s.n_kv_heads)]
                k2[pg, sl, h] = 200.0 * qh / (qh @ qh)
            o = oracle.decode(q, k2, vp, d.block_table, d.cache_len, 1.0, batches=[b])
            assert o[0, 0, 0, 0] == pg + 1 and o[0, 0, 0, 1] == sl + 1


# ----------------------------------------------------------------------------- input generators
def test_generators_are_seeded_and_round_to_nearest_even():
    spec = W.shrink(W.WORKLOADS["bf16_causal_32k"], seqlen_q=300, seqlen_kv=300)
    a, b = W.make_prefill(spec, 7), W.make_prefill(spec, 7)
    assert all(np.array_equal(x, y) for x, y in [(a.q, b.q), (a.k, b.k), (a.v, b.v)])
    assert a.spike_positions.shape == (1, 3) and len(set(a.spike_positions[0])) == 3
    x = np.random.default_rng(0).standard_normal(4096).astype(np.float32) * 3
    for dt, tdt in (("bf16", torch.bfloat16), ("f16", torch.float16)):
        ours = W.as_f32(W.round_to(x, dt), dt)
        ref = torch.from_numpy(x).to(tdt).float().numpy()
        assert np.array_equal(ours, ref)


# ----------------------------------------------------------------------------- attention sinks
def brute_row_sink(q, k, v, b, i, h, scale, causal, window, sink):
    """mpmath, 50 digits: the sink is one more exponential in the normaliser, with no value row."""
    o, logz = brute_row(q, k, v, b, i, h, scale, causal, window)
    z = mpmath.exp(logz) if logz != -mpmath.inf else mpmath.mpf(0)
    zs = z + mpmath.exp(mpmath.mpf(sink))
    return [x * z / zs for x in o], mpmath.log(zs)


SINK_CASES = [
    # B, Hq, Hkv, Sq, Skv, D, causal, window
    (1, 2, 1, 6, 6, 3, True, 0),
    (2, 4, 2, 5, 9, 4, True, 3),  # Sq < Skv, window
    (1, 3, 3, 7, 7, 2, False, 0),
    (1, 2, 1, 9, 4, 3, True, 0),  # Sq > Skv: the first rows see no key, only the sink
]


@pytest.mark.parametrize("case", SINK_CASES)
def test_sinks_bruteforce_mpmath(case):
    B, Hq, Hkv, Sq, Skv, D, causal, window = case
    seed = 71 + sum(case[:6])
    q, k, v = rand((B, Sq, Hq, D), seed), rand((B, Skv, Hkv, D), seed + 1), rand((B, Skv, Hkv, D), seed + 2)
    sinks = np.linspace(-2.0, 3.0, Hq)
    o, lse = oracle.attention(q, k, v, 0.8, causal, window, return_lse=True, sinks=sinks)
    for b in range(B):
        for i in range(Sq):
            for h in range(Hq):
                ref, ref_lse = brute_row_sink(q, k, v, b, i, h, 0.8, causal, window, sinks[h])
                assert np.allclose(o[b, i, h], [float(x) for x in ref], rtol=1e-13, atol=1e-13)
                assert abs(lse[b, i, h] - float(ref_lse)) <= 1e-13 * max(1.0, abs(float(ref_lse)))


def test_sinks_zero_query_closed_form():
    """All visible scores are 0: o = (sum of visible V) / (n + e^sink), lse = log(n + e^sink)."""
    Sq = Skv = 11
    D = 4
    q = np.zeros((1, Sq, 2, D))
    k, v = rand((1, Skv, 1, D), 81), rand((1, Skv, 1, D), 82)
    sinks = np.array([1.5, -0.75])
    o, lse = oracle.attention(q, k, v, 0.5, True, 4, return_lse=True, sinks=sinks)
    for i in range(Sq):
        lo, hi = max(0, i - 3), i + 1
        for h in range(2):
            den = (hi - lo) + math.exp(sinks[h])
            np.testing.assert_allclose(o[0, i, h], v[0, lo:hi, 0].sum(0) / den, rtol=1e-13, atol=1e-15)
            assert abs(lse[0, i, h] - math.log(den)) <= 1e-13


def test_sinks_rescale_the_plain_result():
    """With a sink, o = o_plain * sigmoid(lse_plain - sink) and lse = logaddexp(lse_plain, sink);
    rows without keys give o = 0 and lse = sink. A sink of -inf changes nothing, bit for bit."""
    q, k, v = rand((2, 10, 4, 8), 91), rand((2, 6, 2, 8), 92), rand((2, 6, 2, 8), 93)
    sinks = np.array([0.3, -4.0, 2.5, 9.0])
    o0, l0 = oracle.attention(q, k, v, 0.6, True, 0, return_lse=True)
    o1, l1 = oracle.attention(q, k, v, 0.6, True, 0, return_lse=True, sinks=sinks)
    for h in range(4):
        seen = np.isfinite(l0[:, :, h])
        sig = 1.0 / (1.0 + np.exp(sinks[h] - l0[:, :, h][seen]))
        np.testing.assert_allclose(o1[:, :, h][seen], o0[:, :, h][seen] * sig[:, None], rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(l1[:, :, h][seen], np.logaddexp(l0[:, :, h][seen], sinks[h]), rtol=1e-13)
        assert (o1[:, :, h][~seen] == 0).all() and (l1[:, :, h][~seen] == sinks[h]).all()
    assert (~np.isfinite(l0)).any()  # Sq > Skv: some rows see no key
    o2, l2 = oracle.attention(q, k, v, 0.6, True, 0, return_lse=True, sinks=np.full(4, -np.inf))
    np.testing.assert_array_equal(o2, o0)
    np.testing.assert_array_equal(l2, l0)


def test_nan_and_inf_sinks_give_nan_rows():
    """A NaN sink logit has a NaN exponential, and a +inf one makes the max +inf and its own
    exponential exp(inf - inf) = NaN (IEEE 754), so the normaliser is NaN in both cases: every row
    of that head, also one that sees no key, is NaN (output and lse); other heads are untouched."""
    q, k, v = rand((1, 9, 4, 8), 94), rand((1, 5, 2, 8), 95), rand((1, 5, 2, 8), 96)
    sinks = np.array([np.nan, 0.5, np.inf, -np.inf])
    o, l = oracle.attention(q, k, v, 0.6, True, 0, return_lse=True, sinks=sinks)
    assert np.isnan(o[:, :, [0, 2]]).all() and np.isnan(l[:, :, [0, 2]]).all()
    o1, l1 = oracle.attention(q, k, v, 0.6, True, 0, return_lse=True, sinks=np.array([0.0, 0.5, 0.0, -np.inf]))
    np.testing.assert_array_equal(o[:, :, [1, 3]], o1[:, :, [1, 3]])
    np.testing.assert_array_equal(l[:, :, [1, 3]], l1[:, :, [1, 3]])


# ----------------------------------------------------------------------------- FP8 E4M3 storage of the inputs
def test_e4m3_decode_table_matches_torch():
    """The generator's value of every code equals torch's float8_e4m3fn widening (a library routine)."""
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    mine = W.E4M3_VALUES
    assert np.array_equal(np.isnan(mine), np.isnan(ref))
    assert np.array_equal(mine[~np.isnan(ref)], ref[~np.isnan(ref)])
    assert mine[0x7E] == 448.0 and mine[1] == 2.0 ** -9 and mine[0x38] == 1.0


def test_e4m3_rounding_is_nearest_even_and_saturating():
    rng = np.random.default_rng(17)
    x = np.concatenate([rng.standard_normal(200000) * s for s in (0.004, 1.0, 60.0)]).astype(np.float32)
    mids = (W.E4M3_VALUES[1:127] + W.E4M3_VALUES[0:126]) / 2  # exact ties between neighbours
    x = np.concatenate([x, mids.astype(np.float32), -mids.astype(np.float32), [0.0, -0.0, 448.0, 449.0, 464.0, 1e20]])
    x = x.astype(np.float32)
    mine = W.f32_to_e4m3_bits_by_definition(x)
    # torch's conversion (ties to even; it turns values past the top into NaN, so compare within range)
    within = np.abs(x) <= 448.0
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(mine[within], ref[within])
    assert (mine[np.abs(x) > 448.0] & 0x7F == 0x7E).all()  # saturated at +-448
    # nearest value by search over the decoded table, ties to the even code
    small = x[:20000]
    a = np.minimum(np.abs(small).astype(np.float64), 448.0)
    d = np.abs(a[:, None] - W.E4M3_VALUES[None, :127])
    cand = np.where(d == d.min(1, keepdims=True), np.arange(127)[None, :], 999)
    even = np.where(cand % 2 == 0, cand, 999).min(1)
    code = np.where(even < 999, even, cand.min(1)).astype(np.uint8) | np.where(np.signbit(small), 0x80, 0).astype(np.uint8)
    np.testing.assert_array_equal(mine[:20000], code)
    # the bulk path of the generator is the same rounding
    big = np.tile(x, 3)
    np.testing.assert_array_equal(W.f32_to_e4m3_bits(big), W.f32_to_e4m3_bits_by_definition(big))


# ----------------------------------------------------------------------------- packed sequences
def packed_case(lens_q, lens_kv, Hq, Hkv, D, seed):
    cq = np.concatenate([[0], np.cumsum(lens_q)]).astype(np.int64)
    ck = np.concatenate([[0], np.cumsum(lens_kv)]).astype(np.int64)
    q = rand((int(cq[-1]), Hq, D), seed)
    k, v = rand((int(ck[-1]), Hkv, D), seed + 1), rand((int(ck[-1]), Hkv, D), seed + 2)
    return q, k, v, cq, ck


@pytest.mark.parametrize("causal,window", [(False, 0), (True, 0), (True, 3)])
def test_varlen_matches_sdpa_with_a_segment_mask(causal, window):
    """One float64 SDPA over the whole packed batch with a mask built from
    segment ids and positions (not from per-sequence slices)."""
    lens_q, lens_kv = [5, 0, 9, 3, 7], [5, 4, 12, 3, 0]  # a prefix-prior sequence, an empty q, an empty kv
    Hq, Hkv, D = 6, 2, 8
    q, k, v, cq, ck = packed_case(lens_q, lens_kv, Hq, Hkv, D, 41)
    scale = 0.45
    o, lse = oracle.attention_varlen(q, k, v, cq, ck, scale, causal, window, return_lse=True)
    seg_q = np.repeat(np.arange(len(lens_q)), lens_q)
    seg_k = np.repeat(np.arange(len(lens_kv)), lens_kv)
    pos_q = np.arange(q.shape[0]) - cq[seg_q] + (np.asarray(lens_kv) - np.asarray(lens_q))[seg_q]
    idx_k = np.arange(k.shape[0]) - ck[seg_k]
    mask = seg_q[:, None] == seg_k[None, :]
    if causal:
        mask &= idx_k[None, :] <= pos_q[:, None]
    if window > 0:
        mask &= idx_k[None, :] >= pos_q[:, None] - window + 1
    tq = torch.from_numpy(q).permute(1, 0, 2)[None]
    tk, tv = (torch.from_numpy(x).permute(1, 0, 2)[None] for x in (k, v))
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=torch.from_numpy(mask), scale=scale,
                                                           enable_gqa=True)[0].permute(1, 0, 2).numpy()
    seen = mask.any(axis=1)
    np.testing.assert_allclose(o[seen], ref[seen], rtol=1e-12, atol=1e-12)
    assert np.all(o[~seen] == 0.0) and np.all(lse[~seen] == -np.inf)
    # log-sum-exp over the same mask, from the same scores computed here
    s = scale * np.einsum("qhd,khd->hqk", q, np.repeat(k, Hq // Hkv, axis=1))
    s = np.where(mask[None], s, -np.inf)
    with np.errstate(divide="ignore"):
        ref_lse = np.log(np.exp(s).sum(axis=2)).T
    np.testing.assert_allclose(lse[seen], ref_lse[seen], rtol=1e-12, atol=1e-12)


def test_varlen_equal_lengths_equal_the_batched_oracle_bitwise():
    B, S, Hq, Hkv, D = 3, 11, 4, 2, 8
    q, k, v, cq, ck = packed_case([S] * B, [S] * B, Hq, Hkv, D, 43)
    o = oracle.attention_varlen(q, k, v, cq, ck, 0.3, True, 4)
    ob = oracle.attention(q.reshape(B, S, Hq, D), k.reshape(B, S, Hkv, D), v.reshape(B, S, Hkv, D), 0.3, True, 4)
    assert np.array_equal(o, ob.reshape(B * S, Hq, D))


def test_varlen_sequence_order_does_not_matter():
    lens = [4, 9, 1, 6]
    q, k, v, cq, ck = packed_case(lens, lens, 2, 1, 4, 45)
    o = oracle.attention_varlen(q, k, v, cq, ck, 0.8, True)
    perm = [2, 0, 3, 1]
    take_q = np.concatenate([np.arange(cq[b], cq[b + 1]) for b in perm])
    take_k = np.concatenate([np.arange(ck[b], ck[b + 1]) for b in perm])
    lp = [lens[b] for b in perm]
    cp = np.concatenate([[0], np.cumsum(lp)])
    op = oracle.attention_varlen(q[take_q], k[take_k], v[take_k], cp, cp, 0.8, True)
    assert np.array_equal(op, o[take_q])


# ----------------------------------------------------------------------------- per-row positions
def brute_row_at(q, k, v, b, i, h, scale, causal, window, qpos):
    """brute_row with the query position given, not derived from the shapes."""
    mpmath.mp.dps = 50
    D = q.shape[3]
    Skv, Hkv = k.shape[1], k.shape[2]
    hk = h // (q.shape[2] // Hkv)
    hi = min(Skv, qpos + 1) if causal else Skv
    lo = max(0, qpos - window + 1) if window > 0 else 0
    keys = list(range(lo, max(lo, hi)))
    if not keys:
        return [mpmath.mpf(0)] * D, -mpmath.inf
    e = [mpmath.exp(mpmath.mpf(scale) * mpmath.fsum(mpmath.mpf(q[b, i, h, d]) * mpmath.mpf(k[b, j, hk, d])
                                                  for d in range(D))) for j in keys]
    Z = mpmath.fsum(e)
    return [mpmath.fsum(e[t] * mpmath.mpf(v[b, j, hk, d]) for t, j in enumerate(keys)) / Z for d in range(D)], \
        mpmath.log(Z)


@pytest.mark.parametrize("causal,window", [(True, 0), (True, 3), (False, 0)])
def test_positions_bruteforce_mpmath(causal, window):
    Sq, Skv, Hq, Hkv, D = 7, 12, 2, 1, 4
    q, k, v = rand((1, Sq, Hq, D), 61), rand((1, Skv, Hkv, D), 62), rand((1, Skv, Hkv, D), 63)
    pos = np.array([-2, 0, 0, 3, 7, 11, 15])  # repeats, gaps, a row before the first key, one past the last
    o, lse = oracle.attention(q, k, v, 0.6, causal, window, return_lse=True, positions=pos)
    for i in range(Sq):
        for h in range(Hq):
            ref, ref_lse = brute_row_at(q, k, v, 0, i, h, 0.6, causal, window, int(pos[i]))
            assert np.allclose(o[0, i, h], [float(x) for x in ref], rtol=1e-13, atol=1e-13)
            if ref_lse == -mpmath.inf:
                assert lse[0, i, h] == -np.inf
            else:
                assert abs(lse[0, i, h] - float(ref_lse)) <= 1e-13 * max(1.0, abs(float(ref_lse)))


def test_positions_of_the_default_alignment_change_nothing():
    Sq, Skv = 9, 14
    q, k, v = rand((2, Sq, 4, 8), 64), rand((2, Skv, 2, 8), 65), rand((2, Skv, 2, 8), 66)
    a = oracle.attention(q, k, v, 0.4, True, 5)
    b = oracle.attention(q, k, v, 0.4, True, 5, positions=np.arange(Sq) + Skv - Sq)
    assert np.array_equal(a, b)


def test_varlen_positions_match_sdpa_with_a_position_mask():
    lens_q, lens_kv = [6, 4, 9], [10, 4, 20]
    q, k, v, cq, ck = packed_case(lens_q, lens_kv, 4, 2, 8, 67)
    rng = np.random.default_rng(68)
    pos = np.concatenate([np.sort(rng.integers(0, L, n)) for n, L in zip(lens_q, lens_kv)])
    o = oracle.attention_varlen(q, k, v, cq, ck, 0.5, True, 4, positions=pos)
    seg_q = np.repeat(np.arange(3), lens_q)
    seg_k = np.repeat(np.arange(3), lens_kv)
    idx_k = np.arange(k.shape[0]) - ck[seg_k]
    mask = (seg_q[:, None] == seg_k[None, :]) & (idx_k[None, :] <= pos[:, None]) & (idx_k[None, :] >= pos[:, None] - 3)
    tq = torch.from_numpy(q).permute(1, 0, 2)[None]
    tk, tv = (torch.from_numpy(x).permute(1, 0, 2)[None] for x in (k, v))
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=torch.from_numpy(mask), scale=0.5,
                                                           enable_gqa=True)[0].permute(1, 0, 2).numpy()
    np.testing.assert_allclose(o, ref, rtol=1e-12, atol=1e-12)


def test_attention_rows_rejects_rows_outside_the_tensors():
    """A row index outside [B, Sq, Hq] raises instead of reading out of bounds."""
    rng = np.random.default_rng(5)
    q = rng.standard_normal((2, 5, 3, 8))
    k = rng.standard_normal((2, 7, 1, 8))
    for bad in ((0, -1, 0), (2, 0, 0), (0, 5, 0), (0, 0, 3)):
        with pytest.raises(ValueError):
            oracle.attention_rows(q, k, k, 0.3, True, 0, np.array([bad]))
    o, _ = oracle.attention_rows(q, k, k, 0.3, True, 0, np.array([(1, 4, 2)]))
    assert o.shape == (1, 8)
