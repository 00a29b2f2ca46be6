"""Pins of the CPU oracle to facts that do not come from the oracle itself.

Each test ties one part of the oracle to a value the pages print, a closed form,
an invariant, a library routine on a special case, or brute force on tiny inputs,
so that a dropped term, a wrong sign or index, or a transposed operand anywhere in
the oracle fails at least one of them.
"""
import dataclasses
import itertools
import json
import math
import os
from decimal import Decimal, getcontext
from fractions import Fraction

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from sparse_decode_amd import synth


# ----------------------------------------------------------------------------------
# Worked example printed on the page (Tutorial, "MHA et GQA")
# ----------------------------------------------------------------------------------
def test_cache_bytes_worked_example(golden_dir):
    with open(os.path.join(golden_dir, "cache_size_worked_example.json")) as f:
        gold = json.load(f)
    for c in gold["cases"]:
        got = c["sequences"] * oracle.cache_bytes(c["L"], c["S"], c["n_kv"], c["d_h"], c["b"])
        assert got == c["bytes"], c["what"]
    # 512 MiB and 2 GiB as the page states them
    assert oracle.cache_bytes(32, 4096, 8, 128, 2) == 512 * 2**20
    # GQA shrinks the cache by n_kv / n_h relative to MHA
    assert oracle.cache_bytes(32, 4096, 8, 128, 2) * 4 == oracle.cache_bytes(32, 4096, 32, 128, 2)


def _rand(shape, seed, scale=1.0):
    return (np.random.default_rng(seed).standard_normal(shape) * scale).astype(np.float32)


# ----------------------------------------------------------------------------------
# Softmax rows sum to one: the window score sums to (number of rows that see a key)
# ----------------------------------------------------------------------------------
@pytest.mark.parametrize("n_h,n_kv,w,wic", [(4, 2, 8, True), (8, 1, 4, True), (4, 4, 3, False), (6, 2, 1, False)])
def test_score_rows_sum_to_one(n_h, n_kv, w, wic):
    B, S, d = 2, 97, 16
    q = _rand((B, n_h, w, d), 1)
    k = _rand((B, n_kv, S, d), 2)
    sl = np.array([97, 40], np.int32)
    raw, pooled, raw64 = oracle.score_window(q, k, w, seq_lens=sl, window_in_cache=wic, n_keep=w,
                                             pool=3, want_raw64=True)
    r = n_h // n_kv
    for b in range(B):
        for g in range(n_kv):
            assert abs(raw64[b, g].sum() - r * w) < 1e-11
            assert np.all(raw64[b, g, sl[b]:] == 0.0)
    # one row: exactly a softmax
    raw1, _, raw64_1 = oracle.score_window(q[:, :1, :1], k[:, :1], 1, window_in_cache=False, n_keep=1,
                                           pool=1, want_raw64=True)
    assert abs(raw64_1[0, 0].sum() - 1.0) < 1e-13


def test_score_row_with_no_visible_key_adds_nothing():
    # S_b < w with the window in the cache: rows i < w - S_b see no key.
    q = _rand((1, 2, 8, 4), 3)
    k = _rand((1, 1, 16, 4), 4)
    _, _, raw64 = oracle.score_window(q, k, 8, seq_lens=np.array([5], np.int32), n_keep=8, pool=1,
                                      want_raw64=True)
    assert abs(raw64[0, 0].sum() - 2 * 5) < 1e-12   # rows i = 3..7 of both heads see >= 1 key


# ----------------------------------------------------------------------------------
# Closed form with identical keys: every visible logit of a row is equal, so row i
# gives 1/(S - w + i + 1) to each key it sees (causal alignment, Tutorial section
# "Quand la reutilisation est-elle exacte ?").
# ----------------------------------------------------------------------------------
def _uniform_key_closed_form(S, w, r, t, top_left=False):
    tot = Fraction(0)
    for i in range(w):
        last = i if top_left else S - w + i
        if t <= last:
            tot += Fraction(1, last + 1)
    return r * tot


def test_uniform_keys_closed_form_and_ties():
    wl = synth.WORKLOADS[1]
    S, w, r, d = wl.s_max, wl.w, wl.group, wl.d_h
    q = _rand((1, wl.n_h, w, d), 5)
    row = _rand((d,), 6)
    k = np.broadcast_to(row, (1, wl.n_kv, S, d)).copy()
    raw, pooled, raw64 = oracle.score_window(q, k, w, n_keep=wl.n_keep, pool=wl.pool, want_raw64=True)
    # printed value for the tiny shape: r * (H_S - H_{S-w}) = 0.0634344...
    assert abs(raw64[0, 0, 0] - 0.06343443427670455) < 1e-15
    for t in [0, 1, 200, S - w - 1, S - w, S - w + 1, S - 2, S - 1]:
        want = float(_uniform_key_closed_form(S, w, r, t))
        assert abs(raw64[0, 0, t] - want) <= 1e-14 * want, t
        # a top-left aligned mask would give a different value (the pin sees the mask)
        naive = float(_uniform_key_closed_form(S, w, r, t, top_left=True))
        assert abs(naive - want) > 1e-6 * want or t >= S - w
    # all candidates tie -> the lowest indices win, then the window
    idx, count = oracle.select_topk(pooled, wl.k, wl.n_keep)
    want = list(range(wl.k)) + list(range(S - wl.n_keep, S))
    for g in range(wl.n_kv):
        assert count[0, g] == wl.k + wl.n_keep
        assert idx[0, g].tolist() == want


# ----------------------------------------------------------------------------------
# Brute force at 50 decimal digits on tiny inputs
# ----------------------------------------------------------------------------------
getcontext().prec = 50


def _dec_score(q, k, S, w, wic, scale):
    """p_t = 1 / sum_u exp(x_u - x_t): the softmax written another way."""
    n_h, d = q.shape[0], q.shape[-1]
    n_kv = k.shape[0]
    r = n_h // n_kv
    sc = Decimal(scale)
    raw = [[Decimal(0)] * S for _ in range(n_kv)]
    for h in range(n_h):
        g = h // r
        for i in range(w):
            last = S - w + i if wic else S - 1
            last = min(last, S - 1)
            if last < 0:
                continue
            xs = [sc * sum(Decimal(float(q[h, i, e])) * Decimal(float(k[g, t, e])) for e in range(d))
                  for t in range(last + 1)]
            for t in range(last + 1):
                raw[g][t] += 1 / sum((xu - xs[t]).exp() for xu in xs)
    return raw


def _brute_select(scores, k, n_keep, S):
    C = max(0, S - n_keep)
    k_eff = min(k, C)
    best = None
    for sub in itertools.combinations(range(C), k_eff):
        key = sorted((-scores[t], t) for t in sub)
        if best is None or key < best[0]:
            best = (key, sub)
    return sorted(best[1]) + list(range(C, S))


@pytest.mark.parametrize("seed,n_h,n_kv,S,w,wic,k,pool", [
    (11, 2, 1, 10, 3, True, 3, 3),
    (12, 2, 2, 9, 2, True, 4, 3),
    (13, 3, 1, 8, 1, False, 2, 1),
    (14, 4, 2, 11, 3, True, 3, 5),
])
def test_bruteforce_tiny(seed, n_h, n_kv, S, w, wic, k, pool):
    d = 3
    q = _rand((1, n_h, w, d), seed, 2.0)
    kk = _rand((1, n_kv, S, d), seed + 100, 2.0)
    scale = 1 / math.sqrt(d)
    raw, pooled, raw64 = oracle.score_window(q, kk, w, window_in_cache=wic, n_keep=w, pool=pool,
                                             scale=scale, want_raw64=True)
    dec = _dec_score(q[0], kk[0], S, w, wic, scale)
    for g in range(n_kv):
        for t in range(S):
            assert abs(raw64[0, g, t] - float(dec[g][t])) <= 1e-14 * max(1.0, float(dec[g][t]))
            assert raw[0, g, t] == np.float32(float(dec[g][t]))
        C = S - w
        for t in range(S):
            if t < C:
                lo, hi = max(0, t - pool // 2), min(C - 1, t + pool // 2)
                want = max(raw[0, g, lo:hi + 1])
            else:
                want = raw[0, g, t]
            assert pooled[0, g, t] == want
    idx, count = oracle.select_topk(pooled, k, w)
    for g in range(n_kv):
        want = _brute_select([float(x) for x in pooled[0, g]], k, w, S)
        assert count[0, g] == len(want)
        assert idx[0, g, :len(want)].tolist() == want
    # decode by the direct formula
    qd = _rand((1, n_h, d), seed + 200)
    cnt = np.array([[5] * n_kv], np.int32)
    vv = _rand((1, n_kv, 5, d), seed + 300)
    kc = kk[:, :, :5].copy()
    out, lse = oracle.decode(qd, kc, vv, cnt, scale=scale)
    r = n_h // n_kv
    for h in range(n_h):
        g = h // r
        ys = [Decimal(scale) * sum(Decimal(float(qd[0, h, e])) * Decimal(float(kc[0, g, t, e])) for e in range(d))
              for t in range(5)]
        Z = sum(y.exp() for y in ys)
        for e in range(d):
            want = sum(y.exp() / Z * Decimal(float(vv[0, g, t, e])) for t, y in enumerate(ys))
            assert abs(out[0, h, e] - float(want)) < 1e-14
        assert abs(lse[0, h] - float(Z.ln())) < 1e-14


# ----------------------------------------------------------------------------------
# Special cases that reduce to library routines (torch CPU, float64)
# ----------------------------------------------------------------------------------
def _torch_raw(q, k, w, S, wic, scale, gqa_map="block"):
    qt = torch.from_numpy(q).double()[0]          # [n_h][w][d]
    kt = torch.from_numpy(k).double()[0, :, :S]   # [n_kv][S][d]
    n_h, n_kv = qt.shape[0], kt.shape[0]
    r = n_h // n_kv
    if gqa_map == "block":
        kh = kt.repeat_interleave(r, dim=0)       # head h reads KV head h // r
    else:
        kh = kt.repeat(r, 1, 1)                   # a wrong map: head h reads h % n_kv
    logits = torch.matmul(qt, kh.transpose(1, 2)) * scale
    if wic:
        vis = torch.ones(w, S, dtype=torch.bool).tril(diagonal=S - w)
        logits = logits.masked_fill(~vis, float("-inf"))
    p = torch.softmax(logits, dim=-1)             # [n_h][w][S]
    if gqa_map == "block":
        return p.reshape(n_kv, r * w, S).sum(1)
    return p.reshape(r, n_kv, w, S).sum((0, 2))


@pytest.mark.parametrize("n_h,n_kv,wic", [(8, 2, True), (4, 4, True), (4, 1, False)])
def test_torch_crosscheck(n_h, n_kv, wic):
    S, w, d, pool, k_bud = 300, 8, 32, 7, 40
    q = _rand((1, n_h, w, d), 21)
    kk = _rand((1, n_kv, S, d), 22)
    scale = 1 / math.sqrt(d)
    raw, pooled, raw64 = oracle.score_window(q, kk, w, window_in_cache=wic, n_keep=w, pool=pool,
                                             want_raw64=True)
    ref = _torch_raw(q, kk, w, S, wic, scale)
    assert torch.allclose(torch.from_numpy(raw64[0]), ref, rtol=1e-12, atol=1e-15)
    if 1 < n_kv < n_h:   # the pin would catch a wrong query-head -> KV-head map
        wrong = _torch_raw(q, kk, w, S, wic, scale, gqa_map="mod")
        assert not torch.allclose(torch.from_numpy(raw64[0]), wrong, rtol=1e-6)
    C = S - w
    rt = torch.from_numpy(raw[0]).double()
    mp = F.max_pool1d(rt[:, :C].unsqueeze(0), kernel_size=pool, stride=1, padding=pool // 2)[0]
    assert torch.equal(mp.float(), torch.from_numpy(pooled[0, :, :C]))
    assert np.array_equal(pooled[0, :, C:], raw[0, :, C:])
    idx, count = oracle.select_topk(pooled, k_bud, w)
    for g in range(n_kv):
        order = torch.sort(torch.from_numpy(pooled[0, g, :C]), descending=True, stable=True).indices
        want = sorted(order[:k_bud].tolist()) + list(range(C, S))
        assert idx[0, g].tolist() == want and count[0, g] == k_bud + w
    # decode over the compacted cache == attention over the full cache with a keep mask
    v = _rand((1, n_kv, S, d), 23)
    qd = _rand((1, n_h, d), 24)
    kc, _ = oracle.gather(kk, idx, count)
    vc, _ = oracle.gather(v, idx, count)
    out, lse = oracle.decode(qd, kc, vc, count)
    r = n_h // n_kv
    keep = torch.zeros(n_kv, S, dtype=torch.bool)
    for g in range(n_kv):
        keep[g, torch.from_numpy(idx[0, g].astype(np.int64))] = True
    Kf = torch.from_numpy(kk[0]).double().repeat_interleave(r, 0)
    Vf = torch.from_numpy(v[0]).double().repeat_interleave(r, 0)
    ref_out = F.scaled_dot_product_attention(torch.from_numpy(qd[0]).double()[:, None, :], Kf, Vf,
                                             attn_mask=keep.repeat_interleave(r, 0)[:, None, :])[:, 0]
    assert torch.allclose(torch.from_numpy(out[0]), ref_out, rtol=1e-12, atol=1e-13)


def test_shared_heads_exact_dyadic_sums():
    """Scores that are multiples of 2^-8 below 16 add exactly in any float type, so the
    shared (TSP) score is an integer count of 2^-8 units: the selection is brute-forced
    on Python integers (no floating point at all), ties and all."""
    rng = np.random.default_rng(31)
    for B, H, S, k, n_keep, levels in ((2, 5, 64, 10, 4, 7), (1, 32, 300, 57, 32, 3), (3, 8, 129, 0, 8, 50),
                                       (2, 3, 40, 40, 0, 4), (1, 4, 33, 5, 40, 9)):
        units = rng.integers(0, levels, size=(B, H, S))
        sc = (units / 256.0).astype(np.float32)
        idx, count = oracle.select_topk(sc, k, n_keep, shared_heads=True)
        assert idx.shape == (B, 1, k + n_keep)
        for b in range(B):
            tot = [int(units[b, :, t].sum()) for t in range(S)]
            C = max(0, S - n_keep)
            k_eff = min(k, C)
            best = sorted(range(C), key=lambda t: (-tot[t], t))[:k_eff]
            want = sorted(best) + list(range(C, S))
            assert idx[b, 0, :len(want)].tolist() == want
            assert np.all(idx[b, 0, len(want):] == -1)
            assert count[b, 0] == len(want)


def test_shared_heads_of_identical_heads_equal_per_head_selection():
    """H identical heads: the summed score is H times each head's, which orders the
    tokens as one head does, so the shared selection equals the per-head one."""
    rng = np.random.default_rng(32)
    for H in (1, 2, 7, 32):
        one = rng.random((2, 1, 200)).astype(np.float32)
        one[0, 0, 50:60] = one[0, 0, 10]                       # exact ties too
        sc = np.repeat(one, H, axis=1)
        si, sc_count = oracle.select_topk(sc, 37, 16, shared_heads=True)
        pi, p_count = oracle.select_topk(one, 37, 16)
        assert np.array_equal(si, pi) and np.array_equal(sc_count, p_count)


def test_shared_heads_sum_is_exact_not_float_head_order():
    """The shared score is the exact sum over heads.  Token 0 holds 1 + 3 * 2^-24
    spread as 1, 2^-24, 2^-24, 2^-24; token 1 holds 1 + 2^-23 in its first head.
    Added in float in head order, each 2^-24 is lost (ties to even) and token 1
    would win; exactly, token 0 is larger and is the one kept."""
    e = 2.0 ** -24
    sc = np.zeros((1, 4, 3), np.float32)
    sc[0, :, 0] = [1.0, e, e, e]
    sc[0, :, 1] = [1.0 + 2 * e, 0.0, 0.0, 0.0]
    sc[0, :, 2] = [0.5, 0.0, 0.0, 0.0]
    f = np.float32(0.0)
    for g in range(4):
        f = np.float32(f + sc[0, g, 0])
    assert f == np.float32(1.0) < sc[0, 0, 1]            # the float head-order sum ranks token 1 first
    idx, count = oracle.select_topk(sc, 1, 0, shared_heads=True)
    assert idx.tolist() == [[[0]]] and count.tolist() == [[1]]
    idx, count = oracle.select_topk(sc, 2, 0, shared_heads=True)
    assert idx.tolist() == [[[0, 1]]]


# ----------------------------------------------------------------------------------
# Dense equivalence: a budget covering every candidate gives plain attention
# ----------------------------------------------------------------------------------
def test_dense_equivalence():
    n_h, n_kv, S, d, w = 8, 2, 200, 16, 4
    q = _rand((1, n_h, w, d), 41)
    kk = _rand((1, n_kv, S, d), 42)
    v = _rand((1, n_kv, S, d), 43)
    qd = _rand((1, n_h, d), 44)
    _, pooled = oracle.score_window(q, kk, w, n_keep=w, pool=7)
    idx, count = oracle.select_topk(pooled, S, w)      # k >= S - n_keep
    assert np.all(count == S)
    assert np.array_equal(idx[0, :, :S], np.tile(np.arange(S), (n_kv, 1)))
    kc, _ = oracle.gather(kk, idx, count)
    vc, _ = oracle.gather(v, idx, count)
    out, lse = oracle.decode(qd, kc, vc, count)
    r = n_h // n_kv
    for h in range(n_h):
        g = h // r
        y = kk[0, g].astype(np.float64) @ qd[0, h].astype(np.float64) / math.sqrt(d)
        p = np.exp(y - y.max())
        want = (p / p.sum()) @ v[0, g].astype(np.float64)
        assert np.allclose(out[0, h], want, rtol=1e-12, atol=1e-13)
        assert abs(lse[0, h] - (y.max() + math.log(p.sum()))) < 1e-12


# ----------------------------------------------------------------------------------
# Invariants of selection and gather
# ----------------------------------------------------------------------------------
def test_select_gather_invariants():
    rng = np.random.default_rng(51)
    B, H, s_max = 3, 4, 500
    sc = (rng.integers(0, 20, (B, H, s_max)) / 7.0).astype(np.float32)   # many exact ties
    sl = np.array([500, 37, 3], np.int32)
    k, n_keep = 60, 16
    idx, count = oracle.select_topk(sc, k, n_keep, seq_lens=sl)
    src_pos = rng.permutation(10_000)[: B * s_max].reshape(B, s_max).astype(np.int32)
    rows = rng.integers(0, 2**16, (B, H, s_max, 8)).astype(np.uint16)
    dst, pos = oracle.gather(rows, idx, count, src_pos=src_pos)
    for b in range(B):
        S = int(sl[b])
        C = max(0, S - n_keep)
        for h in range(H):
            n = int(count[b, h])
            assert n == min(k, C) + (S - C)
            sel = idx[b, h, :n]
            assert np.all(np.diff(sel) > 0) and sel.min(initial=0) >= 0 and sel.max(initial=0) < max(S, 1)
            assert set(range(C, S)) <= set(sel.tolist())
            assert np.all(idx[b, h, n:] == -1)
            # every selected candidate beats (or ties with a higher index than) every unselected one
            chosen = [t for t in sel if t < C]
            rest = sorted(set(range(C)) - set(chosen))
            if chosen and rest:
                worst = min((-(-sc[b, h, t]), -t) for t in chosen)
                best_rest = max((sc[b, h, t], -t) for t in rest)
                assert worst > best_rest
            assert np.array_equal(pos[b, h, :n], src_pos[b, sel])
            assert np.all(pos[b, h, n:] == -1)
            assert np.array_equal(dst[b, h, :n], rows[b, h, sel])
            assert np.all(dst[b, h, n:] == 0)


def test_select_degenerate_cases():
    sc = np.random.default_rng(61).random((1, 2, 50)).astype(np.float32)
    # n_keep >= S_b: everything kept, no candidate
    idx, count = oracle.select_topk(sc, 10, 8, seq_lens=np.array([5], np.int32))
    assert count.tolist() == [[5, 5]] and idx[0, 0, :5].tolist() == list(range(5))
    # k = 0: only the window
    idx, count = oracle.select_topk(sc, 0, 8)
    assert count.tolist() == [[8, 8]] and idx[0, 1].tolist() == list(range(42, 50))
    # S_b = 0: nothing
    idx, count = oracle.select_topk(sc, 10, 8, seq_lens=np.array([0], np.int32))
    assert count.tolist() == [[0, 0]] and np.all(idx == -1)


# ----------------------------------------------------------------------------------
# Planted heavy hitters are always selected
# ----------------------------------------------------------------------------------
def test_planted_heavy_hitters_tiny():
    wl = synth.WORKLOADS[1]
    for layer in range(6):
        inp = synth.layer_inputs(wl, layer=layer)
        q = synth.to_host_f32(inp["q_win"])
        k = synth.to_host_f32(inp["k"])
        _, pooled = oracle.score_window(q, k, wl.w, n_keep=wl.n_keep, pool=wl.pool)
        idx, count = oracle.select_topk(pooled, wl.k, wl.n_keep)
        planted = set(inp["planted"][0].tolist())
        assert len(planted) == 8
        for g in range(wl.n_kv):
            assert planted <= set(idx[0, g, : count[0, g]].tolist()), (layer, g)


def test_planted_heavy_hitters_bf16_shape():
    wl = dataclasses.replace(synth.WORKLOADS[2], s_max=6144, k=256)
    inp = synth.layer_inputs(wl, layer=3)
    q = synth.to_host_f32(inp["q_win"])
    k = synth.to_host_f32(inp["k"])
    planted = set(inp["planted"][0].tolist())
    assert len(planted) == math.ceil(0.01 * 6144)
    for pool in (1, 7):
        _, pooled = oracle.score_window(q, k, wl.w, n_keep=wl.n_keep, pool=pool)
        idx, count = oracle.select_topk(pooled, wl.k, wl.n_keep)
        for g in range(wl.n_kv):
            sel = set(idx[0, g, : count[0, g]].tolist())
            if pool == 1 or len(planted) * pool <= wl.k:
                assert planted <= sel, (pool, g)
            else:
                assert len(planted & sel) >= wl.k // pool


# ----------------------------------------------------------------------------------
# Decode closed forms
# ----------------------------------------------------------------------------------
def test_decode_closed_forms():
    n_h, n_kv, cap, d = 4, 2, 9, 8
    q = _rand((1, n_h, d), 71)
    kc = _rand((1, n_kv, cap, d), 72)
    vc = _rand((1, n_kv, cap, d), 73)
    # one token: the output is that V row
    out, lse = oracle.decode(q, kc, vc, np.array([[1, 1]], np.int32))
    for h in range(n_h):
        assert np.allclose(out[0, h], vc[0, h // 2, 0], rtol=0, atol=1e-15)
        assert abs(lse[0, h] - np.dot(q[0, h].astype(np.float64), kc[0, h // 2, 0]) / math.sqrt(d)) < 1e-12
    # identical keys, or q = 0: the mean of the V rows
    same = np.broadcast_to(kc[:, :, :1], kc.shape).copy()
    out, _ = oracle.decode(q, same, vc, np.array([[6, 9]], np.int32))
    assert np.allclose(out[0, 0], vc[0, 0, :6].astype(np.float64).mean(0), atol=1e-14)
    assert np.allclose(out[0, 3], vc[0, 1, :9].astype(np.float64).mean(0), atol=1e-14)
    out, _ = oracle.decode(np.zeros_like(q), kc, vc, np.array([[9, 9]], np.int32))
    assert np.allclose(out[0, 2], vc[0, 1].astype(np.float64).mean(0), atol=1e-14)
    # count 0: output 0, lse -inf
    out, lse = oracle.decode(q, kc, vc, np.array([[0, 3]], np.int32))
    assert np.all(out[0, :2] == 0) and np.all(np.isneginf(lse[0, :2]))
    # MQA (one KV head) reduces to textbook attention per head
    out, _ = oracle.decode(q, kc[:, :1], vc[:, :1], np.array([[cap]], np.int32))
    for h in range(n_h):
        y = kc[0, 0].astype(np.float64) @ q[0, h].astype(np.float64) / math.sqrt(d)
        p = np.exp(y - y.max())
        assert np.allclose(out[0, h], (p / p.sum()) @ vc[0, 0].astype(np.float64), atol=1e-14)


# ----------------------------------------------------------------------------------
# Speculative retrieval with fine-grained correction (FreeKV technical summary 2.A)
# ----------------------------------------------------------------------------------
def test_query_similarity_closed_forms():
    d = 64
    base = np.zeros((1, 8, d), np.float32)
    prev = np.zeros((1, 8, d), np.float32)
    rng = np.random.default_rng(11)
    x = rng.standard_normal(d).astype(np.float32)
    base[0, 0], prev[0, 0] = x, x                        # identical -> 1
    base[0, 1], prev[0, 1] = x, -x                       # opposite -> -1
    base[0, 2, 0], prev[0, 2, 1] = 1.0, 1.0              # orthogonal -> 0
    base[0, 3, :2], prev[0, 3, :2] = (3.0, 4.0), (4.0, 3.0)   # 24 / 25
    base[0, 4], prev[0, 4] = x, np.float32(4.0) * x      # scale invariant -> 1
    prev[0, 5] = x                                       # zero query -> 0 by convention
    base[0, 6, :3], prev[0, 6, :3] = (1.0, 0.0, 0.0), (1.0, 1.0, 0.0)   # 45 degrees
    base[0, 7, :2], prev[0, 7, :2] = (1.0, 2.0), (-2.0, 1.0)            # orthogonal, not axis-aligned
    cos, _ = oracle.query_similarity(base, prev, 2, 0.5)
    want = [1.0, -1.0, 0.0, 24.0 / 25.0, 1.0, 0.0, 1.0 / math.sqrt(2.0), 0.0]
    assert np.allclose(cos[0], want, rtol=0, atol=1e-12)


def test_query_similarity_matches_distance_identity():
    # |a - b|^2 = |a|^2 + |b|^2 - 2 |a| |b| cos: an independent route to the cosine,
    # and invariance under a common rotation of both queries
    rng = np.random.default_rng(12)
    a = rng.standard_normal((3, 16, 128)).astype(np.float32)
    b = (0.9 * a + 0.5 * rng.standard_normal((3, 16, 128))).astype(np.float32)
    cos, _ = oracle.query_similarity(a, b, 4, 0.0)
    A, B = a.astype(np.float64), b.astype(np.float64)
    na, nb = np.linalg.norm(A, axis=2), np.linalg.norm(B, axis=2)
    dist2 = np.sum((A - B) ** 2, axis=2)
    assert np.allclose(dist2, na ** 2 + nb ** 2 - 2 * na * nb * cos, rtol=1e-10, atol=1e-9)
    Q, _ = np.linalg.qr(rng.standard_normal((128, 128)))
    cos_rot, _ = oracle.query_similarity((A @ Q).astype(np.float32), (B @ Q).astype(np.float32), 4, 0.0)
    assert np.allclose(cos_rot, cos, atol=2e-6)


def test_query_similarity_correction_flags():
    # one drifted query head marks exactly its own KV head (h // r), below tau only
    rng = np.random.default_rng(13)
    B, n_h, n_kv, d = 2, 8, 2, 32
    q = rng.standard_normal((B, n_h, d)).astype(np.float32)
    prev = q.copy()
    prev[1, 5] = rng.standard_normal(d).astype(np.float32)   # sequence 1, head 5 -> KV head 1
    cos, ref = oracle.query_similarity(q, prev, n_kv, 0.9)
    assert cos[1, 5] < 0.9 and np.allclose(np.delete(cos.ravel(), 1 * n_h + 5), 1.0)
    assert ref.tolist() == [[0, 0], [0, 1]]
    _, none = oracle.query_similarity(q, prev, n_kv, -1.0)   # cos >= -1: nothing is below -1
    assert not none.any()
    _, everything = oracle.query_similarity(q, prev, n_kv, 1.5)
    assert everything.all()
    # the flag needs a strict drop below tau: cos == tau is kept
    c = float(cos[1, 5])
    _, at = oracle.query_similarity(q, prev, n_kv, c)
    assert at[1, 1] == 0


def _spec_case(seed, S=200, n_h=4, n_kv=2, d=16, k=12, n_keep=4):
    rng = np.random.default_rng(seed)
    kk = rng.standard_normal((1, n_kv, S, d)).astype(np.float32)
    vv = rng.standard_normal((1, n_kv, S, d)).astype(np.float32)
    q0 = rng.standard_normal((1, n_h, d)).astype(np.float32)
    q1 = rng.standard_normal((1, n_h, d)).astype(np.float32)   # unrelated: selections differ
    return kk, vv, q0, q1, dict(seq_lens=np.array([S], np.int32), k_budget=k, n_keep=n_keep, pool=1)


def test_speculative_step_uses_previous_selection_unless_corrected():
    kk, vv, q0, q1, kw = _spec_case(21)
    first = oracle.speculative_step(q0, None, kk, vv, None, tau=0.9, **kw)
    assert first["refresh"].all()                                  # the first step selects fresh
    assert np.array_equal(first["idx"], first["next_sel"][0])
    prev = first["next_sel"]
    fresh = oracle.speculative_step(q1, q0, kk, vv, prev, tau=2.0, **kw)     # tau > 1: correct all
    stale = oracle.speculative_step(q1, q0, kk, vv, prev, tau=-2.0, **kw)    # tau < -1: reuse all
    assert fresh["refresh"].all() and not stale["refresh"].any()
    assert np.array_equal(fresh["idx"], fresh["next_sel"][0])
    assert np.array_equal(stale["idx"], prev[0]) and np.array_equal(stale["count"], prev[1])
    assert not np.array_equal(fresh["idx"], stale["idx"])
    # reused or not, the next step always gets the selection made with q1
    assert np.array_equal(stale["next_sel"][0], fresh["next_sel"][0])
    # attention over the reused subset equals attention over the full cache restricted
    # to prev's kept tokens (torch, float64): the output follows the selection used
    for res, idx in ((stale, prev[0]), (fresh, fresh["next_sel"][0])):
        q = torch.from_numpy(q1).double()
        for g in range(kk.shape[1]):
            keep = torch.zeros(kk.shape[2], dtype=torch.bool)
            keep[torch.from_numpy(idx[0, g][idx[0, g] >= 0].astype(np.int64))] = True
            kf = torch.from_numpy(kk[0, g]).double()[None, None]
            vf = torch.from_numpy(vv[0, g]).double()[None, None]
            for h in range(g * 2, g * 2 + 2):
                ref = F.scaled_dot_product_attention(q[0, h][None, None, None], kf, vf,
                                                     attn_mask=keep[None, None, None])
                assert np.allclose(res["out"][0, h], ref[0, 0, 0].numpy(), atol=1e-12)


def test_speculative_step_corrects_per_kv_head():
    kk, vv, q0, q1, kw = _spec_case(22)
    prev = oracle.speculative_step(q0, None, kk, vv, None, tau=0.9, **kw)["next_sel"]
    mixed = q0.copy()
    mixed[0, 3] = q1[0, 3]                           # only query head 3 (KV head 1) drifts
    res = oracle.speculative_step(mixed, q0, kk, vv, prev, tau=0.9, **kw)
    assert res["refresh"].tolist() == [[0, 1]]
    assert np.array_equal(res["idx"][0, 0], prev[0][0, 0])
    assert np.array_equal(res["idx"][0, 1], res["next_sel"][0][0, 1])
    # an explicit decision overrides the similarity
    forced = oracle.speculative_step(mixed, q0, kk, vv, prev, tau=0.9, refresh=np.array([[1, 0]]), **kw)
    assert np.array_equal(forced["idx"][0, 0], forced["next_sel"][0][0, 0])
    assert np.array_equal(forced["idx"][0, 1], prev[0][0, 1])


# ----------------------------------------------------------------------------------
# Budgets that differ per unit (Tutorial, "Compresser un cache existant": PyramidKV)
# ----------------------------------------------------------------------------------
def test_select_per_unit_budgets_bruteforce():
    rng = np.random.default_rng(41)
    B, H, S, n_keep = 2, 3, 11, 2
    sc = (rng.integers(0, 6, (B, H, S)) / 5.0).astype(np.float32)      # many exact ties
    sl = np.array([S, 8], np.int32)
    ku = np.array([[0, 3, 9], [2, 5, 1]], np.int32)                      # 9 > C for both sequences
    k = 6
    idx, cnt = oracle.select_topk(sc, k, n_keep, seq_lens=sl, k_per_unit=ku)
    for b in range(B):
        S_b = int(sl[b])
        C = S_b - n_keep
        for h in range(H):
            k_eff = min(int(ku[b, h]), k, C)
            # brute force: the lexicographically best k_eff-subset under (score desc, index asc)
            best = None
            for sub in itertools.combinations(range(C), k_eff):
                key = sorted(((-float(sc[b, h, t]), t) for t in sub))
                if best is None or key < best[0]:
                    best = (key, sub)
            want = sorted(best[1]) + list(range(C, S_b))
            n = int(cnt[b, h])
            assert n == len(want) and idx[b, h, :n].tolist() == want
            assert np.all(idx[b, h, n:] == -1)
    # a uniform budget array is the scalar budget
    u_idx, u_cnt = oracle.select_topk(sc, 4, n_keep, seq_lens=sl, k_per_unit=np.full((B, H), 4, np.int32))
    s_idx, s_cnt = oracle.select_topk(sc, 4, n_keep, seq_lens=sl)
    assert np.array_equal(u_idx, s_idx) and np.array_equal(u_cnt, s_cnt)


# ----------------------------------------------------------------------------------
# Role-based retention: core tokens always kept, the budget over scratch (CASK)
# ----------------------------------------------------------------------------------
def test_select_core_bruteforce_and_special_cases():
    rng = np.random.default_rng(51)
    B, H, S, n_keep = 2, 2, 12, 2
    sc = (rng.integers(0, 5, (B, H, S)) / 4.0).astype(np.float32)       # exact ties
    core = (rng.random((B, S)) < 0.3).astype(np.uint8)
    core[0, S - 1] = 1                                                    # a core token inside the window
    sl = np.array([S, 9], np.int32)
    for k in (0, 2, 4, 20):
        idx, cnt = oracle.select_core(sc, core, k, n_keep, seq_lens=sl)
        for b in range(B):
            S_b = int(sl[b])
            C = S_b - n_keep
            cores = [t for t in range(C) if core[b, t]]
            scratch = [t for t in range(C) if not core[b, t]]
            for h in range(H):
                k_eff = min(k, len(scratch))
                best = None
                for sub in itertools.combinations(scratch, k_eff):
                    key = sorted((-float(sc[b, h, t]), t) for t in sub)
                    if best is None or key < best[0]:
                        best = (key, sub)
                want = sorted(set(best[1]) | set(cores)) + list(range(C, S_b))
                n = int(cnt[b, h])
                assert n == len(want) and idx[b, h, :n].tolist() == want, (k, b, h)
                assert np.all(idx[b, h, n:] == -1)
    # no core token: the plain selection; every token core: everything kept
    none = np.zeros((B, S), np.uint8)
    c_idx, c_cnt = oracle.select_core(sc, none, 3, n_keep, seq_lens=sl, core_cap=0)
    p_idx, p_cnt = oracle.select_topk(sc, 3, n_keep, seq_lens=sl)
    assert np.array_equal(c_idx, p_idx) and np.array_equal(c_cnt, p_cnt)
    a_idx, a_cnt = oracle.select_core(sc, np.ones((B, S), np.uint8), 3, n_keep, seq_lens=sl)
    for b in range(B):
        assert a_cnt[0 if b == 0 else 1, 0] == sl[b] and a_idx[b, 0, :sl[b]].tolist() == list(range(sl[b]))


def test_select_core_over_capacity():
    """Fewer output slots than the rule needs (core_cap < |Core|): the unit keeps the
    first k + core_cap candidates of "core by index, then scratch by score".  Pinned
    through the plain selection (itself brute-forced above): with room for every core
    token the scratch tokens are the plain top-k over the scratch tokens alone with
    the budget that is left; without it, the lowest-indexed core tokens."""
    rng = np.random.default_rng(52)
    B, H, S, n_keep = 1, 3, 300, 6
    sc = (rng.integers(0, 40, (B, H, S)) / 39.0).astype(np.float32)
    core = np.zeros((B, S), np.uint8)
    core[0, rng.choice(S - n_keep, 50, replace=False)] = 1
    cores = np.nonzero(core[0, :S - n_keep])[0]
    window = list(range(S - n_keep, S))
    big_i, big_c = oracle.select_core(sc, core, 30, n_keep, core_cap=50)
    for k, core_cap in ((30, 50), (30, 200), (30, 45), (30, 20), (30, 0), (10, 30), (0, 7)):
        idx, cnt = oracle.select_core(sc, core, k, n_keep, core_cap=core_cap)
        assert idx.shape == (B, H, k + core_cap + n_keep)
        room = k + core_cap
        for h in range(H):
            n = int(cnt[0, h])
            got = idx[0, h, :n].tolist()
            assert np.all(idx[0, h, n:] == -1) and n <= k + core_cap + n_keep
            if core_cap >= cores.size:
                # the rule itself: as with ample room
                if k == 30:
                    assert got == big_i[0, h, :big_c[0, h]].tolist()
            if cores.size <= room:
                left = min(k, room - cores.size)
                masked = sc.copy()
                masked[0, :, cores] = -1.0                        # below every scratch score
                pi, pc = oracle.select_topk(masked[:, h:h + 1], left, n_keep)
                want = sorted(set(cores.tolist()) | set(pi[0, 0, :left].tolist())) + window
            else:
                want = sorted(cores[:room].tolist()) + window
            assert got == want, (k, core_cap, h)


# ----------------------------------------------------------------------------------
# Landmark-guided block selection (xKV section 2.3, ShadowKV-style landmarks)
# ----------------------------------------------------------------------------------
def test_block_landmarks_closed_forms():
    B, n_kv, S, d, blk = 2, 2, 37, 4, 8
    a = np.array([1.0, -2.0, 0.5, 3.0], np.float32)
    t = np.arange(S, dtype=np.float32)
    k = np.broadcast_to(t[None, None, :, None] * a, (B, n_kv, S, d)).astype(np.float32).copy()
    sl = np.array([S, 20], np.int32)
    lm = oracle.block_landmarks(k, blk, seq_lens=sl)
    assert lm.shape == (B, n_kv, 5, d)
    for b in range(B):
        S_b = int(sl[b])
        for j in range(5):
            lo, hi = j * blk, min(j * blk + blk, S_b)
            want = ((lo + hi - 1) / 2.0) * a if hi > lo else np.zeros(d)   # mean of an arithmetic run
            assert np.allclose(lm[b, 0, j], want, atol=1e-6), (b, j)
    # the landmarks, weighted by their block sizes, add up to the sum of the keys
    rng = np.random.default_rng(61)
    k2 = rng.standard_normal((1, 1, 45, 8)).astype(np.float32)
    lm2 = oracle.block_landmarks(k2, 7)
    sizes = np.array([7] * 6 + [3], np.float64)
    assert np.allclose((lm2[0, 0].astype(np.float64) * sizes[:, None]).sum(0), k2[0, 0].astype(np.float64).sum(0),
                       atol=1e-5)


def test_block_scores_and_expansion():
    rng = np.random.default_rng(62)
    B, n_h, n_kv, S, d, blk, n_keep = 2, 4, 2, 50, 8, 4, 6
    lm = rng.standard_normal((B, n_kv, (S + blk - 1) // blk, d)).astype(np.float32)
    q = rng.standard_normal((B, n_h, d)).astype(np.float32)
    sl = np.array([S, 17], np.int32)
    sc, cand = oracle.block_scores(q, lm, blk, n_keep, S, seq_lens=sl, scale=0.5)
    assert cand.tolist() == [(S - n_keep) // blk, (17 - n_keep) // blk]
    # linear in the queries; identical group queries give r times one head's logit
    sc2, _ = oracle.block_scores(2.0 * q, lm, blk, n_keep, S, seq_lens=sl, scale=0.5)
    assert np.allclose(sc2, 2.0 * sc, rtol=1e-6, atol=1e-6)
    qs = np.repeat(q[:, ::2], 2, axis=1)                          # heads 2g and 2g+1 equal
    sc3, _ = oracle.block_scores(qs, lm, blk, n_keep, S, seq_lens=sl, scale=0.5)
    j = 3
    assert np.isclose(sc3[0, 1, j], 2 * 0.5 * float(np.dot(q[0, 2].astype(np.float64), lm[0, 1, j])), rtol=1e-6)
    assert np.all(sc[1, :, cand[1]:] == 0)
    # expansion: blocks 1 and 4 of unit (0, 0), block 0 of unit (1, 1); the tail follows
    idx_blk = np.full((B, n_kv, 3), -1, np.int32)
    cnt_blk = np.array([[2, 0], [0, 1]], np.int32)
    idx_blk[0, 0, :2] = [1, 4]
    idx_blk[1, 1, :1] = [0]
    idx, cnt = oracle.expand_blocks(idx_blk, cnt_blk, blk, n_keep, S, 30, seq_lens=sl)
    tail0 = (S - n_keep) // blk * blk
    assert idx[0, 0, :cnt[0, 0]].tolist() == [4, 5, 6, 7, 16, 17, 18, 19] + list(range(tail0, S))
    assert idx[0, 1, :cnt[0, 1]].tolist() == list(range(tail0, S))
    assert idx[1, 1, :cnt[1, 1]].tolist() == [0, 1, 2, 3] + list(range(8, 17))
    assert np.all(idx[1, 1, cnt[1, 1]:] == -1)


def test_block_retrieval_special_cases():
    rng = np.random.default_rng(63)
    B, n_h, n_kv, S, d, n_keep = 1, 4, 2, 40, 16, 4
    k = rng.standard_normal((B, n_kv, S, d)).astype(np.float32)
    v = rng.standard_normal((B, n_kv, S, d)).astype(np.float32)
    q = rng.standard_normal((B, n_h, d)).astype(np.float32)
    # block size 1: the landmark is the key, so the kept tokens are the top k of the
    # group's logit sum (torch float64 einsum) plus the trailing n_keep
    res = oracle.block_retrieval(q, k, v, 7, 1, n_keep)
    logit = torch.einsum("ghd,gtd->gt", torch.from_numpy(q[0]).double().view(n_kv, 2, d),
                         torch.from_numpy(k[0]).double()) / math.sqrt(d)
    for g in range(n_kv):
        order = sorted(range(S - n_keep), key=lambda t: (-float(logit[g, t]), t))[:7]
        want = sorted(order) + list(range(S - n_keep, S))
        assert res["idx"][0, g, :res["count"][0, g]].tolist() == want
    # every block kept: attention over the whole cache (torch scaled_dot_product_attention)
    full = oracle.block_retrieval(q, k, v, 100, 8, n_keep)
    assert np.all(full["count"] == S)
    for h in range(n_h):
        g = h // 2
        ref = F.scaled_dot_product_attention(torch.from_numpy(q[0, h]).double()[None, None, None],
                                             torch.from_numpy(k[0, g]).double()[None, None],
                                             torch.from_numpy(v[0, g]).double()[None, None])
        assert np.allclose(full["out"][0, h], ref[0, 0, 0].numpy(), atol=1e-12)
