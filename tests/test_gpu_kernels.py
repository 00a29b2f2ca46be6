"""Kernel-level GPU parity: each HIP kernel against the CPU oracle on the same seeded
inputs, at sizes that span several tiles and a ragged tail, plus edge cases."""
import sys

import numpy as np
import pytest
import torch

import oracle
from sparse_decode_amd import kvc, synth
from _parity import (assert_decode_close, assert_scores_close, check_selection, host)

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    kvc.lib()
    yield


def _say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def _randn(shape, seed, dtype=torch.bfloat16):
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    return torch.randn(shape, generator=g, device=DEV, dtype=torch.float32).to(dtype).contiguous()


# ===================================================================================== gather

@pytest.mark.parametrize("dtype,d,heads,idx_heads,s_max,cap", [
    (torch.bfloat16, 128, 8, 8, 3000, 700),
    (torch.float32, 64, 2, 2, 512, 80),
    (torch.bfloat16, 64, 4, 1, 1000, 300),
    (torch.bfloat16, 4096, 1, 1, 2000, 600),       # hidden-state rows of 8 KiB
])
def test_gather_bitexact(dtype, d, heads, idx_heads, s_max, cap):
    _say("gather", dtype, d, heads, idx_heads, s_max, cap)
    B = 3
    rng = np.random.default_rng(7)
    src0 = _randn((B, heads, s_max, d), 1, dtype)
    src1 = _randn((B, heads, s_max, d), 2, dtype)
    idx = np.full((B, idx_heads, cap), -1, np.int32)
    count = np.zeros((B, idx_heads), np.int32)
    counts = [cap, 0, 1, cap // 2, 37]
    for b in range(B):
        for h in range(idx_heads):
            n = counts[(b * idx_heads + h) % len(counts)]
            idx[b, h, :n] = np.sort(rng.choice(s_max, n, replace=False))
            count[b, h] = n
    idx[0, 0, 5] = s_max + 3          # out of range: copies nothing, pos -1
    src_pos = rng.permutation(10 * s_max)[: B * s_max].reshape(B, s_max).astype(np.int32)
    sentinel = torch.full((B, heads, cap, d), 7.0, dtype=dtype, device=DEV)
    d0, d1, pos = kvc.gather_compact(src0, torch.from_numpy(idx).to(DEV), torch.from_numpy(count).to(DEV),
                                     src1=src1, src_pos=torch.from_numpy(src_pos).to(DEV),
                                     dst0=sentinel.clone(), dst1=sentinel.clone())
    torch.cuda.synchronize()
    for src, dst in ((src0, d0), (src1, d1)):
        s_np = src.view(torch.int16).cpu().numpy() if dtype == torch.bfloat16 else src.view(torch.int32).cpu().numpy()
        base = sentinel.view(torch.int16 if dtype == torch.bfloat16 else torch.int32).cpu().numpy()
        src_b = np.broadcast_to(s_np, s_np.shape)
        if idx_heads == 1:
            idx_full = np.repeat(idx, heads, axis=1)
            cnt_full = np.repeat(count, heads, axis=1)
        else:
            idx_full, cnt_full = idx, count
        ref, ref_pos = oracle.gather(src_b, np.where((idx_full >= 0) & (idx_full < s_max), idx_full, 0), cnt_full,
                                     src_pos=src_pos, dst=base)
        # the out-of-range index leaves its row untouched and gets pos -1
        ref[0, :heads if idx_heads == 1 else 1, 5] = base[0, :heads if idx_heads == 1 else 1, 5]
        ref_pos[0, :heads if idx_heads == 1 else 1, 5] = -1
        got = dst.view(torch.int16 if dtype == torch.bfloat16 else torch.int32).cpu().numpy()
        assert np.array_equal(got, ref)
        assert np.array_equal(host(pos), ref_pos)


# ===================================================================================== decode

@pytest.mark.parametrize("dtype,d,n_h,n_kv,cap", [
    (torch.bfloat16, 128, 32, 8, 2080),
    (torch.bfloat16, 128, 32, 32, 1056),     # MHA
    (torch.bfloat16, 128, 32, 1, 300),       # MQA: 32 heads per KV head, 4 head chunks
    (torch.bfloat16, 64, 12, 4, 517),        # group of 3
    (torch.float32, 64, 4, 2, 80),
    (torch.float32, 128, 8, 2, 999),
    (torch.bfloat16, 128, 4, 4, 4096),       # 64 splits of one head folded by the last arrival
    (torch.bfloat16, 128, 32, 4, 4096),      # 64 splits of 8 heads: the merge kernel folds
    (torch.bfloat16, 128, 8, 1, 9000),       # 141 splits: the merge kernel folds
    (torch.float32, 64, 8, 1, 9000),
])
def test_decode_vs_oracle(dtype, d, n_h, n_kv, cap):
    _say("decode", dtype, d, n_h, n_kv, cap)
    B = 2
    plan = kvc.decode_attn_plan(kvc.make_dims(B, 1, n_h, n_kv, d, kvc.KVC_BF16), cap)
    assert plan["n_splits"] * plan["split_tokens"] >= cap, plan
    q = _randn((B, n_h, d), 11, dtype)
    kc = _randn((B, n_kv, cap, d), 12, dtype)
    vc = _randn((B, n_kv, cap, d), 13, dtype)
    row0 = [cap, 1] + [cap - 7 * i for i in range(max(0, n_kv - 2))]
    row1 = [0] + [max(0, cap // (i + 1)) for i in range(max(0, n_kv - 1))]
    cnt = np.array([row0[:n_kv], row1[:n_kv]], np.int32)
    out, lse = kvc.decode_attn(q, kc, vc, torch.from_numpy(cnt).to(DEV))
    torch.cuda.synchronize()
    ref, ref_lse = oracle.decode(host(q), host(kc), host(vc), cnt)
    bf16 = dtype == torch.bfloat16
    assert_decode_close(out, ref, bf16)
    g = host(lse)
    fin = np.isfinite(ref_lse)
    assert np.array_equal(np.isfinite(g), fin)
    assert np.allclose(g[fin], ref_lse[fin], rtol=1e-5, atol=1e-5)
    assert np.all(host(out)[~fin] == 0)
    # bit-reproducible
    out2, lse2 = kvc.decode_attn(q, kc, vc, torch.from_numpy(cnt).to(DEV))
    assert torch.equal(out, out2) and torch.equal(lse, lse2)


def test_decode_workspace_reuse():
    # one zero-filled workspace, sized for the largest call, serves calls of other
    # batches, heads, caps and counts, with and without the fused split fold: every call
    # leaves the arrival counters (the first 64 KiB) at zero, and each result equals
    # that of a fresh workspace
    _say("decode ws reuse")
    d = 128
    calls = [(2, 32, 8, 5000, 1), (2, 32, 8, 2080, 2), (2, 8, 1, 9000, 3), (4, 32, 32, 1056, 4),
             (2, 32, 8, 64, 5), (1, 8, 1, 9000, 6), (2, 32, 8, 5000, 7), (2, 32, 8, 1, 8)]
    need = max(kvc.decode_attn_workspace(kvc.make_dims(B, 1, nh, nkv, d, kvc.KVC_BF16), cap)
               for B, nh, nkv, cap, _ in calls)
    ws = torch.zeros(need, dtype=torch.uint8, device=DEV)
    fused = set()
    for B, n_h, n_kv, cap, seed in calls:
        fused.add(kvc.decode_attn_plan(kvc.make_dims(B, 1, n_h, n_kv, d, kvc.KVC_BF16), cap)["fused"])
        q = _randn((B, n_h, d), 20 + seed)
        kc = _randn((B, n_kv, cap, d), 30 + seed)
        vc = _randn((B, n_kv, cap, d), 40 + seed)
        cnt = np.full((B, n_kv), cap, np.int32)
        cnt[0, min(1, n_kv - 1)] = 0
        cnt[B - 1, n_kv - 1] = max(0, cap // 3)
        cnt_d = torch.from_numpy(cnt).to(DEV)
        out, lse = kvc.decode_attn(q, kc, vc, cnt_d, ws=ws)
        out_f, lse_f = kvc.decode_attn(q, kc, vc, cnt_d)      # a fresh zero-filled workspace
        torch.cuda.synchronize()
        assert int(ws[:65536].count_nonzero()) == 0
        assert torch.equal(out, out_f) and torch.equal(lse, lse_f)
        ref, ref_lse = oracle.decode(host(q), host(kc), host(vc), cnt)
        assert_decode_close(out, ref, True)
    assert fused == {True, False}


def test_decode_closed_forms():
    _say("decode closed forms")
    n_h, n_kv, cap, d = 8, 2, 64, 128
    q = _randn((1, n_h, d), 21)
    kc = _randn((1, n_kv, cap, d), 22)
    vc = _randn((1, n_kv, cap, d), 23)
    one = torch.tensor([[1, 1]], dtype=torch.int32, device=DEV)
    out, _ = kvc.decode_attn(q, kc, vc, one)
    # one token: the output is that V row, exactly (p = 1, bf16 round trip is exact)
    for h in range(n_h):
        assert torch.equal(out[0, h], vc[0, h // 4, 0])
    same = kc[:, :, :1].expand(1, n_kv, cap, d).contiguous()
    full = torch.tensor([[cap, cap]], dtype=torch.int32, device=DEV)
    out, _ = kvc.decode_attn(q, same, vc, full)
    mean = vc.float().mean(2)
    assert torch.allclose(out.float()[0, 0], mean[0, 0], atol=2e-2, rtol=1e-2)


# ===================================================================================== select

def _select_case(scores_np, seq_lens, k, n_keep, shared=False, ws=None):
    """Bit-exact against the oracle; shared over heads, the GPU selects on the head sum
    rounded to float and the oracle on the exact sum, so there the near-tie rule
    applies (and bit-exactness where the sums are exact in float)."""
    sc = torch.from_numpy(scores_np).to(DEV)
    idx, cnt = kvc.select_topk(sc, k, n_keep, seq_lens=seq_lens, shared_heads=shared, ws=ws)
    torch.cuda.synchronize()
    ri, rc = oracle.select_topk(scores_np, k, n_keep, seq_lens=seq_lens, shared_heads=shared)
    assert np.array_equal(host(cnt), rc)
    if shared:
        check_selection(idx, cnt, ri, rc, scores_np, seq_lens, k, n_keep, shared=True)
    else:
        assert np.array_equal(host(idx), ri)


@pytest.mark.parametrize("s_max", [100, 4096, 32768, 65536])
def test_select_bitexact_with_ties(s_max):
    _say("select ties", s_max)
    rng = np.random.default_rng(s_max)
    B, H = 2, 8
    sc = (rng.integers(0, 50, (B, H, s_max)) / 37.0).astype(np.float32)   # many exact ties
    sl = np.array([s_max, max(1, s_max * 2 // 3 + 5)], np.int32)
    for k in (1, 17, s_max // 16, s_max // 2, s_max):
        for n_keep in (0, 32):
            if k + n_keep < 1:
                continue
            _select_case(sc, sl, k, n_keep)


@pytest.mark.parametrize("s_max", [4096, 16000, 131072])
def test_select_bitexact_continuous(s_max):
    _say("select continuous", s_max)
    rng = np.random.default_rng(3)
    sc = rng.random((1, 8, s_max)).astype(np.float32) ** 4
    sc[0, 0, 1000:1100] = 0.5                     # a tie wall
    sc[0, 1] = 0.25                               # all equal
    sc[0, 2, ::7] = 0.0
    # window-score-like: one narrow mode (most keys share the top 11 key bits) plus a
    # few large outliers
    sc[0, 3] = (0.004 * (1.0 + 0.12 * rng.standard_normal(s_max))).astype(np.float32)
    sc[0, 3, rng.choice(s_max, s_max // 100, replace=False)] = 0.5
    sc[0, 4] = np.float32(0.004) + np.float32(2 ** -31) * rng.integers(0, 64, s_max).astype(np.float32)
    # max-pooled (window 7) scores with planted heavy hitters of one value: runs of equal
    # keys inside a thread's slots and the same key in many threads at once
    x = rng.random(s_max + 6).astype(np.float32) ** 8
    x[rng.choice(s_max, max(1, s_max // 50), replace=False) + 3] = 0.75
    sc[0, 5] = np.lib.stride_tricks.sliding_window_view(x, 7).max(axis=1)
    sl = np.array([s_max], np.int32)
    for k in (1311, 2048, 7):
        _select_case(sc, sl, k, 32)


@pytest.mark.parametrize("s_max", [3001, 4096, 16000, 32768, 70000])
def test_select_many_units(s_max):
    # many units: every unit's candidates go to one work-group when they fit
    # (s_max - n_keep <= 32768); past that, 128 units of 70000 tokens take the chunked
    # kernels with 8192-key chunks.  Rows of a multiple of 4 floats and not, ties,
    # ragged lengths, per-unit budgets and a unit mask.
    _say("select many units", s_max)
    rng = np.random.default_rng(s_max + 1)
    B, H = (32, 8) if s_max <= 32768 else (16, 8)
    sc = rng.random((B, H, s_max)).astype(np.float32) ** 4
    sc[::3] = (rng.integers(0, 60, (sc[::3].shape)) / 59.0).astype(np.float32)      # many exact ties
    sc[1, 2] = 0.25                                                                   # all equal
    sl = rng.integers(1, s_max + 1, B).astype(np.int32)
    sl[0], sl[1], sl[2] = s_max, 0, 20
    for k, n_keep in ((1, 0), (s_max // 16, 32), (s_max // 2, 8)):
        _select_case(sc, sl, k, n_keep)
    k, n_keep = s_max // 10, 32
    ku = rng.integers(0, k + 1, (B, H)).astype(np.int32)
    ku[0, 0], ku[3, 3] = k + 7, -1
    sc_t = torch.from_numpy(sc).to(DEV)
    idx, cnt = kvc.select_topk(sc_t, k, n_keep, seq_lens=sl, k_per_unit=torch.from_numpy(ku).to(DEV))
    ri, rc = oracle.select_topk(sc, k, n_keep, seq_lens=sl, k_per_unit=ku)
    assert np.array_equal(host(idx), ri) and np.array_equal(host(cnt), rc)
    mask = torch.from_numpy(rng.integers(0, 2, (B, H)).astype(np.int32)).to(DEV)
    idx2 = torch.full_like(idx, -5)
    cnt2 = torch.full_like(cnt, -5)
    kvc.select_topk(sc_t, k, n_keep, seq_lens=sl, k_per_unit=torch.from_numpy(ku).to(DEV), idx=idx2, count=cnt2,
                    unit_mask=mask)
    torch.cuda.synchronize()
    on = mask.bool()
    assert torch.equal(idx2[on], idx[on]) and torch.equal(cnt2[on], cnt[on])
    assert bool((idx2[~on] == -5).all()) and bool((cnt2[~on] == -5).all())


def test_select_shared_heads_many_sequences():
    # one selection per sequence for 128 sequences (the head-summed scores take the
    # one-work-group-per-unit kernel)
    _say("select shared many")
    rng = np.random.default_rng(21)
    B, H, s_max = 128, 4, 5000
    sc = rng.random((B, H, s_max)).astype(np.float32) * 1e-3
    sc[5] = 1e-3
    sl = rng.integers(0, s_max + 1, B).astype(np.int32)
    _select_case(sc, sl, 1000, 32, shared=True)


def test_select_shared_heads_and_degenerate():
    _say("select shared")
    rng = np.random.default_rng(5)
    B, H, s_max = 2, 32, 65536
    sc = rng.random((B, H, s_max)).astype(np.float32) * 1e-3
    _select_case(sc, np.array([s_max, s_max], np.int32), 13108, 32, shared=True)
    # multiples of 2^-18 below 1 over 32 heads add exactly in float: bit-exact
    dy = (rng.integers(0, 1 << 18, (B, H, s_max)) / float(1 << 18)).astype(np.float32)
    idx, cnt = kvc.select_topk(torch.from_numpy(dy).to(DEV), 13108, 32, shared_heads=True)
    ri, rc = oracle.select_topk(dy, 13108, 32, shared_heads=True)
    assert np.array_equal(host(idx), ri) and np.array_equal(host(cnt), rc)
    small = rng.random((3, 2, 64)).astype(np.float32)
    _select_case(small, np.array([0, 5, 64], np.int32), 10, 8)     # S_b = 0, S_b < n_keep
    _select_case(small, np.array([64, 64, 64], np.int32), 0, 8)    # k = 0
    neg = (rng.standard_normal((1, 2, 300))).astype(np.float32)
    neg[0, 0, :10] = -0.0
    neg[0, 0, 10:20] = 0.0
    _select_case(neg, np.array([300], np.int32), 40, 4)            # signed scores, -0.0 == +0.0


def test_select_workspace_reuse_across_shapes():
    # one zero-filled workspace serves a run of calls with the same batch, n_kv and
    # flags but other budgets, windows and lengths: each call must leave it ready
    _say("select ws reuse")
    rng = np.random.default_rng(11)
    s_max = 20000
    sc = (0.004 * (1.0 + 0.12 * rng.standard_normal((4, 8, s_max)))).astype(np.float32)
    sc[:, :, ::97] = 0.5
    for shared in (False, True):
        dims = kvc.make_dims(4, s_max, 8, 8, 128, kvc.KVC_F32)
        flags = kvc.KVC_SELECT_SHARED_HEADS if shared else 0
        ws = torch.zeros(kvc.select_topk_workspace(dims, 1, 0, flags), dtype=torch.uint8, device=DEV)
        for k, n_keep, lens in [(1500, 32, [20000, 7000, 20000, 1]),
                                (10, 0, [20000, 20000, 20000, 20000]),
                                (19990, 16, [20000, 19000, 5, 12000]),     # k >= C for some units
                                (700, 8, [15000, 20000, 3000, 9000]),
                                (1500, 32, [20000, 7000, 20000, 1])]:
            _select_case(sc, np.array(lens, np.int32), k, n_keep, shared=shared, ws=ws)


# ===================================================================================== score

def _score_case(B, n_h, n_kv, d, s_max, w, seq_lens, wic=True, n_keep=None, pool=7, dtype=torch.bfloat16,
                generic=False, seed=0, planted=0):
    _say("score", B, n_h, n_kv, d, s_max, w, list(seq_lens), wic, pool, dtype, "generic" if generic else "mfma")
    q = _randn((B, n_h, w, d), 100 + seed, dtype)
    k = _randn((B, n_kv, s_max, d), 200 + seed, dtype)
    if planted:
        rng = np.random.default_rng(seed)
        pos = torch.from_numpy(rng.choice(max(1, s_max - w), planted, replace=False)).to(DEV)
        u = torch.from_numpy(rng.standard_normal((n_kv, d))).float().to(DEV)
        u = 4 * np.sqrt(d) * u / u.norm(dim=1, keepdim=True)
        k[:, :, pos, :] = u[None, :, None, :].to(dtype)
    n_keep = w if n_keep is None else n_keep
    raw, pooled = kvc.score_window(q, k, w, seq_lens=seq_lens, window_in_cache=wic, n_keep=n_keep, pool=pool,
                                   generic=generic)
    torch.cuda.synchronize()
    rraw, rpooled = oracle.score_window(host(q), host(k), w, seq_lens=seq_lens, window_in_cache=wic,
                                        n_keep=n_keep, pool=pool)
    assert_scores_close(raw, rraw, "raw")
    assert_scores_close(pooled, rpooled, "pooled")
    # pooling is exact given the raw scores the GPU produced
    _, pooled_from_gpu_raw = _pool_np(host(raw), seq_lens, n_keep, pool)
    assert np.array_equal(host(pooled), pooled_from_gpu_raw)
    raw2, pooled2 = kvc.score_window(q, k, w, seq_lens=seq_lens, window_in_cache=wic, n_keep=n_keep, pool=pool,
                                     generic=generic)
    assert torch.equal(raw, raw2) and torch.equal(pooled, pooled2)
    return q, k, raw, pooled, rpooled


def _pool_np(raw, seq_lens, n_keep, pool):
    out = np.zeros_like(raw)
    B, H, s_max = raw.shape
    h = pool // 2
    for b in range(B):
        S = int(seq_lens[b])
        C = max(0, S - n_keep)
        for g in range(H):
            r = raw[b, g]
            for t in range(S):
                out[b, g, t] = r[max(0, t - h):min(C - 1, t + h) + 1].max() if t < C else r[t]
    return raw, out


@pytest.mark.parametrize("generic", [False, True])
def test_score_gqa_ragged(generic):
    _score_case(2, 32, 8, 128, 2500, 32, np.array([2500, 1337], np.int32), generic=generic, planted=20)


def test_score_mqa():
    # one KV head for every query head: R = 8 * 16 = 128 rows (the MFMA path's largest
    # row count), and R = 16 * 16 = 256 with d_h = 64 (the generic path)
    _score_case(1, 8, 1, 128, 2100, 16, np.array([2100], np.int32), seed=5, planted=12)
    _score_case(2, 16, 1, 64, 900, 16, np.array([900, 517], np.int32), seed=6)


def test_score_mha_and_d64():
    _score_case(1, 4, 4, 128, 3001, 32, np.array([3001], np.int32), seed=1)           # R = 32
    _score_case(2, 8, 4, 64, 1500, 32, np.array([1500, 700], np.int32), seed=2)       # d = 64, R = 64
    _score_case(1, 6, 2, 128, 900, 16, np.array([900], np.int32), seed=3, pool=5)     # R = 48 (padded)


@pytest.mark.parametrize("generic", [False, True])
def test_score_decode_query_not_in_cache(generic):
    # one new query per head (w = 1) that sees every cached key; R = 4
    _score_case(3, 32, 8, 128, 4096, 1, np.array([4096, 2049, 3333], np.int32), wic=False, n_keep=32,
                generic=generic, seed=4)


def test_score_fp32_tiny_config():
    wl = synth.WORKLOADS[1]
    _score_case(1, wl.n_h, wl.n_kv, wl.d_h, wl.s_max, wl.w, np.array([wl.s_max], np.int32), pool=wl.pool,
                dtype=torch.float32, seed=5)


def test_score_short_sequences():
    # S_b < w (rows that see no key), S_b = 0, S_b = 1
    _score_case(4, 8, 2, 128, 256, 32, np.array([20, 0, 1, 256], np.int32), seed=6)
    _score_case(4, 8, 2, 128, 256, 32, np.array([20, 0, 1, 256], np.int32), seed=6, generic=True)


def test_score_row_padding_and_ragged_units():
    # many chunks per unit, a ragged last chunk, units shorter than a chunk and of zero length
    _score_case(4, 32, 8, 128, 20000, 32, np.array([20000, 19999, 257, 0], np.int32), seed=11, planted=30)
    # R = 80 (rows 80..127 of the row tile are padding), the query not in the cache
    _score_case(2, 10, 2, 128, 3000, 16, np.array([3000, 1000], np.int32), wic=False, seed=12)
    # R = 96, rows that see no key (S < w), S = 1
    _score_case(3, 12, 4, 128, 600, 32, np.array([20, 1, 600], np.int32), seed=13, pool=3)


def test_score_unit_mask():
    # units whose mask entry is 0 keep what raw/pooled held; the others match the full call
    B, n_h, n_kv, d, s_max, w = 2, 32, 8, 128, 5000, 32
    sl = np.array([5000, 3100], np.int32)
    _say("score unit mask", B, n_h, n_kv, d, s_max, w, list(sl))
    q = _randn((B, n_h, w, d), 300)
    k = _randn((B, n_kv, s_max, d), 301)
    full_raw, full_pooled = kvc.score_window(q, k, w, seq_lens=sl, n_keep=w, pool=7)
    mask = torch.from_numpy(np.random.default_rng(3).integers(0, 2, (B, n_kv)).astype(np.int32)).to(DEV)
    raw = torch.full((B, n_kv, s_max), -7.0, device=DEV)
    pooled = torch.full((B, n_kv, s_max), -9.0, device=DEV)
    kvc.score_window(q, k, w, seq_lens=sl, n_keep=w, pool=7, raw=raw, pooled=pooled, unit_mask=mask)
    torch.cuda.synchronize()
    on = mask.bool()
    assert torch.equal(raw[on], full_raw[on]) and torch.equal(pooled[on], full_pooled[on])
    assert bool((raw[~on] == -7.0).all()) and bool((pooled[~on] == -9.0).all())


def _plan(B, n_h, n_kv, d, s_max, w):
    return kvc.score_window_plan(kvc.make_dims(B, s_max, n_h, n_kv, d, kvc.KVC_BF16), w)


@pytest.mark.parametrize("s_max, d", [(16384, 128), (9000, 128), (5000, 64)])
def test_score_one_row_block_masked_call_matches_full(s_max, d):
    # one query per head over 16 ragged sequences (R = 4): a masked call cuts the
    # tokens into 256-token work-groups whatever the full call's chunks (2048 tokens
    # merged in the last work-group at 16384, 1024 tokens merged by a kernel at 9000,
    # 512 tokens at 5000 with d_h = 64), and its scores are the same bits, the row
    # partials being per 256-token block
    B, n_h, n_kv, w = 16, 32, 8, 1
    plan = _plan(B, n_h, n_kv, d, s_max, w)
    assert plan["rt"] == 1 and plan["chunk_tokens"] >= 512, plan
    rng = np.random.default_rng(7)
    sl = rng.integers(s_max // 4, s_max + 1, B).astype(np.int32)
    sl[0] = s_max
    sl[1] = 257
    _say("score one row block masked", B, n_h, n_kv, d, s_max, w, plan)
    q = _randn((B, n_h, w, d), 320)
    k = _randn((B, n_kv, s_max, d), 321)
    dims = kvc.make_dims(B, s_max, n_h, n_kv, d, kvc.KVC_BF16)
    ws = torch.zeros(kvc.score_window_workspace(dims, w), dtype=torch.uint8, device=DEV)
    args = dict(seq_lens=sl, window_in_cache=False, n_keep=32, pool=7, ws=ws)
    raw, pooled = kvc.score_window(q, k, w, **args)
    for frac in (0.05, 0.5):
        mask_np = (rng.random((B, n_kv)) < frac).astype(np.int32)
        mask_np[0, 0] = 1
        mask_np[1, 1] = 1
        mask = torch.from_numpy(mask_np).to(DEV)
        raw_m = torch.full((B, n_kv, s_max), -7.0, device=DEV)
        pooled_m = torch.full((B, n_kv, s_max), -9.0, device=DEV)
        kvc.score_window(q, k, w, raw=raw_m, pooled=pooled_m, unit_mask=mask, **args)
        torch.cuda.synchronize()
        on = mask.bool()
        assert torch.equal(raw_m[on], raw[on]) and torch.equal(pooled_m[on], pooled[on]), frac
        assert bool((raw_m[~on] == -7.0).all()) and bool((pooled_m[~on] == -9.0).all())
    raw2, pooled2 = kvc.score_window(q, k, w, **args)
    assert torch.equal(raw, raw2) and torch.equal(pooled, pooled2)
    # two sequences against the oracle
    idx = [0, 1]
    rraw, rpooled = oracle.score_window(host(q)[idx], host(k)[idx], w, seq_lens=sl[idx], window_in_cache=False,
                                        n_keep=32, pool=7)
    assert_scores_close(raw[idx], rraw, "raw")
    assert_scores_close(pooled[idx], rpooled, "pooled")


@pytest.mark.parametrize("shape", [(3, 16, 4, 2000, 1, False), (2, 8, 1, 1800, 16, True)])
def test_score_folded_merge_mask_and_reuse(shape):
    # at most 8 items per KV head, all work-groups resident: the last first-pass
    # work-group of a KV head merges its items' row statistics.  Its arrival counters
    # return to zero, so one workspace serves full, masked and repeated calls.
    # R = 4 (logits kept between the passes) and R = 128 (K read twice).
    B, n_h, n_kv, s_max, w, wic = shape
    d = 128
    plan = _plan(B, n_h, n_kv, d, s_max, w)
    assert plan["folded_merge"] and not plan["single_pass"] and plan["chunks_per_unit"] == 8, plan
    sl = np.array([s_max, 1500, 77][:B], np.int32)
    _say("score folded merge", B, n_h, n_kv, d, s_max, w, list(sl), plan)
    q = _randn((B, n_h, w, d), 310)
    k = _randn((B, n_kv, s_max, d), 311)
    dims = kvc.make_dims(B, s_max, n_h, n_kv, d, kvc.KVC_BF16)
    ws = torch.zeros(kvc.score_window_workspace(dims, w), dtype=torch.uint8, device=DEV)
    args = dict(seq_lens=sl, window_in_cache=wic, n_keep=32, pool=7, ws=ws)
    raw, pooled = kvc.score_window(q, k, w, **args)
    torch.cuda.synchronize()
    rraw, rpooled = oracle.score_window(host(q), host(k), w, seq_lens=sl, window_in_cache=wic, n_keep=32, pool=7)
    assert_scores_close(raw, rraw, "raw")
    assert_scores_close(pooled, rpooled, "pooled")
    mask = torch.from_numpy(np.random.default_rng(4).integers(0, 2, (B, n_kv)).astype(np.int32)).to(DEV)
    mask.view(-1)[0] = 1
    raw_m = torch.full((B, n_kv, s_max), -7.0, device=DEV)
    pooled_m = torch.full((B, n_kv, s_max), -9.0, device=DEV)
    kvc.score_window(q, k, w, raw=raw_m, pooled=pooled_m, unit_mask=mask, **args)
    raw2, pooled2 = kvc.score_window(q, k, w, **args)
    torch.cuda.synchronize()
    on = mask.bool()
    assert torch.equal(raw_m[on], raw[on]) and torch.equal(pooled_m[on], pooled[on])
    assert bool((raw_m[~on] == -7.0).all()) and bool((pooled_m[~on] == -9.0).all())
    assert torch.equal(raw, raw2) and torch.equal(pooled, pooled2)


def test_score_single_pass_shapes():
    # 17..32 rows per KV head read K once (1024-token items exchanging row statistics)
    cases = [
        (2, 8, 8, 128, 4097, 32, [4097, 2000], True, 0),        # MHA, R = 32, ragged tail item
        (3, 8, 8, 128, 1000, 32, [20, 0, 1000], True, 1),        # rows that see no key, an empty unit
        (2, 8, 8, 64, 3000, 32, [3000, 1024], True, 2),          # d_h = 64, a unit of exactly one item
        (2, 12, 4, 128, 2600, 8, [2600, 1025], True, 3),         # R = 24: rows 24..31 padding
        (2, 4, 4, 128, 9000, 32, [9000, 8193], True, 4),         # R = 32, 1024-token items and a tail
        (4, 16, 8, 128, 3000, 16, [3000, 1, 1023, 2049], False, 5),  # R = 32, queries not in the cache
    ]
    for B, n_h, n_kv, d, s_max, w, sl, wic, seed in cases:
        plan = _plan(B, n_h, n_kv, d, s_max, w)
        assert plan["single_pass"], plan
        _score_case(B, n_h, n_kv, d, s_max, w, np.array(sl, np.int32), wic=wic, n_keep=max(w, 8), seed=20 + seed,
                    planted=10 if s_max > 2000 else 0)


def test_score_single_pass_deferred_items():
    # every item left to the follow-up kernel (forced from the host): identical results
    B, n_h, n_kv, d, s_max, w = 2, 16, 16, 128, 6000, 32
    sl = np.array([6000, 3333], np.int32)
    _say("score single pass, every item deferred")
    q = _randn((B, n_h, w, d), 310)
    k = _randn((B, n_kv, s_max, d), 311)
    dims = kvc.make_dims(B, s_max, n_h, n_kv, d, kvc.KVC_BF16)
    ws = torch.zeros(kvc.score_window_workspace(dims, w), dtype=torch.uint8, device=DEV)
    raw, pooled = kvc.score_window(q, k, w, seq_lens=sl, n_keep=w, pool=7, ws=ws)
    raw_d, pooled_d = kvc.score_window(q, k, w, seq_lens=sl, n_keep=w, pool=7, ws=ws, defer_all=True)
    raw_n, pooled_n = kvc.score_window(q, k, w, seq_lens=sl, n_keep=w, pool=7, ws=ws)   # the count went back to 0
    torch.cuda.synchronize()
    assert torch.equal(raw, raw_d) and torch.equal(pooled, pooled_d)
    assert torch.equal(raw, raw_n) and torch.equal(pooled, pooled_n)
    rraw, _ = oracle.score_window(host(q), host(k), w, seq_lens=sl, n_keep=w, pool=7)
    assert_scores_close(raw_d, rraw, "raw")


def test_score_single_pass_unit_mask_and_reuse():
    # masked units are left as they were; one workspace reused by calls of other
    # lengths and masks (its counters return to zero)
    B, n_h, n_kv, d, s_max, w = 2, 8, 8, 128, 5000, 32
    q = _randn((B, n_h, w, d), 320)
    k = _randn((B, n_kv, s_max, d), 321)
    dims = kvc.make_dims(B, s_max, n_h, n_kv, d, kvc.KVC_BF16)
    ws = torch.zeros(kvc.score_window_workspace(dims, w), dtype=torch.uint8, device=DEV)
    rng = np.random.default_rng(9)
    for i, sl in enumerate(([5000, 3100], [4000, 5000], [1, 2600])):
        sl = np.array(sl, np.int32)
        _say("score single pass mask", i, list(sl))
        full_raw, full_pooled = kvc.score_window(q, k, w, seq_lens=sl, n_keep=w, pool=7, ws=ws)
        mask = torch.from_numpy(rng.integers(0, 2, (B, n_kv)).astype(np.int32)).to(DEV)
        raw = torch.full((B, n_kv, s_max), -7.0, device=DEV)
        pooled = torch.full((B, n_kv, s_max), -9.0, device=DEV)
        kvc.score_window(q, k, w, seq_lens=sl, n_keep=w, pool=7, raw=raw, pooled=pooled, unit_mask=mask, ws=ws)
        torch.cuda.synchronize()
        on = mask.bool()
        assert torch.equal(raw[on], full_raw[on]) and torch.equal(pooled[on], full_pooled[on])
        assert bool((raw[~on] == -7.0).all()) and bool((pooled[~on] == -9.0).all())
        rraw, _ = oracle.score_window(host(q), host(k), w, seq_lens=sl, n_keep=w, pool=7)
        assert_scores_close(full_raw, rraw, "raw")


def test_score_single_pass_rounds_ragged_reuse():
    # two rounds of the persistent grid (30 items per KV head, 32 KV heads), a
    # short sequence whose later items only write zeros, and one workspace reused by a
    # call of other lengths: the second call must not take the first call's final
    # statistics (their words carry the earlier call's tag)
    B, n_h, n_kv, d, s_max, w = 2, 16, 16, 128, 30000, 32
    plan = _plan(B, n_h, n_kv, d, s_max, w)
    assert plan["single_pass"] and plan["chunks_per_unit"] == 30, plan
    q = _randn((B, n_h, w, d), 330)
    k = _randn((B, n_kv, s_max, d), 331)
    rng = np.random.default_rng(33)
    pos = torch.from_numpy(rng.choice(s_max - w, 12, replace=False)).to(DEV)
    k[:, :, pos, :] = (3.0 * _randn((1, n_kv, 1, d), 332)).to(k.dtype)
    dims = kvc.make_dims(B, s_max, n_h, n_kv, d, kvc.KVC_BF16)
    ws = torch.zeros(kvc.score_window_workspace(dims, w), dtype=torch.uint8, device=DEV)
    for sl in ([30000, 17777], [21000, 30000]):
        sl = np.array(sl, np.int32)
        _say("score single pass rounds", list(sl))
        raw, pooled = kvc.score_window(q, k, w, seq_lens=sl, n_keep=w, pool=7, ws=ws)
        torch.cuda.synchronize()
        rraw, rpooled = oracle.score_window(host(q), host(k), w, seq_lens=sl, n_keep=w, pool=7)
        assert_scores_close(raw, rraw, "raw")
        assert_scores_close(pooled, rpooled, "pooled")


@pytest.mark.parametrize("s_max", [2999, 3000])
def test_pool_kernel_widths(s_max):
    # every compiled window (pool 1, 3, 5, 7 specialised, 9 and 63 walked), rows of a
    # multiple of 4 floats and not, candidate regions ending inside and at a tile edge
    sl = np.array([s_max, 1024 + 40, 17, 2048 + 32], np.int32)
    q = _randn((4, 8, 8, 64), 400)
    k = _randn((4, 2, s_max, 64), 401)
    for pool in (1, 3, 5, 7, 9, 63):
        for n_keep in (0, 8, 40):
            _say("pool", s_max, pool, n_keep)
            raw, pooled = kvc.score_window(q, k, 8, seq_lens=sl, n_keep=n_keep, pool=pool)
            torch.cuda.synchronize()
            _, want = _pool_np(host(raw), sl, n_keep, pool)
            assert np.array_equal(host(pooled), want), (pool, n_keep)


def test_score_then_select_matches_oracle_rule():
    sl = np.array([4000], np.int32)
    q, k, raw, pooled, rpooled = _score_case(1, 32, 8, 128, 4000, 32, sl, planted=40, seed=7)
    idx, cnt = kvc.select_topk(pooled, 256, 32, seq_lens=sl)
    ri, rc = oracle.select_topk(rpooled, 256, 32, seq_lens=sl)
    check_selection(idx, cnt, ri, rc, rpooled, sl, 256, 32)


def test_select_per_unit_budgets():
    # budgets that differ per unit (Tutorial "Compresser un cache existant": PyramidKV),
    # clamped to [0, k]; each unit matches the oracle with its own budget
    _say("select per-unit budgets")
    rng = np.random.default_rng(77)
    B, H, s_max, k, n_keep = 3, 8, 20000, 1500, 32
    sc = rng.random((B, H, s_max)).astype(np.float32) ** 3
    sc[1, 2] = (rng.integers(0, 40, s_max) / 39.0).astype(np.float32)       # exact ties
    sl = np.array([s_max, 12345, 900], np.int32)
    ku = rng.integers(0, k + 1, (B, H)).astype(np.int32)
    ku[0, 0], ku[0, 1], ku[2, 3] = 0, k + 500, -4                              # none, clamped to k, clamped to 0
    idx, cnt = kvc.select_topk(torch.from_numpy(sc).to(DEV), k, n_keep, seq_lens=sl,
                               k_per_unit=torch.from_numpy(ku).to(DEV))
    ri, rc = oracle.select_topk(sc, k, n_keep, seq_lens=sl, k_per_unit=ku)
    assert np.array_equal(host(idx), ri) and np.array_equal(host(cnt), rc)


@pytest.mark.parametrize("s_max", [3000, 32768])
def test_select_core_vs_oracle(s_max):
    # CASK role-based retention: core tokens kept, the budget over the scratch tokens
    _say("select core", s_max)
    rng = np.random.default_rng(s_max + 5)
    B, H, k, core_cap, n_keep = 3, 8, 700, 600, 32
    sc = (rng.random((B, H, s_max)) ** 2).astype(np.float32)
    sc[0, 1] = (rng.integers(0, 30, s_max) / 29.0).astype(np.float32)          # exact ties
    core = (rng.random((B, s_max)) < 0.012).astype(np.uint8)
    core[2, :] = 0                                                                # no core token
    sl = np.array([s_max, max(1, s_max // 3), s_max - 7], np.int32)
    idx, cnt = kvc.select_core(torch.from_numpy(sc).to(DEV), torch.from_numpy(core).to(DEV), k, core_cap, n_keep,
                               seq_lens=sl)
    ri, rc = oracle.select_core(sc, core, k, n_keep, seq_lens=sl, core_cap=core_cap)
    n_core = [int(core[b, :max(0, sl[b] - n_keep)].sum()) for b in range(B)]
    assert max(n_core) <= core_cap
    assert np.array_equal(host(cnt), rc) and np.array_equal(host(idx), ri)
    # every core candidate is kept
    gi = host(idx)
    for b in range(B):
        cores = np.nonzero(core[b, :max(0, sl[b] - n_keep)])[0]
        for h in range(H):
            assert np.isin(cores, gi[b, h]).all()


@pytest.mark.parametrize("k,core_cap", [(10, 20), (70, 60), (50, 0), (300, 99)])
def test_select_core_over_capacity_vs_oracle(k, core_cap):
    # more core candidates (100) than core_cap: the first k + core_cap candidates of
    # "core by index, then scratch by score" are kept, as the oracle defines it
    _say("select core over capacity", k, core_cap)
    s_max, n_keep = 4096, 8
    rng = np.random.default_rng(3 + k)
    sc = rng.random((2, 2, s_max)).astype(np.float32)
    sc[1, 0] = (rng.integers(0, 9, s_max) / 8.0).astype(np.float32)            # exact ties
    core = np.zeros((2, s_max), np.uint8)
    core[0, 100:200] = 1
    core[1, rng.choice(s_max - n_keep, 100, replace=False)] = 1
    sl = np.array([s_max, 3001], np.int32)
    idx, cnt = kvc.select_core(torch.from_numpy(sc).to(DEV), torch.from_numpy(core).to(DEV), k, core_cap, n_keep,
                               seq_lens=sl)
    ri, rc = oracle.select_core(sc, core, k, n_keep, seq_lens=sl, core_cap=core_cap)
    assert np.array_equal(host(cnt), rc) and np.array_equal(host(idx), ri)


def test_calls_on_a_side_stream():
    # stream=: every temporary the binding allocates or fills (workspaces, outputs,
    # host lengths) is ordered on that stream; results equal the default stream's
    _say("calls on a side stream")
    B, n_h, n_kv, S, d, w, k, n_keep = 2, 8, 2, 5000, 128, 16, 300, 16
    q = _randn((B, n_h, w, d), 91)
    kk = _randn((B, n_kv, S, d), 92)
    vv = _randn((B, n_kv, S, d), 93)
    qd = _randn((B, n_h, d), 94)
    lens = np.array([S, 3333], np.int32)

    def run(stream):
        _, pooled = kvc.score_window(q, kk, w, seq_lens=lens, n_keep=n_keep, pool=7, stream=stream)
        idx, cnt = kvc.select_topk(pooled, k, n_keep, seq_lens=lens, stream=stream)
        kc, vc, pos = kvc.gather_compact(kk, idx, cnt, src1=vv, stream=stream)
        out, lse = kvc.decode_attn(qd, kc, vc, cnt, stream=stream)
        return [t for t in (pooled, idx, cnt, kc, vc, pos, out, lse)]

    ref = run(None)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    got = run(side)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for a, b in zip(ref, got):
        assert torch.equal(a, b)
    with pytest.raises(TypeError):
        kvc.decode_attn(qd, got[3], got[4], got[2], stream=123)
