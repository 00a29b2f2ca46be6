"""Seeded random shapes through the whole path (score -> select -> gather -> decode)
against the CPU oracle: odd sequence lengths, empty and ragged sequences, MQA to
MHA groupings (including a group of 3 query heads), both head sizes, bf16 and fp32,
queries in or out of the cache, every pool width the workloads use and budgets from
window-only to dense.  Then the selection alone on scores full of exact ties, at
unit counts and row lengths that take each of its kernel paths."""
import sys

import numpy as np
import pytest
import torch

import oracle
from sparse_decode_amd import kvc
from _parity import assert_decode_close, assert_scores_close, check_selection, host

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    kvc.lib()
    oracle.set_threads(0)
    yield


def _draw(seed):
    rng = np.random.default_rng(seed)
    c = {}
    c["d"] = int(rng.choice([64, 128]))
    c["bf16"] = bool(rng.random() < 0.75)
    c["n_kv"] = int(rng.choice([1, 2, 4, 8]))
    r = int(rng.choice([1, 2, 3, 4, 8]))
    c["n_h"] = c["n_kv"] * r
    c["B"] = int(rng.integers(1, 4))
    c["s_max"] = int(rng.integers(1, 3000))
    c["w"] = int(rng.integers(1, 65))
    c["wic"] = bool(rng.random() < 0.7)
    c["n_keep"] = int(rng.integers(0, c["w"] + 1)) if c["wic"] else int(rng.integers(0, 33))
    c["pool"] = int(rng.choice([1, 3, 5, 7, 9]))
    c["k"] = int(rng.integers(0 if c["n_keep"] > 0 else 1, c["s_max"] + 1))
    lens = rng.integers(0, c["s_max"] + 1, c["B"]).astype(np.int32)
    lens[0] = c["s_max"]
    if c["B"] > 1 and rng.random() < 0.4:
        lens[-1] = 0                                  # an empty sequence
    c["seq_lens"] = lens
    return c


def _bits(t):
    return t.view(torch.int16).cpu().numpy() if t.dtype == torch.bfloat16 else t.view(torch.int32).cpu().numpy()


def _randn(shape, seed, dtype):
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    return torch.randn(shape, generator=g, device=DEV, dtype=torch.float32).to(dtype)


@pytest.mark.parametrize("seed", range(24))
def test_random_shape_path(seed):
    c = _draw(seed)
    print("[case] seed", seed, {k: (v.tolist() if isinstance(v, np.ndarray) else v) for k, v in c.items()}, flush=True)
    sys.stdout.flush()
    dtype = torch.bfloat16 if c["bf16"] else torch.float32
    B, n_h, n_kv, d, s_max, w = c["B"], c["n_h"], c["n_kv"], c["d"], c["s_max"], c["w"]
    sl = c["seq_lens"]
    q_win = _randn((B, n_h, w, d), 10 * seed + 1, dtype)
    k = _randn((B, n_kv, s_max, d), 10 * seed + 2, dtype)
    v = _randn((B, n_kv, s_max, d), 10 * seed + 3, dtype)
    q = _randn((B, n_h, d), 10 * seed + 4, dtype)

    raw, pooled = kvc.score_window(q_win, k, w, seq_lens=sl, window_in_cache=c["wic"], n_keep=c["n_keep"],
                                   pool=c["pool"])
    torch.cuda.synchronize()
    rraw, rpooled = oracle.score_window(host(q_win), host(k), w, seq_lens=sl, window_in_cache=c["wic"],
                                        n_keep=c["n_keep"], pool=c["pool"])
    assert_scores_close(raw, rraw, "raw")
    assert_scores_close(pooled, rpooled, "pooled")

    idx, cnt = kvc.select_topk(pooled, c["k"], c["n_keep"], seq_lens=sl)
    torch.cuda.synchronize()
    ri, rc = oracle.select_topk(rpooled, c["k"], c["n_keep"], seq_lens=sl)
    check_selection(idx, cnt, ri, rc, rpooled, sl, c["k"], c["n_keep"])

    kc, vc, pos = kvc.gather_compact(k, idx, cnt, src1=v)
    torch.cuda.synchronize()
    gi, gc = host(idx), host(cnt)
    for src, dst in ((k, kc), (v, vc)):
        ref, ref_pos = oracle.gather(_bits(src), gi, gc, dst=_bits(dst))
        assert np.array_equal(_bits(dst), ref)
        assert np.array_equal(host(pos), ref_pos)

    out, lse = kvc.decode_attn(q, kc, vc, cnt)
    torch.cuda.synchronize()
    ref_out, ref_lse = oracle.decode(host(q), host(kc), host(vc), gc)
    assert_decode_close(out, ref_out, c["bf16"])


@pytest.mark.parametrize("seed", range(12))
def test_random_selection_ties(seed):
    # selection alone at up to 512 units and 70000 keys (the per-unit kernel and both
    # chunk sizes of the chunked kernels), with scores on few levels so that exact ties
    # are everywhere; per-KV-head, shared over heads, and with per-unit budgets
    rng = np.random.default_rng(7000 + seed)
    n_kv = int(rng.choice([1, 2, 4, 8]))
    B = int(rng.integers(1, 65))
    s_max = int(rng.choice([int(rng.integers(1, 5000)), int(rng.integers(5000, 34000)),
                            int(rng.integers(34000, 70000))]))
    B = max(1, min(B, 8_000_000 // (n_kv * s_max)))
    n_keep = int(rng.integers(0, 64))
    k = int(rng.integers(0 if n_keep else 1, min(s_max, 4096) + 1))
    lens = rng.integers(0, s_max + 1, B).astype(np.int32)
    lens[0] = s_max
    levels = int(rng.choice([3, 50, 1000, 1 << 20]))
    sc_np = (rng.integers(0, levels, (B, n_kv, s_max)).astype(np.float32) / levels) ** 2
    print("[case] seed", seed, dict(B=B, n_kv=n_kv, s_max=s_max, k=k, n_keep=n_keep, levels=levels), flush=True)
    sc = torch.from_numpy(sc_np).to(DEV)
    # shared over heads: dyadic scores (multiples of 2^-20 below 1, at most 8 heads)
    # add exactly in float, so the GPU's rounded head sum equals the oracle's exact one
    den = 1 << min(20, max(2, int(levels - 1).bit_length()))
    dy_np = (rng.integers(0, den, (B, n_kv, s_max)) / den).astype(np.float32)
    for shared, src_np in ((False, sc_np), (True, dy_np)):
        idx, cnt = kvc.select_topk(torch.from_numpy(src_np).to(DEV), k, n_keep, seq_lens=lens, shared_heads=shared)
        torch.cuda.synchronize()
        ri, rc = oracle.select_topk(src_np, k, n_keep, seq_lens=lens, shared_heads=shared)
        assert np.array_equal(host(cnt), rc)
        assert np.array_equal(host(idx), ri)
    kpu = rng.integers(0, k + 1, (B, n_kv)).astype(np.int32)
    idx, cnt = kvc.select_topk(sc, k, n_keep, seq_lens=lens, k_per_unit=torch.from_numpy(kpu).to(DEV))
    torch.cuda.synchronize()
    ri, rc = oracle.select_topk(sc_np, k, n_keep, seq_lens=lens, k_per_unit=kpu)
    assert np.array_equal(host(cnt), rc)
    assert np.array_equal(host(idx), ri)
