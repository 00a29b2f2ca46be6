"""End-to-end GPU parity on the five workloads at their full sizes: one layer (or
step) of score -> select -> gather -> decode against the CPU oracle on the same
seeded inputs."""
import math
import sys

import numpy as np
import pytest
import torch

import oracle
from sparse_decode_amd import kvc, synth
from sparse_decode_amd.pipeline import LayerPath, TspSchedule, TspStep
from _parity import assert_decode_close, assert_scores_close, check_selection, host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    kvc.lib()
    oracle.set_threads(0)
    yield


def _say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def _bits(t):
    return t.view(torch.int16).cpu().numpy() if t.dtype == torch.bfloat16 else t.view(torch.int32).cpu().numpy()


def _layer_parity(wl, layer, *, step=0, s_max=None, k=None, src_pos=None, check_planted=True):
    _say(wl.name, "layer", layer, "step", step, "s_max", s_max or wl.s_max)
    inp = synth.layer_inputs(wl, layer, device="cuda", step=step, s_max=s_max)
    sl = inp["seq_lens"]
    sl_dev = torch.from_numpy(sl).cuda()
    path = LayerPath(wl, s_max=s_max, k=k)
    sp_dev = None if src_pos is None else torch.from_numpy(src_pos).cuda()
    path.run(inp["q_win"], inp["k"], inp["v"], inp["q_dec"], sl_dev, sp_dev)
    torch.cuda.synchronize()
    q_h, k_h = host(inp["q_win"]), host(inp["k"])
    rraw, rpooled = oracle.score_window(q_h, k_h, wl.w, seq_lens=sl, window_in_cache=wl.window_in_cache,
                                        n_keep=wl.n_keep, pool=wl.pool)
    assert_scores_close(path.raw, rraw, "raw")
    assert_scores_close(path.pooled, rpooled, "pooled")
    ri, rc = oracle.select_topk(rpooled, path.k, wl.n_keep, seq_lens=sl)
    differ = check_selection(path.idx, path.count, ri, rc, rpooled, sl, path.k, wl.n_keep)
    _say("  selections differing from the oracle (near ties):", differ)
    # the GPU's own selection, gathered by the oracle, is bit-identical
    gi, gc = host(path.idx), host(path.count)
    for src, dst in ((inp["k"], path.kc), (inp["v"], path.vc)):
        ref, ref_pos = oracle.gather(_bits(src), gi, gc, src_pos=src_pos, dst=_bits(dst))
        assert np.array_equal(_bits(dst), ref)
        assert np.array_equal(host(path.pos), ref_pos)
    ref_out, ref_lse = oracle.decode(host(inp["q_dec"]), host(path.kc), host(path.vc), gc)
    assert_decode_close(path.out, ref_out, wl.dtype == "bf16")
    assert np.allclose(host(path.lse), ref_lse, rtol=1e-5, atol=1e-4)
    if check_planted:
        _planted(wl, inp, path, sl)
    return inp, path, rpooled


def _planted(wl, inp, path, sl):
    """Planted heavy hitters are selected: always without pooling, and with pooling
    whenever their pooled tie blocks fit the budget."""
    path1 = LayerPath(wl, s_max=path.S, k=path.k)
    kvc.score_window(inp["q_win"], inp["k"], wl.w, seq_lens=torch.from_numpy(sl).cuda(),
                     window_in_cache=wl.window_in_cache, n_keep=wl.n_keep, pool=1, raw=path1.raw,
                     pooled=path1.pooled, ws=path1.ws_score)
    path1.select(torch.from_numpy(sl).cuda())
    torch.cuda.synchronize()
    for pooled_path, pool in ((path1, 1), (path, wl.pool)):
        gi, gc = host(pooled_path.idx), host(pooled_path.count)
        for b, pos in enumerate(inp["planted"]):
            planted = set(pos.tolist())
            if not planted:
                continue
            for g in range(wl.n_kv):
                sel = set(gi[b, g, : gc[b, g]].tolist())
                kept = len(planted & sel) / len(planted)
                if pool == 1 or len(planted) * pool <= path.k:
                    assert kept == 1.0, (wl.name, b, g, pool, kept)
        _say("  planted retained with pool", pool)


def test_cfg1_tiny_fp32():
    wl = synth.WORKLOADS[1]
    _layer_parity(wl, 0)


def test_cfg2_llama3_8b_32k():
    wl = synth.WORKLOADS[2]
    _layer_parity(wl, 0)
    _layer_parity(wl, 31, check_planted=False)


def _folded_parity(wl, layers, sampled, want_plan):
    """Compresses the cache of several layers in one call each of score, select and
    gather (the layers folded into the batch, as the benchmark's step does), checks
    that the score call takes the launch configuration the benchmark times, then:
    every layer's selection equals the oracle's selection over the GPU's own pooled
    scores bit for bit, and on the sampled layers the raw and pooled scores, the
    selection and the gathered rows match the oracle on the layer's inputs."""
    L, B = len(layers), wl.batch
    _say(wl.name, "%d layers in one call, sampled" % L, sampled)
    S, d = wl.s_max, wl.d_h
    K = torch.empty((L * B, wl.n_kv, S, d), dtype=wl.torch_dtype, device="cuda")
    V = torch.empty_like(K)
    Q = torch.empty((L * B, wl.n_h, wl.w, d), dtype=wl.torch_dtype, device="cuda")
    sl = None
    for i, l in enumerate(layers):
        x = synth.layer_inputs(wl, l, device="cuda")
        K[i * B:(i + 1) * B].copy_(x["k"])
        V[i * B:(i + 1) * B].copy_(x["v"])
        Q[i * B:(i + 1) * B].copy_(x["q_win"])
        sl = x["seq_lens"]
        del x
    sl_all = np.tile(sl, L)
    sl_dev = torch.from_numpy(sl_all).cuda()
    path = LayerPath(wl, batch=L * B)
    dims = kvc.make_dims(L * B, S, wl.n_h, wl.n_kv, d, kvc.KVC_BF16)
    plan = kvc.score_window_plan(dims, wl.w)
    _say("  score plan", plan)
    assert plan == want_plan
    path.score(Q, K, sl_dev)
    path.select(sl_dev)
    path.gather(K, V)
    torch.cuda.synchronize()
    gp = host(path.pooled)
    ri, rc = oracle.select_topk(gp, wl.k, wl.n_keep, seq_lens=sl_all)
    assert np.array_equal(host(path.idx), ri) and np.array_equal(host(path.count), rc)
    for l in sampled:
        i = layers.index(l)
        _say("  layer", l)
        x = synth.layer_inputs(wl, l, device="cuda")
        rows = slice(i * B, (i + 1) * B)
        rraw, rpooled = oracle.score_window(host(x["q_win"]), host(x["k"]), wl.w, seq_lens=x["seq_lens"],
                                            window_in_cache=wl.window_in_cache, n_keep=wl.n_keep, pool=wl.pool)
        assert_scores_close(path.raw[rows], rraw, "raw")
        assert_scores_close(path.pooled[rows], rpooled, "pooled")
        ri, rc = oracle.select_topk(rpooled, wl.k, wl.n_keep, seq_lens=x["seq_lens"])
        check_selection(path.idx[rows], path.count[rows], ri, rc, rpooled, x["seq_lens"], wl.k, wl.n_keep)
        gi, gc = host(path.idx[rows]), host(path.count[rows])
        for src, dst in ((x["k"], path.kc[rows]), (x["v"], path.vc[rows])):
            ref, ref_pos = oracle.gather(_bits(src), gi, gc, dst=_bits(dst))
            assert np.array_equal(_bits(dst), ref)
        assert np.array_equal(host(path.pos[rows]), ref_pos)
        del x


def test_cfg2_all_layers_folded_as_timed():
    # the benchmark's score call: 32 layers x 8 KV heads in one launch, 2048-token
    # work-groups over 8 blocks of 16 window rows
    wl = synth.WORKLOADS[2]
    _folded_parity(wl, list(range(wl.layers)), (0, 15, 31),
                   {"mfma": True, "rt": 8, "chunk_tokens": 2048, "chunks_per_unit": 16, "single_pass": False,
                    "folded_merge": False})


def test_cfg3_layers_folded():
    wl = synth.WORKLOADS[3]
    _folded_parity(wl, [0, 31], (0, 31), {"mfma": True, "rt": 8, "chunk_tokens": 2048, "chunks_per_unit": 64,
                                          "single_pass": False, "folded_merge": False})


def test_cfg3_ctx_128k():
    wl = synth.WORKLOADS[3]
    assert wl.k == synth.budget_from_rate(0.01, wl.s_max) == 1311
    _layer_parity(wl, 0)


def test_cfg4_ragged_batched_steps():
    wl = synth.WORKLOADS[4]
    for step in (0, 63):
        _layer_parity(wl, 0, step=step, check_planted=(step == 0))


def test_cfg5_mha_tsp():
    wl = synth.WORKLOADS[5]
    k_tsp = synth.budget_from_rate(wl.tsp_rate, wl.s_max)
    assert k_tsp == 13108
    inp, path, rpooled = _layer_parity(wl, wl.tsp_layer, check_planted=False)
    # token-selective propagation at the TSP layer: one set per sequence, hidden states gathered
    _say("mha_tsp TSP select + hidden gather")
    hidden = synth.hidden_states(wl, device="cuda")
    tsp = TspStep(wl, k_tsp)
    hid_out, pos = tsp.run(path.pooled, hidden)
    torch.cuda.synchronize()
    ri, rc = oracle.select_topk(rpooled, k_tsp, wl.n_keep, seq_lens=inp["seq_lens"], shared_heads=True)
    check_selection(tsp.idx, tsp.count, ri, rc, rpooled, inp["seq_lens"], k_tsp, wl.n_keep, shared=True)
    gi, gc = host(tsp.idx), host(tsp.count)
    assert np.all(gc == k_tsp + wl.n_keep)
    hb = _bits(hidden).reshape(wl.batch, 1, wl.s_max, wl.hidden)
    ref, ref_pos = oracle.gather(hb, gi, gc)
    assert np.array_equal(_bits(hid_out), ref)
    assert np.array_equal(host(pos), ref_pos)
    del hidden, hb, ref
    # a later layer runs over the propagated tokens and keeps their original positions
    s2 = k_tsp + wl.n_keep
    src_pos = gi[:, 0, :].astype(np.int32)
    _layer_parity(wl, wl.tsp_layer + 1, s_max=s2, src_pos=src_pos, check_planted=False)


@pytest.mark.parametrize("tsp_layer,tsp_rate", [(8, 0.1), (24, 0.4)])
def test_cfg5_tsp_other_layer_and_rate(tsp_layer, tsp_rate):
    # FastKV 2.A/2.B: the propagation layer and the TSP rate are free parameters,
    # independent of the per-layer KV budget
    import dataclasses
    wl = dataclasses.replace(synth.WORKLOADS[5], tsp_layer=tsp_layer, tsp_rate=tsp_rate)
    k_tsp = synth.budget_from_rate(tsp_rate, wl.s_max)
    inp, path, rpooled = _layer_parity(wl, tsp_layer, check_planted=False)
    _say("mha_tsp TSP at layer", tsp_layer, "rate", tsp_rate, "k", k_tsp)
    hidden = synth.hidden_states(wl, device="cuda")
    tsp = TspStep(wl, k_tsp)
    hid_out, pos = tsp.run(path.pooled, hidden)
    torch.cuda.synchronize()
    ri, rc = oracle.select_topk(rpooled, k_tsp, wl.n_keep, seq_lens=inp["seq_lens"], shared_heads=True)
    check_selection(tsp.idx, tsp.count, ri, rc, rpooled, inp["seq_lens"], k_tsp, wl.n_keep, shared=True)
    gi, gc = host(tsp.idx), host(tsp.count)
    assert np.all(gc == k_tsp + wl.n_keep)
    ref, ref_pos = oracle.gather(_bits(hidden).reshape(wl.batch, 1, wl.s_max, wl.hidden), gi, gc)
    assert np.array_equal(_bits(hid_out), ref)
    assert np.array_equal(host(pos), ref_pos)
    del hidden, ref
    s2 = k_tsp + wl.n_keep
    _layer_parity(wl, tsp_layer + 1, s_max=s2, src_pos=gi[:, 0, :].astype(np.int32), check_planted=False)


def test_tsp_schedule_whole_model():
    # the benchmark's whole-model step (pipeline.TspSchedule) on a 4-layer MHA model of
    # 4096 tokens, propagation at layer 1 keeping 25 %: every layer's selection,
    # compacted cache, positions and attention against the oracle, and the propagation
    import dataclasses
    wl = dataclasses.replace(synth.WORKLOADS[5], layers=4, s_max=4096, tsp_layer=1, tsp_rate=0.25, k=256)
    k_tsp = synth.budget_from_rate(wl.tsp_rate, wl.s_max)
    s2 = k_tsp + wl.n_keep
    _say("tsp schedule", dict(layers=wl.layers, S=wl.s_max, tsp_layer=wl.tsp_layer, k_tsp=k_tsp))
    xs = [synth.layer_inputs(wl, l, device="cuda", s_max=None if l <= wl.tsp_layer else s2)
          for l in range(wl.layers)]
    hidden = synth.hidden_states(wl, device="cuda")
    seq_full = torch.from_numpy(xs[0]["seq_lens"]).cuda()
    seq_after = torch.from_numpy(xs[-1]["seq_lens"]).cuda()
    layers = [{n: x[n] for n in ("q_win", "k", "v", "q_dec")} for x in xs]
    sched = TspSchedule(wl, layers, wl.tsp_layer, k_tsp, seq_full, seq_after, hidden)
    sched.step()
    torch.cuda.synchronize()
    tsp_pos = host(sched.src_pos).astype(np.int32)
    for l, x in enumerate(xs):
        _say("  layer", l)
        sl = x["seq_lens"]
        src_pos = None if l <= wl.tsp_layer else tsp_pos
        _, rpooled = oracle.score_window(host(x["q_win"]), host(x["k"]), wl.w, seq_lens=sl,
                                         window_in_cache=wl.window_in_cache, n_keep=wl.n_keep, pool=wl.pool)
        ri, rc = oracle.select_topk(rpooled, wl.k, wl.n_keep, seq_lens=sl)
        check_selection(sched.idx[l], sched.count[l], ri, rc, rpooled, sl, wl.k, wl.n_keep)
        gi, gc = host(sched.idx[l]), host(sched.count[l])
        for src, dst in ((x["k"], sched.kc[l]), (x["v"], sched.vc[l])):
            ref, ref_pos = oracle.gather(_bits(src), gi, gc, src_pos=src_pos, dst=_bits(dst))
            assert np.array_equal(_bits(dst), ref)
        assert np.array_equal(host(sched.pos[l]), ref_pos)
        ref_out, _ = oracle.decode(host(x["q_dec"]), host(sched.kc[l]), host(sched.vc[l]), gc)
        assert_decode_close(sched.out[l], ref_out, True)
        if l == wl.tsp_layer:
            ti, tc = oracle.select_topk(rpooled, k_tsp, wl.n_keep, seq_lens=sl, shared_heads=True)
            check_selection(sched.tsp.idx, sched.tsp.count, ti, tc, rpooled, sl, k_tsp, wl.n_keep, shared=True)
            hi, hc = host(sched.tsp.idx), host(sched.tsp.count)
            ref, ref_pos = oracle.gather(_bits(hidden).reshape(wl.batch, 1, wl.s_max, wl.hidden), hi, hc)
            assert np.array_equal(_bits(sched.tsp.hidden_out), ref)
            assert np.array_equal(tsp_pos, ref_pos[:, 0, :])
