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
from sparse_decode_amd.pipeline import LayerPath, TspStep
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


def test_cfg2_layers_folded_into_batch():
    # compressing an existing cache of several layers in one call: the layers are
    # independent units of the batch; every layer must match the oracle on its own
    wl = synth.WORKLOADS[2]
    layers = (0, 7, 31)
    _say(wl.name, "layers", layers, "in one call")
    inps = [synth.layer_inputs(wl, l, device="cuda") for l in layers]
    q = torch.cat([x["q_win"] for x in inps]).contiguous()
    k = torch.cat([x["k"] for x in inps]).contiguous()
    v = torch.cat([x["v"] for x in inps]).contiguous()
    sl = np.concatenate([x["seq_lens"] for x in inps])
    sl_dev = torch.from_numpy(sl).cuda()
    path = LayerPath(wl, batch=len(layers))
    path.score(q, k, sl_dev)
    path.select(sl_dev)
    path.gather(k, v)
    torch.cuda.synchronize()
    for i, x in enumerate(inps):
        _say("  layer", layers[i])
        rraw, rpooled = oracle.score_window(host(x["q_win"]), host(x["k"]), wl.w, seq_lens=x["seq_lens"],
                                            window_in_cache=wl.window_in_cache, n_keep=wl.n_keep, pool=wl.pool)
        assert_scores_close(path.raw[i:i + 1], rraw, "raw")
        assert_scores_close(path.pooled[i:i + 1], rpooled, "pooled")
        ri, rc = oracle.select_topk(rpooled, wl.k, wl.n_keep, seq_lens=x["seq_lens"])
        check_selection(path.idx[i:i + 1], path.count[i:i + 1], ri, rc, rpooled, x["seq_lens"], wl.k, wl.n_keep)
        gi, gc = host(path.idx[i:i + 1]), host(path.count[i:i + 1])
        ref, _ = oracle.gather(_bits(x["k"]), gi, gc, dst=_bits(path.kc[i:i + 1]))
        assert np.array_equal(_bits(path.kc[i:i + 1]), ref)


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
