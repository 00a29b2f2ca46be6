"""GPU parity of speculative retrieval with fine-grained correction (FreeKV technical
summary 2.A): the query-similarity call, unit-masked score/select/gather, and the
per-step schedule on the batched ragged decode workload against the CPU oracle."""
import sys

import numpy as np
import pytest
import torch

import oracle
from sparse_decode_amd import kvc, synth
from sparse_decode_amd.pipeline import LayerPath, SpeculativeRetrieval
from _parity import assert_decode_close, assert_scores_close, check_selection, host

pytestmark = pytest.mark.gpu
DEV = "cuda"
TAU = 0.85
MARGIN = 1e-9       # decisions within this of tau may legitimately differ (double sums, other order)


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


def _check_flags(gpu_refresh, ref_refresh, ref_cos, n_kv, tau):
    """Equal flags except for KV heads with a query head within MARGIN of tau."""
    g, r = host(gpu_refresh), np.asarray(ref_refresh)
    B, n_h = ref_cos.shape
    near = np.zeros_like(r, dtype=bool)
    grp = n_h // n_kv
    for b in range(B):
        for h in range(n_h):
            if abs(ref_cos[b, h] - tau) <= MARGIN:
                near[b, h // grp] = True
    assert np.array_equal(g[~near], r[~near]), "correction flags differ"
    return int(near.sum())


@pytest.mark.parametrize("dtype,d", [(torch.bfloat16, 128), (torch.float32, 64)])
def test_query_similarity_vs_oracle(dtype, d):
    _say("similarity", dtype, d)
    g = torch.Generator(device=DEV)
    g.manual_seed(31)
    B, n_h, n_kv = 5, 32, 8
    q = torch.randn((B, n_h, d), generator=g, device=DEV).to(dtype)
    p = (0.9 * q.float() + 0.45 * torch.randn((B, n_h, d), generator=g, device=DEV)).to(dtype)
    p[0, 0] = q[0, 0]              # identical
    p[0, 1] = -q[0, 1]             # opposite
    q[1, 2] = 0                    # zero query
    p[2, 3] = 0                    # zero previous query
    for tau in (TAU, 0.9, 2.0, -1.0):
        cos, ref, keep = kvc.query_similarity(q, p, n_kv, tau)
        torch.cuda.synchronize()
        rcos, rref = oracle.query_similarity(host(q), host(p), n_kv, tau)
        assert np.allclose(host(cos), rcos, rtol=0, atol=1e-6)
        assert host(cos)[0, 0] == 1.0 and host(cos)[0, 1] == -1.0 and host(cos)[1, 2] == 0.0
        _check_flags(ref, rref, rcos, n_kv, tau)
        assert np.array_equal(host(keep), 1 - host(ref))
    _, ref_all, _ = kvc.query_similarity(q, p, n_kv, 2.0)
    _, ref_none, _ = kvc.query_similarity(q, p, n_kv, -1.0)
    assert host(ref_all).all() and not host(ref_none).any()


def test_unit_masked_calls_touch_only_masked_units():
    wl = synth.WORKLOADS[4]
    B = 4
    _say("masked score/select/gather", wl.name, "batch", B)
    inp = synth.layer_inputs(wl, 0, device=DEV, step=5, batch=B)
    sl = torch.from_numpy(inp["seq_lens"]).to(DEV)
    full = LayerPath(wl, batch=B)
    full.score(inp["q_win"], inp["k"], sl)
    full.select(sl)
    full.gather(inp["k"], inp["v"])
    mask_np = (np.arange(B * wl.n_kv).reshape(B, wl.n_kv) % 3 == 1).astype(np.int32)
    mask_np[0, :] = 1
    mask = torch.from_numpy(mask_np).to(DEV)
    part = LayerPath(wl, batch=B)
    for t, fill in ((part.raw, 7.0), (part.pooled, 7.0), (part.idx, -7), (part.count, -7), (part.pos, -7)):
        t.fill_(fill)
    part.kc.fill_(3.0)
    part.vc.fill_(3.0)
    part.score(inp["q_win"], inp["k"], sl, unit_mask=mask)
    part.select(sl, unit_mask=mask)
    part.gather(inp["k"], inp["v"], unit_mask=mask)
    torch.cuda.synchronize()
    on = mask_np.astype(bool)
    for name in ("raw", "pooled", "idx", "count", "pos", "kc", "vc"):
        a = getattr(part, name)
        b = getattr(full, name)
        a_bits = _bits(a) if a.dtype in (torch.bfloat16, torch.float32) else host(a)
        b_bits = _bits(b) if b.dtype in (torch.bfloat16, torch.float32) else host(b)
        assert np.array_equal(a_bits[on], b_bits[on]), name          # masked in: identical to the full call
        untouched = host(a)[~on]
        if name in ("kc", "vc"):
            assert np.all(untouched == 3.0), name
        elif name in ("raw", "pooled"):
            assert np.all(untouched == 7.0), name
        else:
            assert np.all(untouched == -7), name


@pytest.mark.parametrize("tau", [TAU, 2.0])
def test_speculative_schedule_vs_oracle(tau):
    wl = synth.WORKLOADS[4]
    steps = 4
    _say("speculative schedule", wl.name, "tau", tau, "steps", steps)
    inp = synth.layer_inputs(wl, 0, device=DEV, step=0)
    k, v = inp["k"], inp["v"]
    sl = inp["seq_lens"]
    sl_dev = torch.from_numpy(sl).to(DEV)
    spec = SpeculativeRetrieval(wl, tau)
    k_h, v_h = host(k), host(v)
    kw = dict(seq_lens=sl, k_budget=wl.k, n_keep=wl.n_keep, pool=wl.pool, tau=tau)
    prev_q, prev_sel, corrected = None, None, []
    for i in range(steps):
        q = synth.step_query(wl, 0, i, device=DEV)
        spec.critical(q, prev_q, k, v, sl_dev)
        cur = spec.current
        torch.cuda.synchronize()
        q_h = host(q)
        ref = oracle.speculative_step(q_h, None if prev_q is None else host(prev_q), k_h, v_h, prev_sel, **kw)
        if prev_q is not None:
            _check_flags(spec.refresh, ref["refresh"], ref["cos"], wl.n_kv, tau)
            assert np.allclose(host(spec.cos), ref["cos"], rtol=0, atol=1e-6)
        gref = host(spec.refresh) if prev_q is not None else np.ones((wl.batch, wl.n_kv), np.int32)
        corrected.append(float(gref.mean()))
        # corrected heads: the selection made with q now; the others: the previous one
        if prev_q is not None:
            ref = oracle.speculative_step(q_h, host(prev_q), k_h, v_h, prev_sel, refresh=gref, **kw)
        check_selection(cur.idx, cur.count, ref["idx"], ref["count"],
                        np.where(gref[:, :, None] != 0, ref["pooled"], prev_pooled if prev_q is not None else 0),
                        sl, wl.k, wl.n_keep)
        gi, gc = host(cur.idx), host(cur.count)
        for src, dst in ((k, cur.kc), (v, cur.vc)):
            want, _ = oracle.gather(_bits(src), gi, gc, dst=_bits(dst))
            assert np.array_equal(_bits(dst), want)
        out_ref, _ = oracle.decode(q_h, host(cur.kc), host(cur.vc), gc)
        assert_decode_close(cur.out, out_ref, True, "decode step %d" % i)
        # the speculative selection for the next step, with this step's query
        spec.speculate(q, k, v, sl_dev)
        torch.cuda.synchronize()
        nxt = spec.other
        assert_scores_close(nxt.pooled, ref["pooled"], "pooled step %d" % i)
        check_selection(nxt.idx, nxt.count, ref["next_sel"][0], ref["next_sel"][1], ref["pooled"], sl, wl.k,
                        wl.n_keep)
        prev_q, prev_sel, prev_pooled = q, (host(nxt.idx), host(nxt.count)), ref["pooled"]
        spec.swap()
    _say("  corrected fraction per step", corrected)
    if tau > 1.0:
        assert all(c == 1.0 for c in corrected)
    else:
        assert corrected[0] == 1.0 and max(corrected[1:]) < 0.5


def test_overlapped_schedule_matches_sequential():
    # the speculative selection on a second stream beside the critical path (events
    # order the two caches) gives bit-identical attention outputs to running them in turn
    wl = synth.WORKLOADS[4]
    steps = 6
    _say("overlapped schedule", wl.name, "steps", steps)
    inp = synth.layer_inputs(wl, 0, device=DEV, step=0)
    k, v = inp["k"], inp["v"]
    sl = torch.from_numpy(inp["seq_lens"]).to(DEV)
    qs = [synth.step_query(wl, 0, i, device=DEV) for i in range(steps)]
    seq = SpeculativeRetrieval(wl, TAU)
    want = []
    for i, q in enumerate(qs):
        seq.critical(q, qs[i - 1] if i else None, k, v, sl)
        want.append(seq.current.out.clone())
        seq.speculate(q, k, v, sl)
        seq.swap()
    ovl = SpeculativeRetrieval(wl, TAU)
    main = torch.cuda.current_stream()
    side = torch.cuda.Stream()
    side.wait_stream(main)
    got, e_c, e_s = [], None, None
    for i, q in enumerate(qs):
        if e_s is not None:
            main.wait_event(e_s)
        ovl.critical(q, qs[i - 1] if i else None, k, v, sl)
        got.append(ovl.current.out.clone())
        e_prev_c, e_c = e_c, torch.cuda.Event()
        e_c.record(main)
        with torch.cuda.stream(side):
            if e_prev_c is not None:
                side.wait_event(e_prev_c)
            ovl.speculate(q, k, v, sl)
            e_s = torch.cuda.Event()
            e_s.record(side)
        ovl.swap()
    main.wait_stream(side)
    torch.cuda.synchronize()
    for i in range(steps):
        assert torch.equal(got[i].view(torch.int16), want[i].view(torch.int16)), "step %d" % i
