#!/usr/bin/env python3
"""Benchmark of the KV-cache compression hot path on one MI355X.

A step is one pass of the whole path over one batch of synthetic input: for every
layer of the workload, window scoring -> per-KV-head top-k -> compacting gather ->
GQA decode attention over the compacted cache.  The default workload is the
Llama-3-8B-shaped cache (32 layers, S = 32768, 32 query / 8 KV heads, d_h = 128,
bf16, w = 32, pool 7, k = 2048 + 32 kept) with every layer's K/V resident in HBM.

The timed step compresses the existing cache of all layers with one call each of
score, select and gather (the layers are independent units of the batch), then
runs one decode call per layer, as a model's decode step does.  The same step with
one call per layer for every part is timed as well ("layerwise").

Prints one JSON line.  `value` is whole-step algorithmic HBM traffic per second
(GB/s); the per-layer breakdown, the layerwise figures, the roofline of the
dominant call and the CPU-oracle baseline ride along.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

METRIC = "compacted decode-attn HBM GB/s + score/select/gather µs per layer, % roofline"
HBM_PEAK_GBPS = 8000.0
BF16_MFMA_PEAK_TFLOPS = 2500.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="llama3_8b_32k")
    ap.add_argument("--layers", type=int, default=0, help="0: all layers of the workload")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="budget of the CPU-oracle sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-retrieval", action="store_true",
                    help="skip the speculative-retrieval schedules on the batched ragged workload")
    ap.add_argument("--tsp", action="store_true",
                    help="also time the token-selective-propagation workload mha_tsp (64K-token MHA cache, "
                         "selection shared over heads at layer 16, later layers over the kept tokens)")
    ap.add_argument("--copy-probe", action="store_true",
                    help="also run one plain 1 GiB device copy (for scaling PMC byte counters)")
    return ap.parse_args()


def measured_traffic(workload, layers, full_layers):
    """HBM bytes of one folded kvc_score_window call, from the committed PMC summary
    (rocprofv3 FETCH_SIZE / WRITE_SIZE, calibrated on a 1 GiB copy), or None when the
    score sources changed since those counters were taken or the shape differs."""
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles", "hbm_traffic_%s.md" % workload)
    if layers != full_layers or not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        if ":" in line:
            key, _, val = line.partition(":")
            fields[key.strip()] = val.strip()
    try:
        want = fields["score_sources_sha256"]
        srcs = fields["score_sources"].split()
        nbytes = int(fields["score_call_traffic_bytes"])
    except (KeyError, ValueError):
        return None
    h = hashlib.sha256()
    root = os.path.dirname(os.path.abspath(__file__))
    for src in srcs:
        with open(os.path.join(root, src), "rb") as fh:
            h.update(fh.read())
    return nbytes if h.hexdigest() == want else None


def layer_bytes(wl, S, cap):
    """Algorithmic bytes per layer and step (what the method itself must move)."""
    b = wl.elem_bytes
    units = wl.batch * wl.n_kv
    R = wl.group * wl.w
    r = wl.group
    score = units * (S * wl.d_h * b + R * wl.d_h * b + 2 * 4 * S)          # K once, Q, raw + pooled out
    select = units * ((S - wl.n_keep) * 4 + cap * 4 + 4)                    # pooled in, idx + count out
    gather = units * (2 * 2 * cap * wl.d_h * b + 4 * cap + 4 * cap)         # K,V rows read+write, idx, pos
    decode = units * (2 * cap * wl.d_h * b + 2 * r * wl.d_h * b + 4)        # Kc,Vc once, q in, out
    flops_score = units * 2 * R * S * wl.d_h                                # one Q K^T
    return dict(score=score, select=select, gather=gather, decode=decode, flops_score=flops_score)


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU: this path runs on a single MI355X and has no multi-GPU mode "
              "(requested --gpus %d)." % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch

    import oracle
    from sparse_decode_amd import kvc, synth
    from sparse_decode_amd.pipeline import LayerPath

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    kvc.lib()
    wl = synth.by_name(args.workload)
    L = args.layers or wl.layers
    B = wl.batch
    dev = torch.device("cuda")
    print("[bench] generating %s: %d layers" % (wl.name, L), file=sys.stderr, flush=True)
    # Every layer's cache lives in one tensor with the layers folded into the batch
    # ([L*B][n_kv][S][d_h]); a per-layer view is a contiguous slice of it.
    S, d, nh, nkv = wl.s_max, wl.d_h, wl.n_h, wl.n_kv
    K = torch.empty((L * B, nkv, S, d), dtype=wl.torch_dtype, device=dev)
    V = torch.empty_like(K)
    QW = torch.empty((L * B, nh, wl.w, d), dtype=wl.torch_dtype, device=dev)
    QD = torch.empty((L, B, nh, d), dtype=wl.torch_dtype, device=dev)
    seq_np = None
    for l in range(L):
        inp = synth.layer_inputs(wl, l, device=dev)
        K[l * B:(l + 1) * B].copy_(inp["k"])
        V[l * B:(l + 1) * B].copy_(inp["v"])
        QW[l * B:(l + 1) * B].copy_(inp["q_win"])
        QD[l].copy_(inp["q_dec"])
        seq_np = inp["seq_lens"]
        del inp
    torch.cuda.synchronize()
    sl_layer = torch.from_numpy(seq_np).to(dev)
    sl_all = torch.from_numpy(np.tile(seq_np, L)).to(dev)
    layers = [dict(q_win=QW[l * B:(l + 1) * B], k=K[l * B:(l + 1) * B], v=V[l * B:(l + 1) * B], q_dec=QD[l],
                   seq_lens=seq_np, seq_lens_dev=sl_layer) for l in range(L)]

    path = LayerPath(wl, device=dev)                    # one layer per call, buffers reused by every layer
    fold = LayerPath(wl, device=dev, batch=L * B)       # every layer in one call (layers folded into the batch)
    cap = path.cap
    mean_S = float(np.mean(seq_np))
    by = layer_bytes(wl, mean_S, cap)
    step_bytes = L * (by["score"] + by["select"] + by["gather"] + by["decode"])
    outs = torch.empty((L, B, nh, d), dtype=wl.torch_dtype, device=dev)
    lses = torch.empty((L, B, nh), dtype=torch.float32, device=dev)

    def decode_layer(l):
        sl = slice(l * B, (l + 1) * B)
        kvc.decode_attn(QD[l], fold.kc[sl], fold.vc[sl], fold.count[sl], out=outs[l], lse=lses[l],
                        ws=fold.ws_decode)

    def step_folded():
        fold.score(QW, K, sl_all)
        fold.select(sl_all)
        fold.gather(K, V)
        for l in range(L):
            decode_layer(l)

    def step_per_layer():
        for inp in layers:
            path.run(inp["q_win"], inp["k"], inp["v"], inp["q_dec"], inp["seq_lens_dev"])

    folded_calls = {
        "score": lambda: fold.score(QW, K, sl_all),
        "select": lambda: fold.select(sl_all),
        "gather": lambda: fold.gather(K, V),
        "decode": lambda: [decode_layer(l) for l in range(L)],
    }
    layer_calls = {
        "score": lambda inp: path.score(inp["q_win"], inp["k"], inp["seq_lens_dev"]),
        "select": lambda inp: path.select(inp["seq_lens_dev"]),
        "gather": lambda inp: path.gather(inp["k"], inp["v"]),
        "decode": lambda inp: path.decode(inp["q_dec"]),
    }
    names = tuple(layer_calls)

    # Capture every timed sequence as a HIP graph: a serving loop replays the step
    # rather than paying a Python launch per kernel.
    def capture(fn):
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            fn()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            fn()
        torch.cuda.synchronize()
        return g

    step_folded()                       # fills fold.kc/vc/count before the decode graph is captured
    torch.cuda.synchronize()
    g_step = capture(step_folded)
    g_layer_step = capture(step_per_layer)
    g_fold = {n: capture(folded_calls[n]) for n in names}
    g_call = {n: capture(lambda n=n: [layer_calls[n](inp) for inp in layers]) for n in names}

    def timed(fn, reps):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps       # ms

    # ---------------------------------------------------------------- timed region: whole steps
    for _ in range(args.warmup):
        g_step.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ms_per_step = timed(g_step.replay, args.steps)
    wall = time.perf_counter() - t0
    print("[bench] %d steps: %.3f ms/step (wall %.3f s)" % (args.steps, ms_per_step, wall), file=sys.stderr, flush=True)

    # ---------------------------------------------------------------- breakdowns (graphs, HIP events)
    g_layer_step.replay()
    ms_per_step_layerwise = timed(g_layer_step.replay, args.steps)
    us = {}              # folded: one call over all layers, per layer
    us_layer = {}        # one call per layer
    for n in names:
        g_fold[n].replay()
        us[n] = 1000.0 * timed(g_fold[n].replay, args.steps) / L
        g_call[n].replay()
        us_layer[n] = 1000.0 * timed(g_call[n].replay, args.steps) / L
    eager_ms = timed(step_folded, max(1, args.steps // 4))

    # one decode call over every layer's compacted cache (the layers folded into the
    # batch: the shape of a batch-L decode step of one layer), against the per-layer calls
    def decode_all():
        kvc.decode_attn(QD.view(L * B, nh, d), fold.kc, fold.vc, fold.count, out=outs.view(L * B, nh, d),
                        lse=lses.view(L * B, nh), ws=fold.ws_decode)
    g_dec_all = capture(decode_all)
    g_dec_all.replay()
    dec_all_us = 1000.0 * timed(g_dec_all.replay, args.steps)
    del g_dec_all

    # plain device copy of 1 GiB (torch's copy kernel): the bandwidth a read + write stream
    # reaches on this device, as context for the HBM fractions
    cp_a = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    cp_b = torch.empty_like(cp_a)
    cp_b.copy_(cp_a)
    copy_ms = timed(lambda: cp_b.copy_(cp_a), 5)
    copy_gbps = 2.0 * (1 << 30) / (copy_ms * 1e-3) / 1e9
    del cp_a, cp_b

    if args.copy_probe:
        a = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        bcp = torch.empty_like(a)
        bcp.copy_(a)
        torch.cuda.synchronize()
        del a, bcp

    # ---------------------------------------------------------------- CPU oracle baseline (sampled)
    cpu = None
    if not args.no_cpu_baseline:
        threads = oracle.set_threads(0)
        t_cpu, done = 0.0, 0
        for inp in layers:
            q = synth.to_host_f32(inp["q_win"])
            k = synth.to_host_f32(inp["k"])
            v = synth.to_host_f32(inp["v"])
            qd = synth.to_host_f32(inp["q_dec"])
            sl = inp["seq_lens"]
            c0 = time.perf_counter()
            _, pooled = oracle.score_window(q, k, wl.w, seq_lens=sl, window_in_cache=wl.window_in_cache,
                                            n_keep=wl.n_keep, pool=wl.pool)
            idx, cnt = oracle.select_topk(pooled, wl.k, wl.n_keep, seq_lens=sl)
            kc, _ = oracle.gather(k, idx, cnt)
            vc, _ = oracle.gather(v, idx, cnt)
            oracle.decode(qd, kc, vc, cnt)
            t_cpu += time.perf_counter() - c0
            done += 1
            if t_cpu >= args.cpu_seconds:
                break
        lb = by["score"] + by["select"] + by["gather"] + by["decode"]
        cpu = {"value": round(done * lb / t_cpu / 1e9, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
               "sample": "%d of %d layers of %s, all four steps, plain fp64 C oracle (OpenMP), %.1f s" % (
                   done, L, wl.name, t_cpu),
               "ms_per_layer": round(1000.0 * t_cpu / done, 2)}

    gbps = {n: by[n] / (us[n] * 1e-6) / 1e9 for n in names}
    gbps_layer = {n: by[n] / (us_layer[n] * 1e-6) / 1e9 for n in names}
    dominant = max(names, key=lambda n: us[n])
    kern = {"score": "kvc_score_window", "select": "kvc_select_topk", "gather": "kvc_gather_compact",
            "decode": "kvc_decode_attn"}
    traffic = measured_traffic(wl.name, L, wl.layers) if dominant == "score" else None
    roof = {"bound": "hbm", "achieved": round(gbps[dominant], 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
            "frac": round(gbps[dominant] / HBM_PEAK_GBPS, 4), "traffic": traffic,
            "kernel": "%s (one call over all %d layers)" % (kern[dominant], L) if dominant != "decode" else
                      "kvc_decode_attn (one call per layer)",
            "bytes_per_launch": int(by[dominant] * (L if dominant != "decode" else 1)),
            "us_per_launch": round(us[dominant] * (L if dominant != "decode" else 1), 3)}
    value = step_bytes / (ms_per_step * 1e-3) / 1e9
    res = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic (seeded N(0,1) Q/K/V with planted heavy hitters; no model weights)",
        "config": {"workload": wl.name, "layers": L, "batch": wl.batch, "seq_len": S, "n_h": wl.n_h,
                   "n_kv": wl.n_kv, "d_h": wl.d_h, "w": wl.w, "pool": wl.pool, "k": wl.k, "n_keep": wl.n_keep,
                   "schedule": "score/select/gather: one call over all layers; decode: one call per layer"},
        "roofline": roof,
        "cpu_baseline": cpu,
        "per_layer_us": {n: round(us[n], 3) for n in names},
        "per_layer_GBps": {n: round(gbps[n], 1) for n in names},
        "per_layer_hbm_frac": {n: round(gbps[n] / HBM_PEAK_GBPS, 4) for n in names},
        "layerwise": {"ms_per_step": round(ms_per_step_layerwise, 4),
                      "value": round(step_bytes / (ms_per_step_layerwise * 1e-3) / 1e9, 2),
                      "per_call_us": {n: round(us_layer[n], 3) for n in names},
                      "per_call_GBps": {n: round(gbps_layer[n], 1) for n in names}},
        "eager_ms_per_step": round(eager_ms, 4),
        "timing": "HIP graph replays between HIP events on the launch stream",
        "score_mfma_frac_algorithmic": round(by["flops_score"] / (us["score"] * 1e-6) / 1e12 / BF16_MFMA_PEAK_TFLOPS, 4),
        "decode_all_layers_one_call": {
            "us": round(dec_all_us, 3), "GBps": round(L * by["decode"] / (dec_all_us * 1e-6) / 1e9, 1),
            "hbm_frac": round(L * by["decode"] / (dec_all_us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4),
            "note": "kvc_decode_attn over the %d layers' compacted caches folded into the batch (%d sequences x %d "
                    "KV heads): the kernel at a batch-%d decode's size; per_layer_us.decode is the one-layer call"
                    % (L, L * B, nkv, L * B)},
        "copy_probe": {"GBps": round(copy_gbps, 1), "frac_of_peak": round(copy_gbps / HBM_PEAK_GBPS, 4),
                       "what": "torch device copy of 1 GiB, read + write bytes / time (HIP events, 5 copies)"},
        "per_layer_frac_of_copy": {n: round(gbps[n] / copy_gbps, 4) for n in names},
        "wall_s_timed_region": round(wall, 3),
    }
    if not args.no_retrieval:
        print("[bench] per-layer budgets", file=sys.stderr, flush=True)
        del g_step, g_layer_step, g_fold, g_call
        res["pyramid_budgets"] = measure_pyramid(wl, L, B, QW, K, V, QD, sl_all, dev, args.steps)
        print("[bench] role-based retention", file=sys.stderr, flush=True)
        res["core_retention"] = measure_core(wl, fold, sl_all, us["select"], dev, args.steps)
        print("[bench] speculative retrieval on ragged_b16", file=sys.stderr, flush=True)
        res["speculative_retrieval"] = measure_retrieval(dev, 64, 5)
    if args.tsp:
        print("[bench] token-selective propagation on mha_tsp", file=sys.stderr, flush=True)
        res["tsp"] = measure_tsp(dev, args.steps)
    print(json.dumps(res), flush=True)


RETRIEVAL_TAU = 0.85
BLOCK_TOKENS = 16
PYRAMID_BETA = 0.5
CORE_BLOCK, CORE_FRAC = 64, 0.05


def measure_tsp(dev, steps):
    """FastKV's token-selective propagation on mha_tsp (B=2, 32 MHA heads, S=65536): one
    decode-step's compression schedule layer by layer, since the layers after the TSP
    layer run over its selection.  Layers 0-16 run score -> select -> gather -> decode
    over S tokens; at layer 16 one selection per sequence from the head-summed scores
    (20 % of S, plus the window) gathers the hidden states; layers 17-31 run over the
    S' = 13108 + 32 kept tokens with their original positions.  Every layer at S reuses
    one layer's 2 x 1 GiB of K/V (each far above the 256 MB MALL), likewise at S'."""
    import torch

    from sparse_decode_amd import kvc, synth
    from sparse_decode_amd.pipeline import LayerPath, TspStep
    wl = synth.by_name("mha_tsp")
    k_tsp = synth.budget_from_rate(wl.tsp_rate, wl.s_max)
    s2 = k_tsp + wl.n_keep
    full = synth.layer_inputs(wl, 0, device=dev)
    late = synth.layer_inputs(wl, wl.tsp_layer + 1, device=dev, s_max=s2)
    hidden = synth.hidden_states(wl, device=dev)
    sl = torch.from_numpy(full["seq_lens"]).to(dev)
    sl2 = torch.from_numpy(late["seq_lens"]).to(dev)
    path = LayerPath(wl, device=dev)
    path2 = LayerPath(wl, device=dev, s_max=s2)
    tsp = TspStep(wl, k_tsp, device=dev)
    src_pos = torch.zeros((wl.batch, s2), dtype=torch.int32, device=dev)

    def full_layer():
        path.run(full["q_win"], full["k"], full["v"], full["q_dec"], sl)

    def tsp_step():
        tsp.run(path.pooled, hidden)
        src_pos.copy_(tsp.pos[:, 0, :])

    def late_layer():
        path2.run(late["q_win"], late["k"], late["v"], late["q_dec"], sl2, src_pos=src_pos)

    def step():
        for _ in range(wl.tsp_layer + 1):
            full_layer()
        tsp_step()
        for _ in range(wl.tsp_layer + 1, wl.layers):
            late_layer()

    def capture(fn):
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            fn()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            fn()
        torch.cuda.synchronize()
        return g

    def timed(g, reps):
        g.replay()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    full_layer()
    tsp_step()
    torch.cuda.synchronize()
    ms_step = timed(capture(step), max(2, steps // 2))
    us_full = 1000.0 * timed(capture(full_layer), steps)
    us_tsp = 1000.0 * timed(capture(tsp_step), steps)
    us_late = 1000.0 * timed(capture(late_layer), steps)
    by_full = layer_bytes(wl, float(np.mean(full["seq_lens"])), path.cap)
    by_late = layer_bytes(wl, float(np.mean(late["seq_lens"])), path2.cap)
    lb_full = by_full["score"] + by_full["select"] + by_full["gather"] + by_full["decode"]
    lb_late = by_late["score"] + by_late["select"] + by_late["gather"] + by_late["decode"]
    # TSP: head-summed scores read once, kept hidden rows read and written, idx / pos
    tsp_bytes = wl.batch * (wl.n_kv * wl.s_max * 4 + 2 * s2 * wl.hidden * wl.elem_bytes + 3 * 4 * s2)
    step_bytes = (wl.tsp_layer + 1) * lb_full + tsp_bytes + (wl.layers - wl.tsp_layer - 1) * lb_late
    del full, late, hidden
    return {"workload": wl.name, "layers": wl.layers, "tsp_layer": wl.tsp_layer, "k_tsp": k_tsp, "s_after": s2,
            "k_per_layer": wl.k, "ms_per_step": round(ms_step, 4),
            "value_GBps": round(step_bytes / (ms_step * 1e-3) / 1e9, 1),
            "us_per_layer_at_S": round(us_full, 2), "us_tsp_select_and_hidden_gather": round(us_tsp, 2),
            "us_per_layer_after": round(us_late, 2),
            "tsp_GBps": round(tsp_bytes / (us_tsp * 1e-6) / 1e9, 1),
            "timing": "HIP graph per schedule (whole step, one layer at S, the TSP step, one later layer), "
                      "replays between HIP events"}


def measure_core(wl, fold, sl_all, select_us, dev, steps):
    """Role-based retention (CASK core/scratch) over every layer in one call: the pooled
    scores of the folded step, a seeded role mask (5 % of the candidates, in 64-token
    blocks, are core), budget k over the scratch tokens; against the plain selection."""
    import torch

    from sparse_decode_amd import kvc
    LB, nkv, S = fold.pooled.shape
    rng = np.random.Generator(np.random.PCG64([wl.cfg_id, 0x636f7265]))
    nblk = (S - wl.n_keep) // CORE_BLOCK
    core = np.zeros((LB, S), np.uint8)
    for r in range(LB):
        for blk in rng.choice(nblk, int(round(CORE_FRAC * nblk)), replace=False):
            core[r, blk * CORE_BLOCK:(blk + 1) * CORE_BLOCK] = 1
    core_dev = torch.from_numpy(core).to(dev)
    core_cap = int(core.sum(axis=1).max())
    cap = wl.k + core_cap + wl.n_keep
    idx = torch.empty((LB, nkv, cap), dtype=torch.int32, device=dev)
    cnt = torch.empty((LB, nkv), dtype=torch.int32, device=dev)
    dims = kvc.make_dims(LB, S, nkv, nkv, 128, kvc.KVC_F32)
    ws = torch.zeros(kvc.select_core_workspace(dims, wl.n_keep), dtype=torch.uint8, device=dev)

    def call():
        kvc.select_core(fold.pooled, core_dev, wl.k, core_cap, wl.n_keep, seq_lens=sl_all, idx=idx, count=cnt,
                        ws=ws)

    call()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    us = 1000.0 * e0.elapsed_time(e1) / steps / (LB // wl.batch)
    del g
    return {"core_frac": CORE_FRAC, "core_block": CORE_BLOCK, "core_tokens_per_seq": int(core.sum(axis=1).mean()),
            "k_scratch": wl.k, "mean_kept": round(float(cnt.float().mean()), 1),
            "us_per_layer": round(us, 3), "plain_select_us_per_layer": round(select_us, 3)}


def measure_pyramid(wl, L, B, QW, K, V, QD, sl_all, dev, steps):
    """The folded step with per-layer budgets (PyramidKV-style, mean budget k): layer l
    keeps pyramid_budgets(k, L)[l] + n_keep tokens per KV head; one select call over all
    layers takes the budgets as a per-unit array."""
    import torch

    from sparse_decode_amd import kvc, synth
    from sparse_decode_amd.pipeline import LayerPath
    budgets = synth.pyramid_budgets(wl.k, L, PYRAMID_BETA)
    kmax = max(budgets)
    path = LayerPath(wl, device=dev, batch=L * B, k=kmax)
    # unit (l * B + b, g) takes layer l's budget
    kpu = (torch.tensor(budgets, dtype=torch.int32, device=dev).repeat_interleave(B)[:, None]
           .expand(L * B, wl.n_kv).contiguous())
    outs = torch.empty((L, B, wl.n_h, wl.d_h), dtype=wl.torch_dtype, device=dev)

    def step():
        path.score(QW, K, sl_all)
        path.select(sl_all, k_per_unit=kpu)
        path.gather(K, V)
        for l in range(L):
            sl = slice(l * B, (l + 1) * B)
            kvc.decode_attn(QD[l], path.kc[sl], path.vc[sl], path.count[sl], out=outs[l], ws=path.ws_decode)

    step()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    mean_S = float(np.mean(sl_all.cpu().numpy()))
    nbytes = 0.0
    for l in range(L):
        by = layer_bytes(wl, mean_S, budgets[l] + wl.n_keep)
        nbytes += by["score"] + by["select"] + by["gather"] + by["decode"]
    del g
    return {"schedule": "linear from (1+beta) k to (1-beta) k over the layers, mean k", "beta": PYRAMID_BETA,
            "k_first_layer": budgets[0], "k_last_layer": budgets[-1], "k_mean": round(sum(budgets) / L, 2),
            "ms_per_step": round(ms, 4), "value_GBps": round(nbytes / (ms * 1e-3) / 1e9, 2)}


def measure_retrieval(dev, steps, reps):
    """Speculative retrieval with fine-grained correction (FreeKV technical summary
    2.A) on the batched ragged decode workload (16 sequences of 4096..16384 cached
    tokens, 32/8 heads, one query per step that re-scores the cache, k = 512 + 32).

    Three schedules of the same `steps` decode steps, each captured as one HIP graph:
      reselect     score -> select -> gather -> attention of every head, every step
      critical     what attention waits for under speculation: query similarity,
                   correction (score/select/gather of the drifted KV heads only), then
                   attention over the previous step's selection for the other heads
      overlapped   critical on the launch stream and the speculative selection for the
                   next step on a second stream beside it
      blocks       landmark-guided block selection (xKV 2.3): block scores from the block
                   landmarks (built once, timed apart), top k/16 blocks of 16 tokens,
                   their tokens gathered, attention
    """
    import torch

    from sparse_decode_amd import synth
    from sparse_decode_amd.pipeline import BlockRetrieval, LayerPath, SpeculativeRetrieval
    wl = synth.by_name("ragged_b16")
    inp = synth.layer_inputs(wl, 0, device=dev, step=0)
    k, v = inp["k"], inp["v"]
    sl = torch.from_numpy(inp["seq_lens"]).to(dev)
    qs = [synth.step_query(wl, 0, i, device=dev) for i in range(steps)]
    B, nh, d = qs[0].shape
    base = LayerPath(wl, device=dev)
    spec = SpeculativeRetrieval(wl, RETRIEVAL_TAU, device=dev)
    blk = BlockRetrieval(wl, BLOCK_TOKENS, wl.k // BLOCK_TOKENS, device=dev)

    def blocks():
        for q in qs:
            blk.step(q, k, v, sl)

    def landmarks():
        blk.prepare(k, sl)

    def reselect():
        for q in qs:
            base.score(q.view(B, nh, 1, d), k, sl)
            base.select(sl)
            base.gather(k, v)
            base.decode(q)

    def critical():
        spec.cur = 0
        for i, q in enumerate(qs):
            spec.critical(q, qs[i - 1] if i else None, k, v, sl)
            spec.swap()

    def overlapped():
        spec.cur = 0
        main = torch.cuda.current_stream()
        side = torch.cuda.Stream()
        side.wait_stream(main)
        e_c, e_s = None, None
        for i, q in enumerate(qs):
            if e_s is not None:
                main.wait_event(e_s)
            spec.critical(q, qs[i - 1] if i else None, k, v, sl)
            e_prev_c, e_c = e_c, torch.cuda.Event()
            e_c.record(main)
            with torch.cuda.stream(side):
                if e_prev_c is not None:
                    side.wait_event(e_prev_c)
                spec.speculate(q, k, v, sl)
                e_s = torch.cuda.Event()
                e_s.record(side)
            spec.swap()
        main.wait_stream(side)

    # corrected fraction: one eager pass of the sequential schedule
    spec.cur = 0
    corrected = []
    for i, q in enumerate(qs):
        spec.critical(q, qs[i - 1] if i else None, k, v, sl)
        if i:
            corrected.append(spec.refresh.float().mean())
        spec.speculate(q, k, v, sl)
        spec.swap()
    frac = float(torch.stack(corrected).mean()) if corrected else 1.0

    def graph_of(fn):
        fn()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            fn()
        torch.cuda.synchronize()
        return g

    out = {}
    landmarks()
    for name, fn in (("reselect", reselect), ("critical", critical), ("overlapped", overlapped),
                     ("blocks", blocks), ("landmarks_once", landmarks)):
        g = graph_of(fn)
        g.replay()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(reps):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        out[name] = 1000.0 * e0.elapsed_time(e1) / reps / (1 if name == "landmarks_once" else steps)
        del g
    return {"workload": wl.name, "steps": steps, "tau": RETRIEVAL_TAU,
            "corrected_kv_head_frac": round(frac, 4),
            "us_per_step": {n: round(t, 2) for n, t in out.items() if n in ("reselect", "critical", "overlapped")},
            "critical_path_speedup": round(out["reselect"] / out["critical"], 3),
            "block_selection": {"block": BLOCK_TOKENS, "k_blocks": wl.k // BLOCK_TOKENS,
                                "us_per_step": round(out["blocks"], 2),
                                "landmarks_us_once": round(out["landmarks_once"], 2),
                                "speedup_vs_reselect": round(out["reselect"] / out["blocks"], 3)},
            "step_speedup_overlapped": round(out["reselect"] / out["overlapped"], 3),
            "timing": "HIP graph of all steps per schedule, replayed between HIP events on the launch stream"}


if __name__ == "__main__":
    main()
