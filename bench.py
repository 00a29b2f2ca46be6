#!/usr/bin/env python3
"""Benchmark of the KV-cache compression hot path on one MI355X.

The headline workload is the largest one, ``mha_tsp``: B = 2 sequences of S = 65536
cached tokens, 32 MHA layers (n_h = n_kv = 32, d_h = 128, bf16) with every layer's
cache resident in HBM (about 41 GB).  A step is one decode step of FastKV's
layer-by-layer schedule over the whole model: layers 0-16 run window scoring ->
per-head top-k (k = 1024 + 32) -> compacting gather -> decode attention over all S
tokens; layer 16 also selects 20 % of the tokens for every head and gathers their
hidden states; layers 17-31 run over those 13140 tokens with their original
positions.

``value`` is the metric's first quantity: compacted decode-attention GB/s, the
algorithmic bytes of the 32 per-layer decode calls over their time, each layer
reading its own compacted cache, timed as one HIP graph per replay with the
memory-side cache (MALL) flushed by a 512 MiB write before every replay.  The other
calls are reported as µs per layer (cold, likewise) and as a fraction of the HBM
roofline; ``roofline`` describes the call that dominates the step.

The same JSON line carries one row per other workload (``configs``: the tiny fp32
layer, the 32-layer 32K and 128K caches, the batched ragged decode), each with µs
per step, µs per layer of the four calls, its roofline and the CPU oracle timed on
a sample of it; a sweep of the propagation layer and rate (``tsp_sweep``); and the
next rows built on the path (per-layer budgets, core retention, speculative and
block retrieval).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import sys
import time

import numpy as np

METRIC = "compacted decode-attn HBM GB/s + score/select/gather µs per layer, % roofline"
HBM_PEAK_GBPS = 8000.0
BF16_MFMA_PEAK_TFLOPS = 2500.0
FLUSH_BYTES = 512 << 20
TSP_LAYERS = (8, 12, 16, 20, 24)
TSP_RATES = (0.1, 0.2, 0.4)
CPU_SAMPLE_LAYERS = (0, 1, 15, 16, 17, 30, 31)
RETRIEVAL_TAU = 0.85
BLOCK_TOKENS = 16
PYRAMID_BETA = 0.5
CORE_BLOCK, CORE_FRAC = 64, 0.05
ROOT = os.path.dirname(os.path.abspath(__file__))
_ORACLE_THREADS = []


def oracle_threads():
    """The oracle's thread count (all host cores), set again before every sample."""
    import oracle
    if not _ORACLE_THREADS:
        _ORACLE_THREADS.append(oracle.set_threads(0))
    return oracle.set_threads(_ORACLE_THREADS[0])


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--reps", type=int, default=10, help="cold replays per breakdown timing (median)")
    ap.add_argument("--cpu-seconds", type=float, default=8.0,
                    help="budget of each workload's CPU-oracle sample beyond its fixed sampled layers")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--headline-only", action="store_true", help="skip the other workloads, sweep and next rows")
    ap.add_argument("--profile-call", choices=("score", "decode", "gather", "select"), default=None,
                    help="only replay one call of one headline layer (for rocprofv3 runs), then a 1 GiB elementwise kernel")
    ap.add_argument("--calls", type=int, default=10, help="replays of --profile-call")
    ap.add_argument("--only", choices=("tiny_fp32", "llama3_8b_32k", "ctx_128k", "ragged_b16"), default=None,
                    help="measure only this other workload and print its object (for rocprofv3 runs)")
    return ap.parse_args()


# ------------------------------------------------------------------------------ timing

def graph_of(fn):
    """Runs fn once on a side stream (warm-up, lazy allocations), then captures it."""
    import torch
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


class Flusher:
    """A 512 MiB device buffer whose fill evicts the memory-side cache before a timing."""

    def __init__(self, dev):
        import torch
        self.buf = torch.empty(FLUSH_BYTES // 4, dtype=torch.int32, device=dev)
        self.n = 0

    def __call__(self):
        self.n += 1
        self.buf.fill_(self.n)


def timed_cold(g, reps, flush):
    """Median ms of `reps` replays of graph g, the MALL flushed before each (HIP events
    on the launch stream around the replay only)."""
    import torch
    g.replay()
    torch.cuda.synchronize()
    pairs = []
    for _ in range(reps):
        flush()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        g.replay()
        e1.record()
        pairs.append((e0, e1))
    torch.cuda.synchronize()
    return float(np.median([a.elapsed_time(b) for a, b in pairs]))


def timed_steps(g, steps, warmup):
    """The contract's timed region: warmup untimed replays, then exactly `steps`
    back-to-back replays between HIP events, synchronised on both sides."""
    import torch
    for _ in range(warmup):
        g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    for _ in range(steps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps, time.perf_counter() - t0


# --------------------------------------------------------------------- algorithmic bytes

def layer_bytes(wl, S, cap):
    """Algorithmic bytes of one layer's four calls (what the method itself must move):
    score reads K once and the window queries and writes raw + pooled; select reads
    the candidates' scores and writes the kept indices; gather reads and writes the
    kept K and V rows and writes their positions (reading idx); decode reads the
    compacted K and V once, the queries, and writes the outputs."""
    b = wl.elem_bytes
    units = wl.batch * wl.n_kv
    R = wl.group * wl.w
    r = wl.group
    return dict(
        score=units * (S * wl.d_h * b + R * wl.d_h * b + 2 * 4 * S),
        select=units * ((S - wl.n_keep) * 4 + cap * 4 + 4),
        gather=units * (2 * 2 * cap * wl.d_h * b + 4 * cap + 4 * cap),
        decode=units * (2 * cap * wl.d_h * b + 2 * r * wl.d_h * b + 4),
        flops_score=units * 2 * R * S * wl.d_h)


def gbps(nbytes, us):
    return nbytes / (us * 1e-6) / 1e9


def roofline(name, nbytes, us, traffic=None, traffic_note=None, flops=None):
    a = gbps(nbytes, us)
    r = {"bound": "hbm", "achieved": round(a, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
         "frac": round(a / HBM_PEAK_GBPS, 4), "traffic": traffic, "kernel": name,
         "bytes_per_launch": int(nbytes), "us_per_launch": round(us, 3)}
    if traffic_note:
        r["traffic_source"] = traffic_note
    if flops:
        r["mfma_frac_algorithmic"] = round(flops / (us * 1e-6) / 1e12 / BF16_MFMA_PEAK_TFLOPS, 4)
    return r


def stored_traffic(workload):
    """HBM bytes per launch of the dominant call, from a committed rocprofv3 --pmc
    summary (FETCH_SIZE + WRITE_SIZE scaled by a copy of known size), or None when
    the kernel sources changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic_%s.md" % workload)
    if not os.path.exists(path):
        return None, None
    fields = {}
    for line in open(path):
        if ":" in line:
            key, _, val = line.partition(":")
            fields[key.strip()] = val.strip()
    try:
        want = fields["sources_sha256"]
        srcs = fields["sources"].split()
        nbytes = int(fields["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None, None
    h = hashlib.sha256()
    for src in srcs:
        with open(os.path.join(ROOT, src), "rb") as fh:
            h.update(fh.read())
    if h.hexdigest() != want:
        return None, "profiles/hbm_traffic_%s.md is stale (kernel sources changed): not reported" % workload
    return nbytes, ("stored: profiles/hbm_traffic_%s.md, two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE) of "
                    "this build's sources, scaled by a 1 GiB elementwise kernel" % workload)


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "unknown"


# ------------------------------------------------------------------------ CPU oracle

def oracle_layer(wl, q_win, k, v, q_dec, seq_lens, budget, src_pos=None):
    """The oracle's four steps on one layer (host arrays); returns seconds per step."""
    import oracle
    t = {}
    c0 = time.perf_counter()
    _, pooled = oracle.score_window(q_win, k, wl.w, seq_lens=seq_lens, window_in_cache=wl.window_in_cache,
                                    n_keep=wl.n_keep, pool=wl.pool)
    c1 = time.perf_counter()
    idx, cnt = oracle.select_topk(pooled, budget, wl.n_keep, seq_lens=seq_lens)
    c2 = time.perf_counter()
    kc, _ = oracle.gather(k, idx, cnt, src_pos=src_pos)
    vc, _ = oracle.gather(v, idx, cnt, src_pos=src_pos)
    c3 = time.perf_counter()
    oracle.decode(q_dec, kc, vc, cnt)
    c4 = time.perf_counter()
    t.update(score=c1 - c0, select=c2 - c1, gather=c3 - c2, decode=c4 - c3)
    return t, pooled


def cpu_summary(wl, times, by, sample, threads):
    """cpu_baseline object: oracle decode GB/s (the headline's quantity) plus ms per
    layer of every step, from per-layer step times."""
    n = len(times)
    med = {s: float(np.median([t[s] for t in times])) for s in ("score", "select", "gather", "decode")}
    return {"value": round(gbps(by["decode"], 1e6 * med["decode"]), 4), "unit": "GB/s", "cores": threads,
            "kind": "oracle", "sample": sample, "layers_timed": n,
            "ms_per_layer": {s: round(1e3 * v, 3) for s, v in med.items()},
            "ms_per_layer_all_steps": round(1e3 * sum(med.values()), 2),
            "what": "plain fp64 C oracle (OpenMP over units), median over the sampled layers; value = decode "
                    "bytes / oracle decode time"}


# ------------------------------------------------------------------------ headline: mha_tsp

def build_tsp_model(wl, dev, k_tsp, n_full, late_layers, late_distinct=None):
    """Per-layer inputs of the whole model: n_full distinct layers at S, then the later
    layers at S' = k_tsp + n_keep (late_distinct distinct caches, cycled)."""
    from sparse_decode_amd import synth
    s2 = k_tsp + wl.n_keep
    full = [synth.layer_inputs(wl, l, device=dev) for l in range(n_full)]
    nd = late_layers if late_distinct is None else min(late_distinct, late_layers)
    late = [synth.layer_inputs(wl, n_full + j, device=dev, s_max=s2) for j in range(nd)]
    return full, late


def strip(x):
    return {k: x[k] for k in ("q_win", "k", "v", "q_dec")}


def measure_headline(args, dev, flush):
    import torch

    from sparse_decode_amd import synth
    from sparse_decode_amd.pipeline import TspSchedule
    wl = synth.by_name("mha_tsp")
    L, T = wl.layers, wl.tsp_layer
    k_tsp = synth.budget_from_rate(wl.tsp_rate, wl.s_max)
    print("[bench] mha_tsp: generating the 32-layer cache", file=sys.stderr, flush=True)
    full, late = build_tsp_model(wl, dev, k_tsp, T + 1, L - T - 1)
    hidden = synth.hidden_states(wl, device=dev)
    seq_full = torch.from_numpy(full[0]["seq_lens"]).to(dev)
    seq_after = torch.from_numpy(late[0]["seq_lens"]).to(dev)
    layers = [strip(x) for x in full] + [strip(x) for x in late]
    sched = TspSchedule(wl, layers, T, k_tsp, seq_full, seq_after, hidden, device=dev)
    torch.cuda.synchronize()
    print("[bench] mha_tsp: resident cache %.1f GB" % (torch.cuda.memory_allocated() / 1e9), file=sys.stderr,
          flush=True)

    g_step = graph_of(sched.step)
    ms_step, wall = timed_steps(g_step, args.steps, args.warmup)
    print("[bench] mha_tsp: %d steps, %.3f ms/step" % (args.steps, ms_step), file=sys.stderr, flush=True)

    lf, la = list(range(T + 1)), list(range(T + 1, L))
    parts = {
        "score_at_S": lambda: [sched.score(l) for l in lf],
        "score_after": lambda: [sched.score(l) for l in la],
        "select_at_S": lambda: [sched.select(l) for l in lf],
        "select_after": lambda: [sched.select(l) for l in la],
        "gather_at_S": lambda: [sched.gather(l) for l in lf],
        "gather_after": lambda: [sched.gather(l) for l in la],
        "decode": lambda: [sched.decode(l) for l in range(L)],
        "tsp": sched.propagate,
    }
    us = {}
    for name, fn in parts.items():
        g = graph_of(fn)
        n = len(lf) if name.endswith("_at_S") else (len(la) if name.endswith("_after") else
                                                      (L if name == "decode" else 1))
        us[name] = 1000.0 * timed_cold(g, args.reps, flush) / n
        del g
    g_step.replay()
    torch.cuda.synchronize()

    by_S = layer_bytes(wl, wl.s_max, sched.full.cap)
    by_A = layer_bytes(wl, sched.s_after, sched.full.cap)
    tsp_bytes = wl.batch * (wl.n_kv * wl.s_max * 4 + 2 * sched.s_after * wl.hidden * wl.elem_bytes +
                            3 * 4 * sched.s_after)
    dec_bytes = by_S["decode"]                        # same cap and heads at every layer
    value = gbps(dec_bytes, us["decode"])
    step_bytes = (T + 1) * sum(by_S[c] for c in ("score", "select", "gather", "decode")) + tsp_bytes + \
        (L - T - 1) * sum(by_A[c] for c in ("score", "select", "gather", "decode"))
    traffic, note = stored_traffic(wl.name)
    roof = roofline("kvc_score_window, one layer at S = 65536 (64 KV heads, R = 32 rows each)", by_S["score"],
                    us["score_at_S"], traffic, note, flops=by_S["flops_score"])
    per_call = {
        "score": {"at_S": round(us["score_at_S"], 2), "after": round(us["score_after"], 2)},
        "select": {"at_S": round(us["select_at_S"], 2), "after": round(us["select_after"], 2)},
        "gather": {"at_S": round(us["gather_at_S"], 2), "after": round(us["gather_after"], 2)},
        "decode": round(us["decode"], 3),
        "tsp_select_and_hidden_gather": round(us["tsp"], 2),
    }
    per_gbps = {
        "score": {"at_S": round(gbps(by_S["score"], us["score_at_S"]), 1),
                  "after": round(gbps(by_A["score"], us["score_after"]), 1)},
        "select": {"at_S": round(gbps(by_S["select"], us["select_at_S"]), 1),
                   "after": round(gbps(by_A["select"], us["select_after"]), 1)},
        "gather": {"at_S": round(gbps(by_S["gather"], us["gather_at_S"]), 1),
                   "after": round(gbps(by_A["gather"], us["gather_after"]), 1)},
        "decode": round(value, 1),
        "tsp_select_and_hidden_gather": round(gbps(tsp_bytes, us["tsp"]), 1),
    }
    res = {
        "value": round(value, 2),
        "ms_per_step": round(ms_step, 4),
        "wall_s_timed_region": round(wall, 3),
        "config": {"workload": wl.name, "layers": L, "batch": wl.batch, "seq_len": wl.s_max, "n_h": wl.n_h,
                   "n_kv": wl.n_kv, "d_h": wl.d_h, "w": wl.w, "pool": wl.pool, "k": wl.k, "n_keep": wl.n_keep,
                   "tsp_layer": T, "tsp_rate": wl.tsp_rate, "k_tsp": k_tsp, "s_after_tsp": sched.s_after,
                   "hidden": wl.hidden,
                   "schedule": "layer by layer: score -> select -> gather -> decode per layer; shared selection "
                               "and hidden-state gather at the propagation layer; later layers over the kept "
                               "tokens"},
        "value_definition": "decode bytes of one layer (Kc and Vc read once, q in, out) / median cold time per "
                            "layer of the 32 per-layer kvc_decode_attn calls (one graph per replay, MALL "
                            "flushed by a 512 MiB write before each replay)",
        "roofline": roof,
        "per_layer_us": per_call,
        "per_layer_GBps": per_gbps,
        "per_layer_hbm_frac": {"decode": round(value / HBM_PEAK_GBPS, 4),
                               "score_at_S": round(gbps(by_S["score"], us["score_at_S"]) / HBM_PEAK_GBPS, 4),
                               "gather_at_S": round(gbps(by_S["gather"], us["gather_at_S"]) / HBM_PEAK_GBPS, 4)},
        "step_GBps_algorithmic": round(step_bytes / (ms_step * 1e-3) / 1e9, 1),
        "timing": "step: HIP-graph replays between HIP events on the launch stream; per-layer figures: one graph "
                  "per call type over the layers it runs on (each layer its own buffers), median of %d cold "
                  "replays" % args.reps,
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_headline(wl, sched, full, late, hidden, k_tsp, by_S, args)
    ctx = {"wl": wl, "full": full, "hidden": hidden, "seq_full": seq_full}
    del sched, g_step, late, layers
    return res, ctx


def cpu_headline(wl, sched, full, late, hidden, k_tsp, by_S, args):
    """The oracle on the sampled layers of the headline step (their own inputs), and
    the propagation at layer 16: its shared selection and hidden-state gather."""
    import torch

    import oracle
    from sparse_decode_amd import synth
    threads = oracle_threads()
    times, t_tsp, T = [], None, wl.tsp_layer
    src_pos = sched.src_pos.cpu().numpy().astype(np.int32)
    for l in CPU_SAMPLE_LAYERS:
        x = full[l] if l <= T else late[(l - T - 1) % len(late)]
        h = {n: synth.to_host_f32(x[n]) for n in ("q_win", "k", "v", "q_dec")}
        t, pooled = oracle_layer(wl, h["q_win"], h["k"], h["v"], h["q_dec"], x["seq_lens"], wl.k,
                                 src_pos=None if l <= T else src_pos)
        times.append(t)
        if l == T:
            hb = hidden.view(torch.int16).cpu().numpy().reshape(wl.batch, 1, wl.s_max, wl.hidden)
            c0 = time.perf_counter()
            idx, cnt = oracle.select_topk(pooled, k_tsp, wl.n_keep, seq_lens=x["seq_lens"], shared_heads=True)
            oracle.gather(hb, idx, cnt)
            t_tsp = time.perf_counter() - c0
            del hb
        del h, pooled
    s = cpu_summary(wl, times, by_S, "layers %s of mha_tsp (their own inputs; layers 17-31 over the 13140 "
                    "propagated tokens) and the propagation at layer 16" % (list(CPU_SAMPLE_LAYERS),), threads)
    s["ms_tsp_select_and_hidden_gather"] = round(1e3 * t_tsp, 2)
    s["cpu_model"] = cpu_model()
    return s


# ------------------------------------------------------------- TSP sweep (FastKV 2.A/2.B)

def measure_tsp_sweep(args, dev, flush, ctx):
    """The headline step with the propagation layer in {8, 12, 16, 20, 24} and the TSP
    rate in {0.1, 0.2, 0.4} (independent of the per-layer budget k = 1024).  Layers
    at S cycle over the 17 distinct caches of the headline model (1 GiB of K each, far
    above the MALL); later layers over 8 distinct caches of S' tokens per rate."""
    import torch

    from sparse_decode_amd import synth
    from sparse_decode_amd.pipeline import TspSchedule
    wl, full = ctx["wl"], ctx["full"]
    out = {"layers": list(TSP_LAYERS), "rates": list(TSP_RATES), "points": []}
    for rate in TSP_RATES:
        k_tsp = synth.budget_from_rate(rate, wl.s_max)
        s2 = k_tsp + wl.n_keep
        late = [synth.layer_inputs(wl, 100 + j, device=dev, s_max=s2) for j in range(8)]
        seq_after = torch.from_numpy(late[0]["seq_lens"]).to(dev)
        for T in TSP_LAYERS:
            layers = [strip(full[l % len(full)]) for l in range(T + 1)] + \
                     [strip(late[j % len(late)]) for j in range(wl.layers - T - 1)]
            sched = TspSchedule(wl, layers, T, k_tsp, ctx["seq_full"], seq_after, ctx["hidden"], device=dev)
            g = graph_of(sched.step)
            ms = timed_cold(g, 3, flush)
            by_S = layer_bytes(wl, wl.s_max, sched.full.cap)
            by_A = layer_bytes(wl, s2, sched.full.cap)
            nb = (T + 1) * sum(by_S[c] for c in ("score", "select", "gather", "decode")) + \
                (wl.layers - T - 1) * sum(by_A[c] for c in ("score", "select", "gather", "decode"))
            out["points"].append({"tsp_layer": T, "tsp_rate": rate, "k_tsp": k_tsp, "s_after": s2,
                                  "ms_per_step": round(ms, 4), "GBps_algorithmic": round(nb / (ms * 1e-3) / 1e9, 1)})
            print("[bench] tsp sweep layer %d rate %.1f: %.3f ms" % (T, rate, ms), file=sys.stderr, flush=True)
            del g, sched, layers
        del late
        torch.cuda.empty_cache()
    out["timing"] = "one HIP graph per step, median of 3 cold replays"
    return out


# ------------------------------------------------------- 32-layer caches: one call over all layers

def measure_folded(name, args, dev, flush, extras=False):
    """A whole model's cache compressed with one call each of score, select and gather
    over all layers (the layers folded into the batch), then one decode call per layer;
    and the same step with one call per layer for every part (layerwise)."""
    import torch

    import oracle
    from sparse_decode_amd import kvc, synth
    from sparse_decode_amd.pipeline import LayerPath
    wl = synth.by_name(name)
    L, B = wl.layers, wl.batch
    S, d, nh, nkv = wl.s_max, wl.d_h, wl.n_h, wl.n_kv
    print("[bench] %s: generating %d layers" % (name, L), file=sys.stderr, flush=True)
    K = torch.empty((L * B, nkv, S, d), dtype=wl.torch_dtype, device=dev)
    V = torch.empty_like(K)
    QW = torch.empty((L * B, nh, wl.w, d), dtype=wl.torch_dtype, device=dev)
    QD = torch.empty((L, B, nh, d), dtype=wl.torch_dtype, device=dev)
    seq_np = None
    for l in range(L):
        x = synth.layer_inputs(wl, l, device=dev)
        K[l * B:(l + 1) * B].copy_(x["k"])
        V[l * B:(l + 1) * B].copy_(x["v"])
        QW[l * B:(l + 1) * B].copy_(x["q_win"])
        QD[l].copy_(x["q_dec"])
        seq_np = x["seq_lens"]
        del x
    sl_layer = torch.from_numpy(seq_np).to(dev)
    sl_all = torch.from_numpy(np.tile(seq_np, L)).to(dev)
    fold = LayerPath(wl, device=dev, batch=L * B)
    path = LayerPath(wl, device=dev)
    cap = fold.cap
    outs = torch.empty((L, B, nh, d), dtype=wl.torch_dtype, device=dev)
    lses = torch.empty((L, B, nh), dtype=torch.float32, device=dev)
    views = [dict(q_win=QW[l * B:(l + 1) * B], k=K[l * B:(l + 1) * B], v=V[l * B:(l + 1) * B], q_dec=QD[l])
             for l in range(L)]

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

    def step_layerwise():
        for x in views:
            path.run(x["q_win"], x["k"], x["v"], x["q_dec"], sl_layer)

    g = graph_of(step_folded)
    ms_step, _ = timed_steps(g, args.steps, args.warmup)
    del g
    g = graph_of(step_layerwise)
    ms_layerwise, _ = timed_steps(g, max(2, args.steps // 2), 1)
    del g
    folded = {"score": lambda: fold.score(QW, K, sl_all), "select": lambda: fold.select(sl_all),
              "gather": lambda: fold.gather(K, V), "decode": lambda: [decode_layer(l) for l in range(L)]}
    layerwise = {"score": lambda: [path.score(x["q_win"], x["k"], sl_layer) for x in views],
                 "select": lambda: [path.select(sl_layer) for _ in views],
                 "gather": lambda: [path.gather(x["k"], x["v"]) for x in views],
                 "decode": lambda: [path.decode(x["q_dec"]) for x in views]}
    us, us_lw = {}, {}
    for c in ("score", "select", "gather", "decode"):
        g = graph_of(folded[c])
        us[c] = 1000.0 * timed_cold(g, args.reps, flush) / L
        del g
        g = graph_of(layerwise[c])
        us_lw[c] = 1000.0 * timed_cold(g, args.reps, flush) / L
        del g
    step_folded()
    torch.cuda.synchronize()
    by = layer_bytes(wl, float(np.mean(seq_np)), cap)
    traffic, note = stored_traffic(name) if name != "mha_tsp" else (None, None)
    row = {
        "workload": name, "layers": L, "batch": B, "seq_len": S, "n_h": nh, "n_kv": nkv, "d_h": d, "w": wl.w,
        "pool": wl.pool, "k": wl.k, "n_keep": wl.n_keep,
        "ms_per_step": round(ms_step, 4),
        "schedule": "score/select/gather: one call over all layers; decode: one call per layer",
        "per_layer_us": {c: round(v, 3) for c, v in us.items()},
        "per_layer_GBps": {c: round(gbps(by[c], us[c]), 1) for c in us},
        "per_layer_hbm_frac": {c: round(gbps(by[c], us[c]) / HBM_PEAK_GBPS, 4) for c in us},
        "decode_GBps": round(gbps(by["decode"], us["decode"]), 1),
        "layerwise": {"ms_per_step": round(ms_layerwise, 4),
                      "per_call_us": {c: round(v, 3) for c, v in us_lw.items()},
                      "per_call_GBps": {c: round(gbps(by[c], us_lw[c]), 1) for c in us_lw}},
        "roofline": roofline("kvc_score_window, one call over all %d layers" % L, L * by["score"], L * us["score"],
                             traffic, note, flops=L * by["flops_score"]),
        "timing": "per-layer figures: one graph per call type, median of %d cold replays (MALL flushed)" % args.reps,
    }

    def decode_all():
        kvc.decode_attn(QD.view(L * B, nh, d), fold.kc, fold.vc, fold.count, out=outs.view(L * B, nh, d),
                        lse=lses.view(L * B, nh), ws=fold.ws_decode)
    g = graph_of(decode_all)
    dec_all = 1000.0 * timed_cold(g, args.reps, flush)
    del g
    row["decode_all_layers_one_call"] = {
        "us": round(dec_all, 3), "GBps": round(gbps(L * by["decode"], dec_all), 1),
        "hbm_frac": round(gbps(L * by["decode"], dec_all) / HBM_PEAK_GBPS, 4),
        "what": "kvc_decode_attn over the %d layers' compacted caches folded into the batch (the kernel at a "
                "batch-%d decode's size)" % (L, L * B)}
    if extras:
        print("[bench] %s: per-layer budgets, core retention" % name, file=sys.stderr, flush=True)
        row["pyramid_budgets"] = measure_pyramid(wl, L, B, QW, K, V, QD, sl_all, dev, args)
        row["core_retention"] = measure_core(wl, fold, sl_all, us["select"], dev, args, flush)
    if not args.no_cpu_baseline:
        threads = oracle_threads()
        sample = CPU_SAMPLE_LAYERS if name == "ctx_128k" else tuple(range(L))
        times, t_used, t1 = [], 0.0, None
        for l in sample:
            h = {n: synth.to_host_f32(views[l][n]) for n in ("q_win", "k", "v", "q_dec")}
            t, _ = oracle_layer(wl, h["q_win"], h["k"], h["v"], h["q_dec"], seq_np, wl.k)
            times.append(t)
            t_used += sum(t.values())
            if name == "llama3_8b_32k" and t1 is None:
                oracle.set_threads(1)
                t1, _ = oracle_layer(wl, h["q_win"], h["k"], h["v"], h["q_dec"], seq_np, wl.k)
                oracle_threads()
            del h
            if name != "ctx_128k" and t_used >= args.cpu_seconds:
                break
        cb = cpu_summary(wl, times, by, "%s of %s, all four steps per layer" % (
            "layers %s" % (list(sample),) if name == "ctx_128k" else "the first %d layers" % len(times), name),
            threads)
        cb["cpu_model"] = cpu_model()
        if t1 is not None:
            cb["one_thread"] = {"value": round(gbps(by["decode"], 1e6 * t1["decode"]), 4), "unit": "GB/s",
                                "cores": 1, "ms_per_layer": {s: round(1e3 * v, 2) for s, v in t1.items()},
                                "sample": "layer 0, one OpenMP thread"}
        row["cpu_baseline"] = cb
    del K, V, QW, QD, fold, path
    torch.cuda.empty_cache()
    return row


def measure_pyramid(wl, L, B, QW, K, V, QD, sl_all, dev, args):
    """The folded step with per-layer budgets (PyramidKV-style, mean budget k): layer l
    keeps pyramid_budgets(k, L)[l] + n_keep tokens per KV head; one select call over all
    layers takes the budgets as a per-unit array."""
    import torch

    from sparse_decode_amd import kvc, synth
    from sparse_decode_amd.pipeline import LayerPath
    budgets = synth.pyramid_budgets(wl.k, L, PYRAMID_BETA)
    path = LayerPath(wl, device=dev, batch=L * B, k=max(budgets))
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

    g = graph_of(step)
    ms, _ = timed_steps(g, args.steps, 1)
    del g
    mean_S = float(np.mean(sl_all.cpu().numpy()))
    nbytes = sum(sum(layer_bytes(wl, mean_S, budgets[l] + wl.n_keep)[c] for c in ("score", "select", "gather",
                                                                                   "decode")) for l in range(L))
    return {"schedule": "linear from (1+beta) k to (1-beta) k over the layers, mean k", "beta": PYRAMID_BETA,
            "k_first_layer": budgets[0], "k_last_layer": budgets[-1], "k_mean": round(sum(budgets) / L, 2),
            "ms_per_step": round(ms, 4), "value_GBps": round(nbytes / (ms * 1e-3) / 1e9, 2)}


def measure_core(wl, fold, sl_all, select_us, dev, args, flush):
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
    g = graph_of(lambda: kvc.select_core(fold.pooled, core_dev, wl.k, core_cap, wl.n_keep, seq_lens=sl_all,
                                         idx=idx, count=cnt, ws=ws))
    us = 1000.0 * timed_cold(g, args.reps, flush) / (LB // wl.batch)
    del g
    return {"core_frac": CORE_FRAC, "core_block": CORE_BLOCK, "core_tokens_per_seq": int(core.sum(axis=1).mean()),
            "k_scratch": wl.k, "mean_kept": round(float(cnt.float().mean()), 1),
            "us_per_layer": round(us, 3), "plain_select_us_per_layer": round(select_us, 3)}


# ------------------------------------------------------------------------ tiny fp32 layer

def measure_tiny(args, dev, flush):
    import torch

    import oracle
    from sparse_decode_amd import synth
    from sparse_decode_amd.pipeline import LayerPath
    wl = synth.by_name("tiny_fp32")
    x = synth.layer_inputs(wl, 0, device=dev)
    sl = torch.from_numpy(x["seq_lens"]).to(dev)
    p = LayerPath(wl, device=dev)
    calls = {"score": lambda: p.score(x["q_win"], x["k"], sl), "select": lambda: p.select(sl),
             "gather": lambda: p.gather(x["k"], x["v"]), "decode": lambda: p.decode(x["q_dec"])}
    reps = 50
    g = graph_of(lambda: [p.run(x["q_win"], x["k"], x["v"], x["q_dec"], sl) for _ in range(reps)])
    ms_step, _ = timed_steps(g, 3, 1)
    del g
    us = {}
    for c, fn in calls.items():
        g = graph_of(lambda fn=fn: [fn() for _ in range(reps)])
        us[c] = 1000.0 * timed_cold(g, args.reps, flush) / reps
        del g
    by = layer_bytes(wl, wl.s_max, p.cap)
    row = {"workload": wl.name, "layers": 1, "batch": 1, "seq_len": wl.s_max, "n_h": wl.n_h, "n_kv": wl.n_kv,
           "d_h": wl.d_h, "dtype": "f32", "w": wl.w, "pool": wl.pool, "k": wl.k, "n_keep": wl.n_keep,
           "us_per_step": round(1000.0 * ms_step / reps, 3),
           "per_layer_us": {c: round(v, 3) for c, v in us.items()},
           "per_layer_GBps": {c: round(gbps(by[c], v), 2) for c, v in us.items()},
           "roofline": dict(roofline("kvc_score_window (portable fp32 kernels)", by["score"], us["score"]),
                            bound="latency"),
           "timing": "graphs of %d back-to-back calls (latency-bound: 0.3 MB per layer)" % reps}
    if not args.no_cpu_baseline:
        h = {n: synth.to_host_f32(x[n]) for n in ("q_win", "k", "v", "q_dec")}
        threads = oracle_threads()
        ta = [oracle_layer(wl, h["q_win"], h["k"], h["v"], h["q_dec"], x["seq_lens"], wl.k)[0] for _ in range(20)]
        oracle.set_threads(1)
        t1 = [oracle_layer(wl, h["q_win"], h["k"], h["v"], h["q_dec"], x["seq_lens"], wl.k)[0] for _ in range(20)]
        oracle_threads()
        cb = cpu_summary(wl, ta, by, "20 runs of the layer, all four steps", threads)
        cb["cpu_model"] = cpu_model()
        c1 = cpu_summary(wl, t1, by, "20 runs of the layer, one thread", 1)
        cb["one_thread"] = {k: c1[k] for k in ("value", "unit", "cores", "ms_per_layer", "sample")}
        row["cpu_baseline"] = cb
    return row


# ------------------------------------------------------- batched ragged decode + retrieval

def measure_ragged(args, dev, flush):
    """ragged_b16: 16 sequences of 4096..16384 tokens; each of 64 decode steps re-scores
    the cache with its one query, selects 512 + 32 tokens per KV head, gathers them and
    attends.  Per-call figures are graphs of the 64 steps' calls of one kind."""
    import torch

    import oracle
    from sparse_decode_amd import synth
    from sparse_decode_amd.pipeline import LayerPath
    wl = synth.by_name("ragged_b16")
    x = synth.layer_inputs(wl, 0, device=dev, step=0)
    k, v = x["k"], x["v"]
    sl = torch.from_numpy(x["seq_lens"]).to(dev)
    steps = wl.steps
    qs = [synth.step_query(wl, 0, i, device=dev) for i in range(steps)]
    B, nh, d = qs[0].shape
    p = LayerPath(wl, device=dev)

    def step_all():
        for q in qs:
            p.score(q.view(B, nh, 1, d), k, sl)
            p.select(sl)
            p.gather(k, v)
            p.decode(q)

    g = graph_of(step_all)
    ms_all, _ = timed_steps(g, max(2, args.steps // 4), 1)
    del g
    calls = {"score": lambda: [p.score(q.view(B, nh, 1, d), k, sl) for q in qs],
             "select": lambda: [p.select(sl) for _ in qs], "gather": lambda: [p.gather(k, v) for _ in qs],
             "decode": lambda: [p.decode(q) for q in qs]}
    us = {}
    for c, fn in calls.items():
        g = graph_of(fn)
        us[c] = 1000.0 * timed_cold(g, args.reps, flush) / steps
        del g
    by = layer_bytes(wl, float(np.mean(x["seq_lens"])), p.cap)
    row = {"workload": wl.name, "batch": B, "seq_len_range": list(wl.ragged), "n_h": nh, "n_kv": wl.n_kv,
           "d_h": d, "w": wl.w, "pool": wl.pool, "k": wl.k, "n_keep": wl.n_keep, "decode_steps": steps,
           "us_per_step": round(1000.0 * ms_all / steps, 3),
           "per_step_us": {c: round(v, 3) for c, v in us.items()},
           "per_step_GBps": {c: round(gbps(by[c], v), 1) for c, v in us.items()},
           "per_step_hbm_frac": {c: round(gbps(by[c], v) / HBM_PEAK_GBPS, 4) for c, v in us.items()},
           "decode_GBps": round(gbps(by["decode"], us["decode"]), 1),
           "roofline": roofline("kvc_score_window, one step (16 sequences, one query per head)", by["score"],
                                us["score"]),
           "timing": "graph of the 64 steps per call type, median of %d cold replays" % args.reps}
    if not args.no_cpu_baseline:
        threads = oracle_threads()
        kh, vh = synth.to_host_f32(k), synth.to_host_f32(v)
        times, used = [], 0.0
        for i, q in enumerate(qs):
            qh = synth.to_host_f32(q)
            t, _ = oracle_layer(wl, qh[:, :, None, :], kh, vh, qh, x["seq_lens"], wl.k)
            times.append(t)
            used += sum(t.values())
            if used >= args.cpu_seconds:
                break
        cb = cpu_summary(wl, times, by, "the first %d of the 64 decode steps, all four steps each" % len(times),
                         threads)
        cb["cpu_model"] = cpu_model()
        row["cpu_baseline"] = cb
    print("[bench] ragged_b16: speculative and block retrieval", file=sys.stderr, flush=True)
    row["speculative_retrieval"] = measure_retrieval(dev, wl, x, qs, flush, args)
    return row


def measure_retrieval(dev, wl, x, qs, flush, args):
    """Speculative retrieval with fine-grained correction (FreeKV technical summary
    2.A) on the batched ragged decode, and landmark-guided block selection (xKV 2.3).

    Schedules of the 64 decode steps, each captured as one HIP graph:
      reselect     score -> select -> gather -> attention of every head, every step
      critical     what attention waits for under speculation: query similarity,
                   correction (score/select/gather of the drifted KV heads only), then
                   attention over the previous step's selection for the other heads
      overlapped   critical on the launch stream and the speculative selection for the
                   next step on a second stream beside it
      blocks       block scores from the block landmarks (built once, timed apart), top
                   k/16 blocks of 16 tokens, their tokens gathered, attention
    """
    import torch

    from sparse_decode_amd.pipeline import BlockRetrieval, LayerPath, SpeculativeRetrieval
    k, v = x["k"], x["v"]
    sl = torch.from_numpy(x["seq_lens"]).to(dev)
    B, nh, d = qs[0].shape
    steps = len(qs)
    base = LayerPath(wl, device=dev)
    spec = SpeculativeRetrieval(wl, RETRIEVAL_TAU, device=dev)
    blk = BlockRetrieval(wl, BLOCK_TOKENS, wl.k // BLOCK_TOKENS, device=dev)

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

    def blocks():
        for q in qs:
            blk.step(q, k, v, sl)

    spec.cur = 0
    corrected = []
    for i, q in enumerate(qs):
        spec.critical(q, qs[i - 1] if i else None, k, v, sl)
        if i:
            corrected.append(spec.refresh.float().mean())
        spec.speculate(q, k, v, sl)
        spec.swap()
    frac = float(torch.stack(corrected).mean()) if corrected else 1.0
    blk.prepare(k, sl)
    out = {}
    for name, fn in (("reselect", reselect), ("critical", critical), ("overlapped", overlapped),
                     ("blocks", blocks), ("landmarks_once", lambda: blk.prepare(k, sl))):
        g = graph_of(fn)
        out[name] = 1000.0 * timed_cold(g, max(3, args.reps // 2), flush) / (1 if name == "landmarks_once" else steps)
        del g
    return {"steps": steps, "tau": RETRIEVAL_TAU, "corrected_kv_head_frac": round(frac, 4),
            "us_per_step": {n: round(t, 2) for n, t in out.items() if n in ("reselect", "critical", "overlapped")},
            "critical_path_speedup": round(out["reselect"] / out["critical"], 3),
            "step_speedup_overlapped": round(out["reselect"] / out["overlapped"], 3),
            "block_selection": {"block": BLOCK_TOKENS, "k_blocks": wl.k // BLOCK_TOKENS,
                                "us_per_step": round(out["blocks"], 2),
                                "landmarks_us_once": round(out["landmarks_once"], 2),
                                "speedup_vs_reselect": round(out["reselect"] / out["blocks"], 3)},
            "timing": "HIP graph of all steps per schedule, median of cold replays"}


# ------------------------------------------------------------------ profiling entry

def profile_call(args, dev):
    """Replays one call of one headline layer (mha_tsp at S) `--calls` times, then one
    elementwise kernel over 1 GiB: a short program for rocprofv3 kernel-trace and --pmc
    runs (the elementwise kernel calibrates the byte counters)."""
    import torch

    from sparse_decode_amd import synth
    from sparse_decode_amd.pipeline import LayerPath
    wl = synth.by_name("mha_tsp")
    x = synth.layer_inputs(wl, 0, device=dev)
    sl = torch.from_numpy(x["seq_lens"]).to(dev)
    p = LayerPath(wl, device=dev)
    p.run(x["q_win"], x["k"], x["v"], x["q_dec"], sl)
    fn = {"score": lambda: p.score(x["q_win"], x["k"], sl), "select": lambda: p.select(sl),
          "gather": lambda: p.gather(x["k"], x["v"]), "decode": lambda: p.decode(x["q_dec"])}[args.profile_call]
    for _ in range(args.calls):
        fn()
    torch.cuda.synchronize()
    # calibration: an elementwise kernel that reads 1 GiB and writes 1 GiB (a same-dtype
    # copy_ would go to the copy engine, which the counters do not see)
    a = torch.zeros(1 << 28, dtype=torch.float32, device=dev)
    b = torch.empty_like(a)
    torch.neg(a, out=b)
    torch.cuda.synchronize()
    print("[bench] profiled %d %s calls of mha_tsp layer 0, then a 1 GiB elementwise negation" %
          (args.calls, args.profile_call), flush=True)


# ------------------------------------------------------------------------------ main

def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU: this path runs on a single MI355X and has no multi-GPU mode "
              "(requested --gpus %d)." % args.gpus, file=sys.stderr)
        sys.exit(2)
    import torch

    from sparse_decode_amd import kvc
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    kvc.lib()
    dev = torch.device("cuda")
    if args.profile_call:
        profile_call(args, dev)
        return
    flush = Flusher(dev)
    if args.only:
        fn = {"tiny_fp32": lambda: measure_tiny(args, dev, flush),
              "llama3_8b_32k": lambda: measure_folded("llama3_8b_32k", args, dev, flush, extras=True),
              "ctx_128k": lambda: measure_folded("ctx_128k", args, dev, flush),
              "ragged_b16": lambda: measure_ragged(args, dev, flush)}[args.only]
        print(json.dumps({args.only: fn()}), flush=True)
        return
    head, ctx = measure_headline(args, dev, flush)
    res = {"metric": METRIC, "value": head.pop("value"), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": head.pop("ms_per_step"), "higher_is_better": True,
           "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
           "data": "synthetic (seeded N(0,1) Q/K/V and hidden states with planted heavy hitters; no model weights)"}
    res.update(head)
    if not args.headline_only:
        print("[bench] TSP sweep", file=sys.stderr, flush=True)
        res["tsp_sweep"] = measure_tsp_sweep(args, dev, flush, ctx)
    del ctx
    torch.cuda.empty_cache()
    if not args.headline_only:
        cfgs = {}
        cfgs["tiny_fp32"] = measure_tiny(args, dev, flush)
        cfgs["llama3_8b_32k"] = measure_folded("llama3_8b_32k", args, dev, flush, extras=True)
        cfgs["ctx_128k"] = measure_folded("ctx_128k", args, dev, flush)
        cfgs["ragged_b16"] = measure_ragged(args, dev, flush)
        res["configs"] = cfgs
    # a plain device copy of 1 GiB: the bandwidth a read + write stream reaches here
    a = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    b = torch.empty_like(a)
    g = graph_of(lambda: b.copy_(a))
    copy_ms = timed_cold(g, 5, flush)
    cgb = 2.0 * (1 << 30) / (copy_ms * 1e-3) / 1e9
    res["copy_probe"] = {"GBps": round(cgb, 1), "frac_of_peak": round(cgb / HBM_PEAK_GBPS, 4),
                         "what": "torch device copy of 1 GiB, read + write bytes / time (median of 5 cold copies)"}
    res["decode_frac_of_copy"] = round(res["value"] / cgb, 4)
    res["roofline"]["frac_of_copy_probe"] = round(res["roofline"]["achieved"] / cgb, 4)
    # plain launch latency: a graph of 100 dependent one-element kernels
    t1 = torch.zeros(1, device=dev)
    g = graph_of(lambda: [t1.add_(1.0) for _ in range(100)])
    res["launch_probe"] = {"us_per_kernel": round(1000.0 * timed_cold(g, 5, flush) / 100, 3),
                           "what": "graph of 100 dependent one-element torch kernels, median replay / 100"}
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
