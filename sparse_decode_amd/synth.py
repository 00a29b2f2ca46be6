"""Seeded synthetic inputs shaped like the long-context workloads on the pages.

This module only draws inputs.  It holds none of the method's arithmetic (no
scoring, selection, gather or attention), so both the HIP path and the CPU
oracle can be fed from it.  Bulk tensors come from torch's seeded generator on
the requested device; heavy-hitter positions, directions and ragged lengths come
from numpy's PCG64, so they are identical on every device.

Workloads (the pages evaluate 8B-class models with contexts up to 128K on
LongBench/RULER/NIAH-style suites -- FastKV section 4, FreeKV technical summary
section 4; none of those suites is used, these synthetic shapes stand in):

1. ``tiny_fp32``      S=512, n_h=4, n_kv=2, d_h=64, fp32, w=16, pool 5, k=64 (+16),
                      8 planted keys = 3*sqrt(d_h) * unit mean window-query direction.
2. ``llama3_8b_32k``  32 layers, S=32768, 32/8 heads, d_h=128, bf16, w=32, pool 7,
                      k=2048 (+32), 1% planted keys = 4*sqrt(d_h) * per-head random unit.
3. ``ctx_128k``       as 2 with S=131072, 0.5% planted, k=ceil(1% of S)=1311 (+32).
4. ``ragged_b16``     batch 16, S_b ~ U{4096..16384}, 32/8 heads, bf16, one new query
                      per step (not in the cache), n_keep=32, pool 7, k=512, 64 steps.
                      Each head's query is (3 m + z_t) / sqrt(10): a persistent N(0,1)
                      component m plus fresh noise z_t, so adjacent steps have cosine
                      ~0.9 (FreeKV technical summary 2.A observes > 0.9); planted keys
                      lie along the unit mean of the group's persistent components.
5. ``mha_tsp``        batch 2, n_h=n_kv=32, S=65536, bf16, w=32, pool 7; at layer 16 the
                      top ceil(20%) tokens by window score (+32) keep their hidden
                      states [S][4096]; every layer keeps k=1024 (+32) for decode.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np
import torch

STREAM_QWIN, STREAM_K, STREAM_V, STREAM_QDEC, STREAM_HIDDEN, STREAM_QMEAN = 0, 1, 2, 3, 4, 5


@dataclass(frozen=True)
class Workload:
    cfg_id: int
    name: str
    batch: int
    layers: int
    s_max: int
    n_h: int
    n_kv: int
    d_h: int
    dtype: str                  # "f32" or "bf16"
    w: int                      # observation-window rows per query head
    window_in_cache: bool       # window queries are the last w cached tokens
    n_keep: int                 # trailing tokens always kept
    pool: int                   # odd max-pool width
    k: int                      # retention budget (candidates), per KV head
    hh_frac: float = 0.0        # planted heavy hitters as a fraction of S_b (ceil)
    hh_count: int = 0           # or an absolute count
    hh_mag: float = 4.0         # magnitude in units of sqrt(d_h)
    hh_dir: str = "random"      # "random" per (layer, KV head), "window_mean" or "query_mean"
    query_mode: str = "iid"     # "iid", or "persistent" (per-step queries share a component)
    ragged: tuple | None = None  # (lo, hi) inclusive range of S_b
    steps: int = 1
    tsp_layer: int | None = None
    tsp_rate: float = 0.0
    hidden: int = 0
    notes: dict = field(default_factory=dict, compare=False)

    @property
    def group(self) -> int:
        return self.n_h // self.n_kv

    @property
    def cap(self) -> int:
        return self.k + self.n_keep

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == "f32" else torch.bfloat16


WORKLOADS = {
    1: Workload(1, "tiny_fp32", 1, 1, 512, 4, 2, 64, "f32", 16, True, 16, 5, 64,
                hh_count=8, hh_mag=3.0, hh_dir="window_mean"),
    2: Workload(2, "llama3_8b_32k", 1, 32, 32768, 32, 8, 128, "bf16", 32, True, 32, 7, 2048,
                hh_frac=0.01),
    3: Workload(3, "ctx_128k", 1, 32, 131072, 32, 8, 128, "bf16", 32, True, 32, 7, 1311,
                hh_frac=0.005),
    4: Workload(4, "ragged_b16", 16, 1, 16384, 32, 8, 128, "bf16", 1, False, 32, 7, 512,
                hh_frac=0.01, hh_dir="query_mean", query_mode="persistent", ragged=(4096, 16384), steps=64),
    5: Workload(5, "mha_tsp", 2, 32, 65536, 32, 32, 128, "bf16", 32, True, 32, 7, 1024,
                hh_frac=0.01, tsp_layer=16, tsp_rate=0.2, hidden=4096),
}


def by_name(name: str) -> Workload:
    for wl in WORKLOADS.values():
        if wl.name == name:
            return wl
    raise KeyError(name)


def budget_from_rate(rate: float, s: int) -> int:
    """A retention rate becomes an integer budget by rounding up (1% of 131072 -> 1311)."""
    return int(math.ceil(rate * s - 1e-9))


def pyramid_budgets(k: int, layers: int, beta: float = 0.5) -> list[int]:
    """Per-layer budgets that fall linearly from (1 + beta) k at the first layer to
    (1 - beta) k at the last, rounded, so that their mean is k (a PyramidKV-style
    schedule: the Tutorial, "Compresser un cache existant", gives layers different
    budgets; the shape of the schedule is this reading's)."""
    if layers == 1:
        return [k]
    return [int(round(k * (1.0 + beta * (1.0 - 2.0 * l / (layers - 1))))) for l in range(layers)]


def seed_for(cfg_id: int, layer: int, stream: int, step: int = 0) -> int:
    return ((cfg_id * 1000 + layer) * 1000 + step) * 10 + stream


def seq_lens(wl: Workload, s_max: int | None = None) -> np.ndarray:
    """Per-sequence lengths: s_max each, or for a ragged workload its seeded lengths,
    none above s_max (a smaller s_max cuts the longer sequences at s_max)."""
    s_max = wl.s_max if s_max is None else s_max
    if wl.ragged is None:
        return np.full(wl.batch, s_max, np.int32)
    lo, hi = wl.ragged
    rng = np.random.Generator(np.random.PCG64([wl.cfg_id, 0x6C656E73]))
    return np.minimum(rng.integers(lo, hi + 1, size=wl.batch), s_max).astype(np.int32)


def planted_positions(wl: Workload, b: int, s_b: int, n_keep: int | None = None) -> np.ndarray:
    """Heavy-hitter positions of sequence b, drawn once per sequence from the candidate
    region [0, S_b - n_keep) and shared by every layer and KV head."""
    n_keep = wl.n_keep if n_keep is None else n_keep
    region = max(0, s_b - n_keep)
    n = wl.hh_count if wl.hh_count else int(math.ceil(wl.hh_frac * s_b - 1e-9))
    n = min(n, region)
    rng = np.random.Generator(np.random.PCG64([wl.cfg_id, 0x68680000 + b, s_b]))
    return np.sort(rng.choice(region, size=n, replace=False)).astype(np.int64)


def _randn(shape, seed, device):
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return torch.randn(shape, generator=g, device=device, dtype=torch.float32)


def _unit_dirs(wl: Workload, layer: int, n: int, d: int) -> np.ndarray:
    rng = np.random.Generator(np.random.PCG64([wl.cfg_id, 0x64697200 + layer]))
    u = rng.standard_normal((n, d))
    return u / np.linalg.norm(u, axis=1, keepdims=True)


def _step_queries(wl: Workload, layer: int, step: int, B: int, device):
    """The per-step query rows [B][n_h][w][d_h] (fp32) of a workload whose query is
    not in the cache, and the persistent component (None for iid queries)."""
    d, nh = wl.d_h, wl.n_h
    q_win = _randn((B, nh, wl.w, d), seed_for(wl.cfg_id, layer, STREAM_QDEC, step), device)
    qm = None
    if wl.query_mode == "persistent":
        qm = _randn((B, nh, d), seed_for(wl.cfg_id, layer, STREAM_QMEAN), device)
        q_win = (3.0 * qm[:, :, None, :] + q_win) / math.sqrt(10.0)
    return q_win, qm


def step_query(wl: Workload, layer: int, step: int, device="cpu", batch: int | None = None):
    """Decode query [B][n_h][d_h] of one step (workload dtype), identical to the q_dec
    that layer_inputs returns for that step, without drawing the cache again."""
    B = wl.batch if batch is None else batch
    q_win, _ = _step_queries(wl, layer, step, B, device)
    return q_win[:, :, -1, :].to(wl.torch_dtype).contiguous()


def layer_inputs(wl: Workload, layer: int = 0, device="cpu", step: int = 0, s_max: int | None = None,
                 batch: int | None = None):
    """Draws one layer's window queries, cache and decode query.

    Returns a dict with q_win [B][n_h][w][d_h], k and v [B][n_kv][s_max][d_h],
    q_dec [B][n_h][d_h] (all in the workload's dtype on ``device``), seq_lens
    (int32 numpy [B]) and planted (list of int64 numpy arrays, one per sequence).
    For a workload whose query is not in the cache (window_in_cache False, w=1) the
    per-step query is q_win and q_dec holds the same values.
    """
    B = wl.batch if batch is None else batch
    S = wl.s_max if s_max is None else s_max
    sl = seq_lens(wl, S)[:B]
    dt = wl.torch_dtype
    d, nh, nkv = wl.d_h, wl.n_h, wl.n_kv
    if wl.window_in_cache:
        q_win = _randn((B, nh, wl.w, d), seed_for(wl.cfg_id, layer, STREAM_QWIN), device)
        q_dec = _randn((B, nh, d), seed_for(wl.cfg_id, layer, STREAM_QDEC), device)
    else:
        q_win, qm = _step_queries(wl, layer, step, B, device)
        q_dec = q_win[:, :, -1, :].clone()
    k = _randn((B, nkv, S, d), seed_for(wl.cfg_id, layer, STREAM_K), device)
    v = _randn((B, nkv, S, d), seed_for(wl.cfg_id, layer, STREAM_V), device)
    planted = []
    for b in range(B):
        pos = planted_positions(wl, b, int(sl[b]))
        planted.append(pos)
        if pos.size == 0:
            continue
        if wl.hh_dir == "window_mean":
            r = wl.group
            m = q_win[b].reshape(nkv, r * wl.w, d).mean(dim=1)
            dirs = m / m.norm(dim=1, keepdim=True)
        elif wl.hh_dir == "query_mean":
            m = qm[b].reshape(nkv, wl.group, d).mean(dim=1)
            dirs = m / m.norm(dim=1, keepdim=True)
        else:
            dirs = torch.from_numpy(_unit_dirs(wl, layer, nkv, d)).to(device=device, dtype=torch.float32)
        vecs = (wl.hh_mag * math.sqrt(d)) * dirs                     # [n_kv][d]
        pos_t = torch.from_numpy(pos).to(device)
        k[b][:, pos_t, :] = vecs[:, None, :].expand(nkv, pos.size, d)
    return {
        "q_win": q_win.to(dt).contiguous(),
        "k": k.to(dt).contiguous(),
        "v": v.to(dt).contiguous(),
        "q_dec": q_dec.to(dt).contiguous(),
        "seq_lens": sl,
        "planted": planted,
    }


def hidden_states(wl: Workload, device="cpu", s_max: int | None = None):
    """Hidden states [B][S][hidden] of the token-selective propagation layer."""
    S = wl.s_max if s_max is None else s_max
    return _randn((wl.batch, S, wl.hidden), seed_for(wl.cfg_id, wl.tsp_layer or 0, STREAM_HIDDEN),
                  device).to(wl.torch_dtype).contiguous()


def to_host_f32(t: torch.Tensor) -> np.ndarray:
    """Exact widening of a device tensor to a float32 host array (bf16 -> f32 is exact)."""
    return t.detach().to("cpu").to(torch.float32).contiguous().numpy()
