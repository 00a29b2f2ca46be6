"""Per-layer driver of the four-step path: preallocated buffers plus the call
sequence score -> select -> gather -> decode through the C ABI binding.

This is host-side orchestration only (no arithmetic of its own): it is what a
serving loop would do after prefill (FastKV section 2.B: one retention budget per
layer; Tutorial "Variantes de l'attention et compression du cache KV", section
"Compresser un cache existant") or at every decode step of a retrieval method
(FreeKV technical summary section 2.A).
"""
from __future__ import annotations

import torch

from . import kvc
from .synth import Workload


class LayerPath:
    """Buffers for one layer shape; `run` enqueues the four steps on the current stream."""

    def __init__(self, wl: Workload, device="cuda", s_max: int | None = None, batch: int | None = None,
                 k: int | None = None):
        self.wl = wl
        self.B = wl.batch if batch is None else batch
        self.S = wl.s_max if s_max is None else s_max
        self.k = wl.k if k is None else k
        self.cap = self.k + wl.n_keep
        dev = torch.device(device)
        B, S, nkv, nh, d = self.B, self.S, wl.n_kv, wl.n_h, wl.d_h
        dt = wl.torch_dtype
        self.raw = torch.empty((B, nkv, S), dtype=torch.float32, device=dev)
        self.pooled = torch.empty((B, nkv, S), dtype=torch.float32, device=dev)
        self.idx = torch.empty((B, nkv, self.cap), dtype=torch.int32, device=dev)
        self.count = torch.empty((B, nkv), dtype=torch.int32, device=dev)
        self.kc = torch.empty((B, nkv, self.cap, d), dtype=dt, device=dev)
        self.vc = torch.empty((B, nkv, self.cap, d), dtype=dt, device=dev)
        self.pos = torch.empty((B, nkv, self.cap), dtype=torch.int32, device=dev)
        self.out = torch.empty((B, nh, d), dtype=dt, device=dev)
        self.lse = torch.empty((B, nh), dtype=torch.float32, device=dev)
        code = kvc.KVC_BF16 if wl.dtype == "bf16" else kvc.KVC_F32
        dims = kvc.make_dims(B, S, nh, nkv, d, code)
        self.ws_score = torch.zeros(max(256, kvc.score_window_workspace(dims, wl.w)), dtype=torch.uint8, device=dev)
        self.ws_decode = torch.zeros(max(256, kvc.decode_attn_workspace(dims, self.cap)), dtype=torch.uint8,
                                     device=dev)
        sdims = kvc.make_dims(B, S, nkv, nkv, 128, kvc.KVC_F32)
        self.ws_select = torch.zeros(max(256, kvc.select_topk_workspace(sdims, self.k, wl.n_keep)),
                                     dtype=torch.uint8, device=dev)

    def score(self, q_win, k, seq_lens=None, unit_mask=None):
        wl = self.wl
        return kvc.score_window(q_win, k, wl.w, seq_lens=seq_lens, window_in_cache=wl.window_in_cache,
                                n_keep=wl.n_keep, pool=wl.pool, raw=self.raw, pooled=self.pooled,
                                ws=self.ws_score, unit_mask=unit_mask)

    def select(self, seq_lens=None, unit_mask=None, k_per_unit=None):
        return kvc.select_topk(self.pooled, self.k, self.wl.n_keep, seq_lens=seq_lens, idx=self.idx,
                               count=self.count, ws=self.ws_select, unit_mask=unit_mask, k_per_unit=k_per_unit)

    def gather(self, k, v, src_pos=None, unit_mask=None):
        return kvc.gather_compact(k, self.idx, self.count, src1=v, src_pos=src_pos, dst0=self.kc, dst1=self.vc,
                                  pos_out=self.pos, unit_mask=unit_mask)

    def decode(self, q_dec):
        return kvc.decode_attn(q_dec, self.kc, self.vc, self.count, out=self.out, lse=self.lse,
                               ws=self.ws_decode)

    def run(self, q_win, k, v, q_dec, seq_lens=None, src_pos=None):
        self.score(q_win, k, seq_lens)
        self.select(seq_lens)
        self.gather(k, v, src_pos)
        self.decode(q_dec)
        return self.out


class TspStep:
    """FastKV section 2.A token-selective propagation at one layer: one selection per
    sequence from the head-summed window scores, then the gather of those tokens'
    hidden states (the sliding-window tokens always propagate)."""

    def __init__(self, wl: Workload, k_tsp: int, device="cuda", s_max: int | None = None):
        self.wl = wl
        self.S = wl.s_max if s_max is None else s_max
        self.k = k_tsp
        self.cap = k_tsp + wl.n_keep
        dev = torch.device(device)
        B = wl.batch
        self.idx = torch.empty((B, 1, self.cap), dtype=torch.int32, device=dev)
        self.count = torch.empty((B, 1), dtype=torch.int32, device=dev)
        self.hidden_out = torch.empty((B, 1, self.cap, wl.hidden), dtype=wl.torch_dtype, device=dev)
        self.pos = torch.empty((B, 1, self.cap), dtype=torch.int32, device=dev)
        dims = kvc.make_dims(B, self.S, wl.n_kv, wl.n_kv, wl.d_h, kvc.KVC_F32)
        need = kvc.select_topk_workspace(dims, self.k, wl.n_keep, kvc.KVC_SELECT_SHARED_HEADS)
        self.ws = torch.zeros(max(256, need), dtype=torch.uint8, device=dev)

    def run(self, pooled, hidden, seq_lens=None):
        kvc.select_topk(pooled, self.k, self.wl.n_keep, seq_lens=seq_lens, shared_heads=True, idx=self.idx,
                        count=self.count, ws=self.ws)
        h = hidden.view(hidden.shape[0], 1, hidden.shape[1], hidden.shape[2])
        kvc.gather_compact(h, self.idx, self.count, dst0=self.hidden_out, pos_out=self.pos)
        return self.hidden_out, self.pos


class SpeculativeRetrieval:
    """FreeKV technical summary section 2.A on one GPU: speculative retrieval with
    fine-grained correction, for a workload whose per-step query re-scores the cache.

    Two compacted caches alternate.  At step i the current one holds the selection
    made with q_{i-1}; `critical` finds the KV heads whose query drifted (cosine
    below tau for some query head of the group), redoes score -> select -> gather
    for those heads only (unit masks), and attends over the current cache.
    `speculate` then selects with q_i for every head into the other cache, which
    step i + 1 reuses; it does not depend on step i's attention and may run on a
    second stream beside it.  `swap` makes the other cache current.  The first
    step has no previous query: every head is selected before attention.
    """

    def __init__(self, wl: Workload, tau: float, device="cuda", s_max: int | None = None,
                 batch: int | None = None):
        self.wl = wl
        self.tau = float(tau)
        self.paths = [LayerPath(wl, device, s_max, batch), LayerPath(wl, device, s_max, batch)]
        self.cur = 0
        B, dev = self.paths[0].B, torch.device(device)
        self.cos = torch.empty((B, wl.n_h), dtype=torch.float32, device=dev)
        self.refresh = torch.empty((B, wl.n_kv), dtype=torch.int32, device=dev)
        self.keep = torch.empty((B, wl.n_kv), dtype=torch.int32, device=dev)

    @property
    def current(self) -> LayerPath:
        return self.paths[self.cur]

    @property
    def other(self) -> LayerPath:
        return self.paths[1 - self.cur]

    def critical(self, q, q_prev, k, v, seq_lens=None):
        """The work before step i's attention, then the attention itself.
        q, q_prev [B][n_h][d_h] (q_prev None at the first step)."""
        p = self.current
        q_win = q.view(q.shape[0], q.shape[1], 1, q.shape[2])
        if q_prev is None:
            self.refresh.fill_(1)
            self.keep.fill_(0)
            p.score(q_win, k, seq_lens)
            p.select(seq_lens)
            p.gather(k, v)
        else:
            kvc.query_similarity(q, q_prev, self.wl.n_kv, self.tau, cos=self.cos, refresh=self.refresh,
                                 keep=self.keep)
            p.score(q_win, k, seq_lens, unit_mask=self.refresh)
            p.select(seq_lens, unit_mask=self.refresh)
            p.gather(k, v, unit_mask=self.refresh)
        return p.decode(q)

    def speculate(self, q, k, v, seq_lens=None):
        """Selection with q for every head into the other cache (used by the next step)."""
        p = self.other
        p.score(q.view(q.shape[0], q.shape[1], 1, q.shape[2]), k, seq_lens)
        p.select(seq_lens)
        p.gather(k, v)

    def swap(self):
        self.cur = 1 - self.cur


class BlockRetrieval:
    """xKV section 2.3 selective reconstruction's token choice on one GPU: landmark-
    guided block selection (ShadowKV-style).  `prepare` builds the block landmarks of
    the cache once; `step` scores the blocks with the step's query, keeps the best
    k_blocks blocks of every KV head (plus the trailing tokens that start no candidate
    block), gathers their rows and attends over them."""

    def __init__(self, wl: Workload, block: int, k_blocks: int, device="cuda", s_max: int | None = None,
                 batch: int | None = None):
        self.wl = wl
        self.block = int(block)
        self.k_blocks = int(k_blocks)
        dev = torch.device(device)
        self.B = wl.batch if batch is None else batch
        self.S = wl.s_max if s_max is None else s_max
        B, S, nkv, nh, d = self.B, self.S, wl.n_kv, wl.n_h, wl.d_h
        self.n_blk = (S + self.block - 1) // self.block
        self.cap = self.k_blocks * self.block + wl.n_keep + self.block - 1
        self.landmarks = torch.empty((B, nkv, self.n_blk, d), dtype=torch.float32, device=dev)
        self.scores = torch.empty((B, nkv, self.n_blk), dtype=torch.float32, device=dev)
        self.cand = torch.empty((B,), dtype=torch.int32, device=dev)
        self.bidx = torch.empty((B, nkv, self.k_blocks), dtype=torch.int32, device=dev)
        self.bcount = torch.empty((B, nkv), dtype=torch.int32, device=dev)
        self.idx = torch.empty((B, nkv, self.cap), dtype=torch.int32, device=dev)
        self.count = torch.empty((B, nkv), dtype=torch.int32, device=dev)
        dt = wl.torch_dtype
        self.kc = torch.empty((B, nkv, self.cap, d), dtype=dt, device=dev)
        self.vc = torch.empty((B, nkv, self.cap, d), dtype=dt, device=dev)
        self.pos = torch.empty((B, nkv, self.cap), dtype=torch.int32, device=dev)
        self.out = torch.empty((B, nh, d), dtype=dt, device=dev)
        self.lse = torch.empty((B, nh), dtype=torch.float32, device=dev)
        sdims = kvc.make_dims(B, self.n_blk, nkv, nkv, 128, kvc.KVC_F32)
        self.ws_select = torch.zeros(max(256, kvc.select_topk_workspace(sdims, self.k_blocks, 0)),
                                     dtype=torch.uint8, device=dev)
        dims = kvc.make_dims(B, S, nh, nkv, d, kvc.KVC_BF16 if wl.dtype == "bf16" else kvc.KVC_F32)
        self.ws_decode = torch.zeros(max(256, kvc.decode_attn_workspace(dims, self.cap)), dtype=torch.uint8,
                                     device=dev)

    def prepare(self, k, seq_lens=None):
        return kvc.block_landmarks(k, self.block, seq_lens=seq_lens, out=self.landmarks)

    def step(self, q, k, v, seq_lens=None):
        wl = self.wl
        kvc.block_scores(q, self.landmarks, self.block, wl.n_keep, self.S, seq_lens=seq_lens, scores=self.scores,
                         cand=self.cand)
        kvc.select_topk(self.scores, self.k_blocks, 0, seq_lens=self.cand, idx=self.bidx, count=self.bcount,
                        ws=self.ws_select)
        kvc.expand_blocks(self.bidx, self.bcount, self.block, wl.n_keep, self.S, self.cap, seq_lens=seq_lens,
                          idx=self.idx, count=self.count)
        kvc.gather_compact(k, self.idx, self.count, src1=v, dst0=self.kc, dst1=self.vc, pos_out=self.pos)
        return kvc.decode_attn(q, self.kc, self.vc, self.count, out=self.out, lse=self.lse, ws=self.ws_decode)


class TspSchedule:
    """One decode step of FastKV's layer-by-layer schedule over a whole model's cache
    (FastKV sections 2.A and 2.B): layers up to and including the propagation layer
    run score -> select -> gather -> decode over all S cached tokens; at the
    propagation layer one selection per sequence from the head-summed scores keeps
    k_tsp tokens plus the window and gathers their hidden states; every later layer
    runs over those S' = k_tsp + n_keep tokens, its compacted cache keeping their
    original positions.  The per-layer retention budget (wl.k) and the TSP budget are
    independent.

    layers   list of per-layer dicts (q_win, k, v, q_dec), one per model layer; the
             first tsp_layer + 1 hold caches of s_full tokens, the others of s_after
             tokens (entries may repeat the same tensors)
    Each layer keeps its own selection and compacted cache (idx, count, kc, vc, pos,
    out, lse), so a layer's decode reads that layer's cache; score and select scratch
    is shared by the layers of one length, which run one after another.
    """

    def __init__(self, wl: Workload, layers, tsp_layer: int, k_tsp: int, seq_full, seq_after, hidden,
                 device="cuda"):
        self.wl = wl
        self.layers = layers
        self.tsp_layer = int(tsp_layer)
        self.k_tsp = int(k_tsp)
        self.s_full = int(layers[0]["k"].shape[2])
        self.s_after = self.k_tsp + wl.n_keep
        self.seq_full = seq_full
        self.seq_after = seq_after
        self.hidden = hidden
        dev = torch.device(device)
        self.full = LayerPath(wl, device=dev, s_max=self.s_full)
        self.after = LayerPath(wl, device=dev, s_max=self.s_after)
        self.tsp = TspStep(wl, self.k_tsp, device=dev, s_max=self.s_full)
        B, nkv, nh, d, cap = wl.batch, wl.n_kv, wl.n_h, wl.d_h, self.full.cap
        dt = wl.torch_dtype
        L = len(layers)
        self.idx = torch.empty((L, B, nkv, cap), dtype=torch.int32, device=dev)
        self.count = torch.empty((L, B, nkv), dtype=torch.int32, device=dev)
        self.kc = torch.empty((L, B, nkv, cap, d), dtype=dt, device=dev)
        self.vc = torch.empty((L, B, nkv, cap, d), dtype=dt, device=dev)
        self.pos = torch.empty((L, B, nkv, cap), dtype=torch.int32, device=dev)
        self.out = torch.empty((L, B, nh, d), dtype=dt, device=dev)
        self.lse = torch.empty((L, B, nh), dtype=torch.float32, device=dev)
        # the propagation layer's kept original positions, [B][S'], are the later
        # layers' source positions
        self.src_pos = self.tsp.pos.view(B, self.s_after)

    def path_of(self, l: int) -> LayerPath:
        return self.full if l <= self.tsp_layer else self.after

    def seq_of(self, l: int):
        return self.seq_full if l <= self.tsp_layer else self.seq_after

    def score(self, l: int):
        x = self.layers[l]
        self.path_of(l).score(x["q_win"], x["k"], self.seq_of(l))

    def select(self, l: int):
        p = self.path_of(l)
        kvc.select_topk(p.pooled, p.k, self.wl.n_keep, seq_lens=self.seq_of(l), idx=self.idx[l],
                        count=self.count[l], ws=p.ws_select)

    def gather(self, l: int):
        x = self.layers[l]
        sp = None if l <= self.tsp_layer else self.src_pos
        kvc.gather_compact(x["k"], self.idx[l], self.count[l], src1=x["v"], src_pos=sp, dst0=self.kc[l],
                           dst1=self.vc[l], pos_out=self.pos[l])

    def decode(self, l: int):
        kvc.decode_attn(self.layers[l]["q_dec"], self.kc[l], self.vc[l], self.count[l], out=self.out[l],
                        lse=self.lse[l], ws=self.full.ws_decode)

    def propagate(self):
        """The propagation layer's shared selection and hidden-state gather (its kept
        original positions are src_pos)."""
        self.tsp.run(self.full.pooled, self.hidden, self.seq_full)

    def layer(self, l: int):
        self.score(l)
        self.select(l)
        self.gather(l)
        self.decode(l)
        if l == self.tsp_layer:
            self.propagate()

    def step(self):
        for l in range(len(self.layers)):
            self.layer(l)
        return self.out
