"""ctypes binding of the plain C oracle ``kvc_oracle.c`` (test infrastructure only).

Every function takes and returns numpy arrays on the host.  Floating-point inputs
are float32 arrays; bf16 data is passed after an exact widening to float32 by the
caller.  The C file states, step by step, what each function computes and which
page section it follows.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kvc_oracle.c")
_LIB_PATH = os.path.join(_HERE, "_build", "libkvc_oracle.so")
_lock = threading.Lock()
_lib = None


def build(force: bool = True) -> str:
    """Compiles the oracle with gcc (plain -O2, OpenMP, no fast-math)."""
    if not force and os.path.exists(_LIB_PATH):
        return _LIB_PATH
    os.makedirs(os.path.dirname(_LIB_PATH), exist_ok=True)
    tmp = _LIB_PATH + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-std=c11", "-O2", "-fopenmp", "-fPIC", "-shared", "-fvisibility=hidden",
           _SRC, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(_LIB_PATH):
                build()
            lib = ctypes.CDLL(_LIB_PATH)
            P = ctypes.c_void_p
            I = ctypes.c_int
            lib.kvo_cache_bytes.restype = ctypes.c_uint64
            lib.kvo_cache_bytes.argtypes = [ctypes.c_int64] * 5
            lib.kvo_set_threads.restype = I
            lib.kvo_set_threads.argtypes = [I]
            lib.kvo_score_window.restype = None
            lib.kvo_score_window.argtypes = [I, I, P, I, I, I, P, P, I, I, I, I, ctypes.c_double, P, P, P]
            lib.kvo_select_topk.restype = None
            lib.kvo_select_topk.argtypes = [I, I, I, P, P, I, I, I, P, P]
            lib.kvo_gather.restype = None
            lib.kvo_gather.argtypes = [I, I, I, I, P, P, P, P, I, P, P]
            lib.kvo_decode.restype = None
            lib.kvo_decode.argtypes = [I, I, I, I, P, P, P, P, I, ctypes.c_double, P, P]
            lib.kvo_block_landmarks.restype = None
            lib.kvo_block_landmarks.argtypes = [I, I, I, I, P, P, I, P]
            lib.kvo_block_scores.restype = None
            lib.kvo_block_scores.argtypes = [I, I, I, I, I, P, P, P, I, I, ctypes.c_double, P, P]
            lib.kvo_expand_blocks.restype = None
            lib.kvo_expand_blocks.argtypes = [I, I, I, P, I, I, P, P, I, P, P, I]
            lib.kvo_select_core.restype = None
            lib.kvo_select_core.argtypes = [I, I, I, P, P, P, I, I, I, P, P]
            lib.kvo_query_similarity.restype = None
            lib.kvo_query_similarity.argtypes = [I, I, I, I, P, P, ctypes.c_double, P, P]
            _lib = lib
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _f32(a):
    a = np.ascontiguousarray(a)
    if a.dtype != np.float32:
        raise TypeError("oracle expects float32 input, got %s" % a.dtype)
    return a


def _i32(a):
    return None if a is None else np.ascontiguousarray(np.asarray(a, dtype=np.int32))


def set_threads(n: int = 0) -> int:
    return int(_load().kvo_set_threads(int(n)))


def cache_bytes(L: int, S: int, n_kv: int, d_h: int, b: int) -> int:
    """Tutorial, "MHA et GQA": 2 * L * S * n_kv * d_h * b bytes per sequence."""
    return int(_load().kvo_cache_bytes(L, S, n_kv, d_h, b))


def score_window(q_win, k, w, *, seq_lens=None, window_in_cache=True, n_keep=None, pool=1,
                 scale=None, want_raw64=False):
    """Window saliency + candidate-region max pool (FastKV 2.A; Tutorial,
    "Compresser un cache existant").

    q_win [B][n_h][w][d_h] float32, k [B][n_kv][s_max][d_h] float32.
    Returns (raw, pooled) float32 [B][n_kv][s_max] (and raw64 float64 if asked).
    """
    q_win = _f32(q_win)
    k = _f32(k)
    B, n_h, w_, d_h = q_win.shape
    Bk, n_kv, s_max, d_k = k.shape
    assert w_ == w and Bk == B and d_k == d_h and n_h % n_kv == 0
    if n_keep is None:
        n_keep = w
    if scale is None:
        scale = 1.0 / np.sqrt(d_h)
    sl = _i32(seq_lens)
    raw = np.zeros((B, n_kv, s_max), np.float32)
    pooled = np.zeros((B, n_kv, s_max), np.float32)
    raw64 = np.zeros((B, n_kv, s_max), np.float64) if want_raw64 else None
    _load().kvo_score_window(B, s_max, _ptr(sl), n_h, n_kv, d_h, _ptr(q_win), _ptr(k), int(w),
                             int(bool(window_in_cache)), int(n_keep), int(pool), float(scale),
                             _ptr(raw64), _ptr(raw), _ptr(pooled))
    if want_raw64:
        return raw, pooled, raw64
    return raw, pooled


def select_topk(scores, k, n_keep, *, seq_lens=None, shared_heads=False, k_per_unit=None):
    """Per-head top-k (score desc, index asc) + trailing n_keep tokens, ascending.

    scores [B][H][s_max] float32.  Returns (idx int32 [B][H_out][k+n_keep], count int32 [B][H_out]).
    With k_per_unit ([B][H_out]), unit u takes min(k_per_unit[u], k) candidates (clamped at 0)
    and its row keeps the width k + n_keep, -1 padded (per-layer budgets, Tutorial
    "Compresser un cache existant": PyramidKV gives layers different cache budgets).
    """
    scores = _f32(scores)
    B, H, s_max = scores.shape
    H_out = 1 if shared_heads else H
    cap = k + n_keep
    sl = _i32(seq_lens)
    if k_per_unit is not None:
        ku = np.clip(np.asarray(k_per_unit, np.int64).reshape(B, H_out), 0, k)
        idx = np.full((B, H_out, cap), -1, np.int32)
        count = np.empty((B, H_out), np.int32)
        for b in range(B):
            slb = None if sl is None else sl[b:b + 1]
            for h in range(H_out):
                src = scores[b:b + 1] if shared_heads else scores[b:b + 1, h:h + 1]
                i1, c1 = select_topk(src, int(ku[b, h]), n_keep, seq_lens=slb, shared_heads=shared_heads)
                idx[b, h, :i1.shape[-1]] = i1[0, 0]
                count[b, h] = c1[0, 0]
        return idx, count
    idx = np.empty((B, H_out, cap), np.int32)
    count = np.empty((B, H_out), np.int32)
    _load().kvo_select_topk(B, H, s_max, _ptr(sl), _ptr(scores), int(k), int(n_keep),
                            int(bool(shared_heads)), _ptr(idx), _ptr(count))
    return idx, count


def gather(src, idx, count, *, src_pos=None, dst=None):
    """Compacting gather of rows; src [B][heads][s_max][...] any dtype.

    Returns (dst [B][heads][cap][...], pos_out [B][heads][cap]).  Rows past count
    keep what ``dst`` held (zeros when it is not given); their pos_out is -1.
    """
    src = np.ascontiguousarray(src)
    B, heads, s_max = src.shape[:3]
    row_shape = src.shape[3:]
    row_bytes = int(np.prod(row_shape, dtype=np.int64)) * src.itemsize
    idx = _i32(idx)
    count = _i32(count)
    cap = idx.shape[-1]
    if dst is None:
        dst = np.zeros((B, heads, cap) + row_shape, src.dtype)
    else:
        dst = np.ascontiguousarray(dst).copy()
    pos = np.empty((B, heads, cap), np.int32)
    sp = _i32(src_pos)
    _load().kvo_gather(B, heads, s_max, row_bytes, _ptr(src), _ptr(sp), _ptr(idx), _ptr(count),
                       cap, _ptr(dst), _ptr(pos))
    return dst, pos


def decode(q, kc, vc, count, *, scale=None):
    """GQA decode attention over the compacted cache, in double.

    q [B][n_h][d_h], kc/vc [B][n_kv][cap][d_h] float32, count [B][n_kv].
    Returns (out float64 [B][n_h][d_h], lse float64 [B][n_h]).
    """
    q = _f32(q)
    kc = _f32(kc)
    vc = _f32(vc)
    B, n_h, d_h = q.shape
    _, n_kv, cap, _ = kc.shape
    assert n_h % n_kv == 0
    if scale is None:
        scale = 1.0 / np.sqrt(d_h)
    count = _i32(count)
    out = np.zeros((B, n_h, d_h), np.float64)
    lse = np.zeros((B, n_h), np.float64)
    _load().kvo_decode(B, n_h, n_kv, d_h, _ptr(q), _ptr(kc), _ptr(vc), _ptr(count), int(cap),
                       float(scale), _ptr(out), _ptr(lse))
    return out, lse


def query_similarity(q_cur, q_prev, n_kv, tau):
    """FreeKV technical summary 2.A: per query head cosine of the queries of two
    adjacent decode steps, and the KV heads to correct (some query head below tau).

    q_cur, q_prev [B][n_h][d_h] float32.  Returns (cos float64 [B][n_h],
    refresh int32 [B][n_kv]).
    """
    q_cur = _f32(q_cur)
    q_prev = _f32(q_prev)
    B, n_h, d_h = q_cur.shape
    assert q_prev.shape == q_cur.shape and n_h % n_kv == 0
    cos = np.zeros((B, n_h), np.float64)
    refresh = np.zeros((B, n_kv), np.int32)
    _load().kvo_query_similarity(B, n_h, n_kv, d_h, _ptr(q_cur), _ptr(q_prev), float(tau), _ptr(cos),
                                 _ptr(refresh))
    return cos, refresh


def speculative_step(q_cur, q_prev, k, v, prev_sel, *, seq_lens, k_budget, n_keep, pool, tau,
                     refresh=None, scale=None):
    """One decode step of speculative retrieval with fine-grained correction
    (FreeKV technical summary 2.A), composed from the steps above.

    q_cur, q_prev [B][n_h][d_h] (q_prev None at the first step), k, v
    [B][n_kv][s_max][d_h] float32; prev_sel = (idx, count) selected with q_prev
    (None at the first step).  The query of a step is not in the cache: it scores
    every cached key (w = 1, window_in_cache False) and the n_keep trailing tokens
    are always kept.

    Heads are corrected where the similarity says so (every head at the first
    step, or ``refresh`` when the caller fixes the decision); a corrected head
    attends over the selection made with q_cur, every other head over prev_sel.
    Returns a dict: out, lse (float64), refresh, cos (None at the first step),
    idx/count used by attention, and next_sel = the selection made with q_cur for
    every head (what the next step reuses).
    """
    B, n_h, d_h = q_cur.shape
    n_kv = k.shape[1]
    q1 = np.ascontiguousarray(q_cur[:, :, None, :])
    _, pooled = score_window(q1, k, 1, seq_lens=seq_lens, window_in_cache=False, n_keep=n_keep,
                             pool=pool, scale=scale)
    sel_idx, sel_cnt = select_topk(pooled, k_budget, n_keep, seq_lens=seq_lens)
    cos = None
    if prev_sel is None:
        ref = np.ones((B, n_kv), np.int32)
    elif refresh is not None:
        ref = np.asarray(refresh, np.int32)
    else:
        cos, ref = query_similarity(q_cur, q_prev, n_kv, tau)
    if prev_sel is None:
        use_idx, use_cnt = sel_idx, sel_cnt
    else:
        use_idx = np.where(ref[:, :, None] != 0, sel_idx, prev_sel[0]).astype(np.int32)
        use_cnt = np.where(ref != 0, sel_cnt, prev_sel[1]).astype(np.int32)
    kc, _ = gather(k, use_idx, use_cnt)
    vc, _ = gather(v, use_idx, use_cnt)
    out, lse = decode(q_cur, kc, vc, use_cnt, scale=scale)
    return dict(out=out, lse=lse, refresh=ref, cos=cos, idx=use_idx, count=use_cnt,
                next_sel=(sel_idx, sel_cnt), pooled=pooled)


def select_core(scores, core, k, n_keep, *, seq_lens=None, core_cap=None):
    """CASK role-based retention: core tokens always kept, the budget k over the
    scratch tokens only (score desc, index asc), the n_keep trailing tokens kept.

    scores [B][H][s_max] float32, core [B][s_max] (nonzero = core).  Returns
    (idx int32 [B][H][k + core_cap + n_keep], count int32 [B][H]).  core_cap is the
    room the caller leaves for core tokens (default s_max: always enough); a unit
    with more core candidates keeps the first k + core_cap candidates of the list
    "core by ascending index, then scratch in the selection order".
    """
    scores = _f32(scores)
    B, H, s_max = scores.shape
    core = np.ascontiguousarray(np.asarray(core) != 0, dtype=np.uint8)
    assert core.shape == (B, s_max)
    if core_cap is None:
        core_cap = s_max
    cap = k + core_cap + n_keep
    idx = np.empty((B, H, cap), np.int32)
    count = np.empty((B, H), np.int32)
    sl = _i32(seq_lens)
    _load().kvo_select_core(B, H, s_max, _ptr(sl), _ptr(scores), _ptr(core), int(k), int(core_cap), int(n_keep),
                            _ptr(idx), _ptr(count))
    return idx, count


def block_landmarks(k, block, *, seq_lens=None):
    """xKV 2.3 / ShadowKV-style landmarks: the mean key of each block of `block`
    tokens, k [B][n_kv][s_max][d_h] float32 -> [B][n_kv][ceil(s_max/block)][d_h]."""
    k = _f32(k)
    B, n_kv, s_max, d_h = k.shape
    n_blk = (s_max + block - 1) // block
    lm = np.zeros((B, n_kv, n_blk, d_h), np.float32)
    _load().kvo_block_landmarks(B, n_kv, s_max, d_h, _ptr(_i32(seq_lens)), _ptr(k), int(block), _ptr(lm))
    return lm


def block_scores(q, landmarks, block, n_keep, s_max, *, seq_lens=None, scale=None):
    """Group logit of each candidate block's landmark: q [B][n_h][d_h] float32.
    Returns (scores [B][n_kv][n_blk] float32, cand int32 [B] candidate blocks)."""
    q = _f32(q)
    landmarks = _f32(landmarks)
    B, n_h, d_h = q.shape
    _, n_kv, n_blk, _ = landmarks.shape
    if scale is None:
        scale = 1.0 / np.sqrt(d_h)
    sc = np.zeros((B, n_kv, n_blk), np.float32)
    cand = np.zeros(B, np.int32)
    _load().kvo_block_scores(B, n_h, n_kv, int(s_max), d_h, _ptr(_i32(seq_lens)), _ptr(q), _ptr(landmarks),
                             int(block), int(n_keep), float(scale), _ptr(sc), _ptr(cand))
    return sc, cand


def expand_blocks(idx_blk, count_blk, block, n_keep, s_max, cap, *, seq_lens=None):
    """Token indices of the kept blocks, then the tail after the last candidate block."""
    idx_blk = _i32(idx_blk)
    count_blk = _i32(count_blk)
    B, H, cap_blk = idx_blk.shape
    idx = np.empty((B, H, cap), np.int32)
    count = np.empty((B, H), np.int32)
    _load().kvo_expand_blocks(B, H, int(s_max), _ptr(_i32(seq_lens)), int(block), int(n_keep), _ptr(idx_blk),
                              _ptr(count_blk), cap_blk, _ptr(idx), _ptr(count), int(cap))
    return idx, count


def block_retrieval(q, k, v, k_blocks, block, n_keep, *, seq_lens=None, scale=None):
    """One decode step of landmark-guided block selection: landmarks -> block scores ->
    top k_blocks blocks (score desc, block index asc) -> their tokens plus the tail ->
    gather -> attention.  Returns a dict with out/lse (float64), idx/count (tokens),
    block scores and the candidate block counts."""
    B, n_kv, s_max, d_h = k.shape
    lm = block_landmarks(k, block, seq_lens=seq_lens)
    sc, cand = block_scores(q, lm, block, n_keep, s_max, seq_lens=seq_lens, scale=scale)
    bi, bc = select_topk(sc, k_blocks, 0, seq_lens=cand)
    cap = k_blocks * block + n_keep + block - 1
    idx, cnt = expand_blocks(bi, bc, block, n_keep, s_max, cap, seq_lens=seq_lens)
    kc, _ = gather(k, idx, cnt)
    vc, _ = gather(v, idx, cnt)
    out, lse = decode(q, kc, vc, cnt, scale=scale)
    return dict(out=out, lse=lse, idx=idx, count=cnt, block_scores=sc, cand=cand, landmarks=lm,
                block_idx=bi, block_count=bc)
