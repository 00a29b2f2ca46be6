"""Thin ctypes binding of ``libkvc.so`` (include/kvc.h): argument marshalling only.

Every step of the path runs in the library's HIP kernels; this module only turns
torch tensors into device pointers, allocates outputs and workspaces when the
caller does not pass them, and raises on a non-OK status.  There is no fallback:
if the library is not built, every call raises.
"""
from __future__ import annotations

import contextlib
import ctypes
import functools
import os
import threading

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "_build", "libkvc.so")

KVC_OK, KVC_ERR_INVALID_ARG, KVC_ERR_UNSUPPORTED, KVC_ERR_WORKSPACE, KVC_ERR_HIP = range(5)
KVC_F32, KVC_BF16 = 0, 1
KVC_SELECT_SHARED_HEADS = 1
KVC_SCORE_GENERIC = 1
KVC_SCORE_DEFER_ALL = 2

EXPORTED = (
    "kvc_abi_version", "kvc_status_str",
    "kvc_score_window_workspace", "kvc_score_window", "kvc_score_window_plan",
    "kvc_select_topk_workspace", "kvc_select_topk",
    "kvc_select_core_workspace", "kvc_select_core",
    "kvc_gather_compact",
    "kvc_decode_attn_workspace", "kvc_decode_attn", "kvc_decode_attn_plan", "kvc_decode_attn_noalloc",
    "kvc_query_similarity",
    "kvc_block_landmarks", "kvc_block_scores", "kvc_expand_blocks",
)


class Dims(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("s_max", ctypes.c_int32), ("seq_lens", ctypes.c_void_p),
                ("n_h", ctypes.c_int32), ("n_kv", ctypes.c_int32), ("d_h", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("unit_mask", ctypes.c_void_p)]


class KvcError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__("%s failed: %s (status %d)" % (what, status_str(status), status))


_lock = threading.Lock()
_lib = None


def lib():
    """Loads libkvc.so and declares its signatures; raises if it is not built."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise RuntimeError("libkvc.so is not built (%s); run __graft_entry__.build() first" % LIB_PATH)
            L = ctypes.CDLL(LIB_PATH)
            P, I, Z, F = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t, ctypes.c_float
            D = ctypes.POINTER(Dims)
            sig = {
                "kvc_abi_version": (I, []),
                "kvc_status_str": (ctypes.c_char_p, [I]),
                "kvc_score_window_workspace": (Z, [D, I, I]),
                "kvc_score_window": (I, [D, P, P, I, I, I, I, F, P, P, I, P, Z, P]),
                "kvc_score_window_plan": (I, [D, I, I, P]),
                "kvc_select_topk_workspace": (Z, [D, I, I, I]),
                "kvc_select_topk": (I, [D, P, I, I, I, P, P, P, P, Z, P]),
                "kvc_select_core_workspace": (Z, [D, I]),
                "kvc_select_core": (I, [D, P, P, I, I, I, P, P, P, Z, P]),
                "kvc_gather_compact": (I, [I, I, I, I, P, P, P, P, P, I, I, P, P, P, P, P]),
                "kvc_decode_attn_workspace": (Z, [D, I]),
                "kvc_decode_attn": (I, [D, P, P, P, P, I, F, P, P, P, Z, P]),
                "kvc_decode_attn_plan": (I, [D, I, P]),
                "kvc_decode_attn_noalloc": (I, [D, P, P, P, P, I, F, P, P, P]),
                "kvc_query_similarity": (I, [D, P, P, ctypes.c_double, P, P, P, P]),
                "kvc_block_landmarks": (I, [D, P, I, P, P]),
                "kvc_block_scores": (I, [D, P, P, I, I, F, P, P, P]),
                "kvc_expand_blocks": (I, [I, I, I, P, I, I, P, P, I, P, P, I, P]),
            }
            for name, (res, args) in sig.items():
                fn = getattr(L, name)
                fn.restype = res
                fn.argtypes = args
            _lib = L
    return _lib


def status_str(status: int) -> str:
    return lib().kvc_status_str(int(status)).decode()


def _check(status: int, what: str):
    if status != KVC_OK:
        raise KvcError(status, what)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return KVC_BF16
    if t.dtype == torch.float32:
        return KVC_F32
    raise TypeError("unsupported dtype %s (bf16 or fp32)" % t.dtype)


def _ptr(t):
    return None if t is None else t.data_ptr()


def _dev(t: torch.Tensor, name: str):
    if not t.is_cuda:
        raise ValueError("%s must be a device tensor" % name)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    return t


def _stream():
    """The hipStream_t of the launch: torch's current stream (which on_stream sets)."""
    return torch.cuda.current_stream().cuda_stream


def on_stream(fn):
    """Runs a binding call with its ``stream=`` argument (a torch.cuda.Stream) made
    torch's current stream, so that the temporaries the call allocates or fills
    (workspaces, outputs, host-to-device copies of lengths) are ordered on the same
    stream as its kernels and released to that stream's pool."""
    @functools.wraps(fn)
    def call(*args, stream=None, **kw):
        if stream is None:
            ctx = contextlib.nullcontext()
        elif isinstance(stream, torch.cuda.Stream):
            ctx = torch.cuda.stream(stream)
        else:
            raise TypeError("stream must be a torch.cuda.Stream")
        with ctx:
            return fn(*args, **kw)
    return call


def _seq_lens(seq_lens, device):
    if seq_lens is None:
        return None
    if isinstance(seq_lens, torch.Tensor) and seq_lens.is_cuda:
        if seq_lens.dtype != torch.int32 or not seq_lens.is_contiguous():
            raise ValueError("seq_lens must be a contiguous int32 device tensor")
        return seq_lens
    return torch.as_tensor(seq_lens, dtype=torch.int32).to(device)


def _mask(unit_mask, shape, device, name="unit_mask"):
    """A per-unit int32 device array (unit mask or budgets) of the given shape, or None."""
    if unit_mask is None:
        return None
    if not (isinstance(unit_mask, torch.Tensor) and unit_mask.is_cuda and unit_mask.dtype == torch.int32
            and unit_mask.is_contiguous()):
        raise ValueError("%s must be a contiguous int32 device tensor" % name)
    if tuple(unit_mask.shape) != tuple(shape):
        raise ValueError("%s must have shape %s" % (name, tuple(shape)))
    return unit_mask


def make_dims(batch, s_max, n_h, n_kv, d_h, dtype_code, seq_lens=None, unit_mask=None) -> Dims:
    return Dims(int(batch), int(s_max), _ptr(seq_lens), int(n_h), int(n_kv), int(d_h), int(dtype_code),
                _ptr(unit_mask))


# ------------------------------------------------------------------------------- score

def score_window_workspace(dims: Dims, w: int, flags: int = 0) -> int:
    return int(lib().kvc_score_window_workspace(ctypes.byref(dims), int(w), int(flags)))


def score_window_plan(dims: Dims, w: int, flags: int = 0) -> dict:
    """kvc_score_window_plan: the launch configuration of kvc_score_window for dims."""
    out = (ctypes.c_int32 * 6)()
    _check(lib().kvc_score_window_plan(ctypes.byref(dims), int(w), int(flags), out), "kvc_score_window_plan")
    return {"mfma": bool(out[0]), "rt": int(out[1]), "chunk_tokens": int(out[2]), "chunks_per_unit": int(out[3]),
            "single_pass": bool(out[4]), "folded_merge": bool(out[5])}


@on_stream
def score_window(q_win, k, w, *, seq_lens=None, window_in_cache=True, n_keep=None, pool=1, scale=0.0,
                 generic=False, defer_all=False, raw=None, pooled=None, ws=None, unit_mask=None):
    """kvc_score_window: q_win [B][n_h][w][d_h], k [B][n_kv][s_max][d_h] -> (raw, pooled) fp32.
    With unit_mask ([B][n_kv] int32), units whose entry is 0 are skipped."""
    _dev(q_win, "q_win")
    _dev(k, "k")
    B, n_h, w_, d_h = q_win.shape
    _, n_kv, s_max, _ = k.shape
    if w_ != w or k.dtype != q_win.dtype:
        raise ValueError("q_win/k shapes or dtypes disagree")
    sl = _seq_lens(seq_lens, k.device)
    um = _mask(unit_mask, (B, n_kv), k.device)
    dims = make_dims(B, s_max, n_h, n_kv, d_h, _dtype_code(k), sl, um)
    flags = (KVC_SCORE_GENERIC if generic else 0) | (KVC_SCORE_DEFER_ALL if defer_all else 0)
    if n_keep is None:
        n_keep = w
    if raw is None:
        raw = torch.empty((B, n_kv, s_max), dtype=torch.float32, device=k.device)
    if pooled is None:
        pooled = torch.empty((B, n_kv, s_max), dtype=torch.float32, device=k.device)
    need = score_window_workspace(dims, w, flags)
    if ws is None:
        ws = torch.zeros(max(need, 256), dtype=torch.uint8, device=k.device)
    st = lib().kvc_score_window(ctypes.byref(dims), _ptr(q_win), _ptr(k), int(w), int(bool(window_in_cache)),
                                int(n_keep), int(pool), float(scale), _ptr(raw), _ptr(pooled), flags,
                                _ptr(ws), ws.numel() * ws.element_size(), _stream())
    _check(st, "kvc_score_window")
    return raw, pooled


# ------------------------------------------------------------------------------ select

def select_topk_workspace(dims: Dims, k: int, n_keep: int, flags: int = 0) -> int:
    return int(lib().kvc_select_topk_workspace(ctypes.byref(dims), int(k), int(n_keep), int(flags)))


@on_stream
def select_topk(scores, k, n_keep, *, seq_lens=None, shared_heads=False, idx=None, count=None, ws=None,
                unit_mask=None, k_per_unit=None):
    """kvc_select_topk: scores [B][n_kv][s_max] fp32 -> (idx [B][H][k+n_keep], count [B][H]) int32.
    With unit_mask ([B][n_kv] int32), units whose entry is 0 are skipped; with k_per_unit
    ([B][H] int32 device tensor), unit u takes min(k_per_unit[u], k) candidates."""
    _dev(scores, "scores")
    if scores.dtype != torch.float32:
        raise TypeError("scores must be float32")
    B, n_kv, s_max = scores.shape
    sl = _seq_lens(seq_lens, scores.device)
    um = _mask(unit_mask, (B, n_kv), scores.device)
    dims = make_dims(B, s_max, n_kv, n_kv, 128, KVC_F32, sl, um)
    flags = KVC_SELECT_SHARED_HEADS if shared_heads else 0
    H = 1 if shared_heads else n_kv
    cap = k + n_keep
    if idx is None:
        idx = torch.empty((B, H, cap), dtype=torch.int32, device=scores.device)
    if count is None:
        count = torch.empty((B, H), dtype=torch.int32, device=scores.device)
    need = select_topk_workspace(dims, k, n_keep, flags)
    if ws is None and need:
        ws = torch.zeros(need, dtype=torch.uint8, device=scores.device)
    kpu = _mask(k_per_unit, (B, H), scores.device, "k_per_unit")
    st = lib().kvc_select_topk(ctypes.byref(dims), _ptr(scores), int(k), int(n_keep), flags, _ptr(kpu),
                               _ptr(idx), _ptr(count), _ptr(ws),
                               0 if ws is None else ws.numel() * ws.element_size(), _stream())
    _check(st, "kvc_select_topk")
    return idx, count


def select_core_workspace(dims: Dims, n_keep: int) -> int:
    return int(lib().kvc_select_core_workspace(ctypes.byref(dims), int(n_keep)))


@on_stream
def select_core(scores, core, k, core_cap, n_keep, *, seq_lens=None, idx=None, count=None, ws=None,
                unit_mask=None):
    """kvc_select_core: scores [B][n_kv][s_max] fp32, core [B][s_max] uint8 ->
    (idx [B][n_kv][k+core_cap+n_keep], count [B][n_kv]) int32."""
    _dev(scores, "scores")
    _dev(core, "core")
    if scores.dtype != torch.float32 or core.dtype != torch.uint8:
        raise TypeError("scores must be float32 and core uint8")
    B, n_kv, s_max = scores.shape
    if tuple(core.shape) != (B, s_max):
        raise ValueError("core must have shape (B, s_max)")
    sl = _seq_lens(seq_lens, scores.device)
    um = _mask(unit_mask, (B, n_kv), scores.device)
    dims = make_dims(B, s_max, n_kv, n_kv, 128, KVC_F32, sl, um)
    cap = k + core_cap + n_keep
    if idx is None:
        idx = torch.empty((B, n_kv, cap), dtype=torch.int32, device=scores.device)
    if count is None:
        count = torch.empty((B, n_kv), dtype=torch.int32, device=scores.device)
    need = select_core_workspace(dims, n_keep)
    if ws is None:
        ws = torch.zeros(max(need, 256), dtype=torch.uint8, device=scores.device)
    st = lib().kvc_select_core(ctypes.byref(dims), _ptr(scores), _ptr(core), int(k), int(core_cap), int(n_keep),
                               _ptr(idx), _ptr(count), _ptr(ws), ws.numel() * ws.element_size(), _stream())
    _check(st, "kvc_select_core")
    return idx, count


# ------------------------------------------------------------------------------ gather

@on_stream
def gather_compact(src0, idx, count, *, src1=None, src_pos=None, dst0=None, dst1=None, pos_out=None,
                   want_pos=True, unit_mask=None):
    """kvc_gather_compact: src [B][heads][s_max][...] -> dst [B][heads][cap][...] (+ pos_out).
    With unit_mask ([B][idx_heads] int32), lists whose entry is 0 are skipped."""
    _dev(src0, "src0")
    _dev(idx, "idx")
    _dev(count, "count")
    B, heads, s_max = src0.shape[:3]
    row_shape = tuple(src0.shape[3:])
    row_bytes = src0.element_size()
    for s in row_shape:
        row_bytes *= s
    idx_heads, cap = idx.shape[1], idx.shape[2]
    if dst0 is None:
        dst0 = torch.empty((B, heads, cap) + row_shape, dtype=src0.dtype, device=src0.device)
    if src1 is not None and dst1 is None:
        dst1 = torch.empty_like(dst0)
    if want_pos and pos_out is None:
        pos_out = torch.empty((B, heads, cap), dtype=torch.int32, device=src0.device)
    st = lib().kvc_gather_compact(int(B), int(heads), int(s_max), int(row_bytes), _ptr(src0), _ptr(src1),
                                  _ptr(src_pos), _ptr(idx), _ptr(count), int(idx_heads), int(cap), _ptr(dst0),
                                  _ptr(dst1), _ptr(pos_out), _ptr(_mask(unit_mask, (B, idx_heads), src0.device)),
                                  _stream())
    _check(st, "kvc_gather_compact")
    return dst0, dst1, pos_out


# ------------------------------------------------------------------------------ decode

def decode_attn_workspace(dims: Dims, cap: int) -> int:
    return int(lib().kvc_decode_attn_workspace(ctypes.byref(dims), int(cap)))


def decode_attn_plan(dims: Dims, cap: int) -> dict:
    """kvc_decode_attn_plan: the launch configuration of kvc_decode_attn for dims and cap."""
    out = (ctypes.c_int32 * 4)()
    _check(lib().kvc_decode_attn_plan(ctypes.byref(dims), int(cap), out), "kvc_decode_attn_plan")
    return {"n_splits": int(out[0]), "split_tokens": int(out[1]), "head_chunk": int(out[2]), "fused": bool(out[3])}


@on_stream
def decode_attn(q, kc, vc, count, *, scale=0.0, out=None, lse=None, want_lse=True, ws=None):
    """kvc_decode_attn: q [B][n_h][d_h], kc/vc [B][n_kv][cap][d_h] -> (out [B][n_h][d_h], lse [B][n_h])."""
    for t, nm in ((q, "q"), (kc, "kc"), (vc, "vc"), (count, "count")):
        _dev(t, nm)
    B, n_h, d_h = q.shape
    _, n_kv, cap, _ = kc.shape
    dims = make_dims(B, 1, n_h, n_kv, d_h, _dtype_code(q))
    if out is None:
        out = torch.empty((B, n_h, d_h), dtype=q.dtype, device=q.device)
    if want_lse and lse is None:
        lse = torch.empty((B, n_h), dtype=torch.float32, device=q.device)
    need = decode_attn_workspace(dims, cap)
    if ws is None:
        ws = torch.zeros(max(need, 256), dtype=torch.uint8, device=q.device)
    st = lib().kvc_decode_attn(ctypes.byref(dims), _ptr(q), _ptr(kc), _ptr(vc), _ptr(count), int(cap),
                               float(scale), _ptr(out), _ptr(lse), _ptr(ws), ws.numel() * ws.element_size(),
                               _stream())
    _check(st, "kvc_decode_attn")
    return out, lse


DECODE_NOALLOC_LIMIT = 4 << 20   # bytes of the library's static decode scratch, per GPU


@on_stream
def decode_attn_noalloc(q, kc, vc, count, out, lse=None, *, scale=0.0):
    """kvc_decode_attn_noalloc: decode attention with the library's static scratch
    (no workspace, nothing allocated here either: out and lse are the caller's)."""
    for t, nm in ((q, "q"), (kc, "kc"), (vc, "vc"), (count, "count"), (out, "out")):
        _dev(t, nm)
    B, n_h, d_h = q.shape
    _, n_kv, cap, _ = kc.shape
    dims = make_dims(B, 1, n_h, n_kv, d_h, _dtype_code(q))
    st = lib().kvc_decode_attn_noalloc(ctypes.byref(dims), _ptr(q), _ptr(kc), _ptr(vc), _ptr(count), int(cap),
                                       float(scale), _ptr(out), _ptr(lse), _stream())
    _check(st, "kvc_decode_attn_noalloc")
    return out, lse


# ----------------------------------------------------------------------- query similarity

@on_stream
def query_similarity(q_cur, q_prev, n_kv, tau, *, cos=None, refresh=None, keep=None, want_cos=True):
    """kvc_query_similarity: q_cur, q_prev [B][n_h][d_h] -> (cos [B][n_h] fp32, refresh, keep [B][n_kv] int32)."""
    _dev(q_cur, "q_cur")
    _dev(q_prev, "q_prev")
    if q_cur.shape != q_prev.shape or q_cur.dtype != q_prev.dtype:
        raise ValueError("q_cur/q_prev shapes or dtypes disagree")
    B, n_h, d_h = q_cur.shape
    dims = make_dims(B, 1, n_h, n_kv, d_h, _dtype_code(q_cur))
    dev = q_cur.device
    if want_cos and cos is None:
        cos = torch.empty((B, n_h), dtype=torch.float32, device=dev)
    if refresh is None:
        refresh = torch.empty((B, n_kv), dtype=torch.int32, device=dev)
    if keep is None:
        keep = torch.empty((B, n_kv), dtype=torch.int32, device=dev)
    st = lib().kvc_query_similarity(ctypes.byref(dims), _ptr(q_cur), _ptr(q_prev), float(tau), _ptr(cos),
                                    _ptr(refresh), _ptr(keep), _stream())
    _check(st, "kvc_query_similarity")
    return cos, refresh, keep


# ------------------------------------------------------- landmark-guided block selection

@on_stream
def block_landmarks(k, block, *, seq_lens=None, out=None):
    """kvc_block_landmarks: k [B][n_kv][s_max][d_h] -> mean keys [B][n_kv][ceil(s_max/block)][d_h] fp32."""
    _dev(k, "k")
    B, n_kv, s_max, d_h = k.shape
    n_blk = (s_max + block - 1) // block
    sl = _seq_lens(seq_lens, k.device)
    dims = make_dims(B, s_max, n_kv, n_kv, d_h, _dtype_code(k), sl)
    if out is None:
        out = torch.empty((B, n_kv, n_blk, d_h), dtype=torch.float32, device=k.device)
    st = lib().kvc_block_landmarks(ctypes.byref(dims), _ptr(k), int(block), _ptr(out), _stream())
    _check(st, "kvc_block_landmarks")
    return out


@on_stream
def block_scores(q, landmarks, block, n_keep, s_max, *, seq_lens=None, scale=0.0, scores=None, cand=None):
    """kvc_block_scores: q [B][n_h][d_h], landmarks -> (scores [B][n_kv][n_blk] fp32, cand [B] int32)."""
    _dev(q, "q")
    _dev(landmarks, "landmarks")
    B, n_h, d_h = q.shape
    _, n_kv, n_blk, _ = landmarks.shape
    sl = _seq_lens(seq_lens, q.device)
    dims = make_dims(B, s_max, n_h, n_kv, d_h, _dtype_code(q), sl)
    if scores is None:
        scores = torch.empty((B, n_kv, n_blk), dtype=torch.float32, device=q.device)
    if cand is None:
        cand = torch.empty((B,), dtype=torch.int32, device=q.device)
    st = lib().kvc_block_scores(ctypes.byref(dims), _ptr(q), _ptr(landmarks), int(block), int(n_keep), float(scale),
                                _ptr(scores), _ptr(cand), _stream())
    _check(st, "kvc_block_scores")
    return scores, cand


@on_stream
def expand_blocks(idx_blocks, count_blocks, block, n_keep, s_max, cap, *, seq_lens=None, idx=None, count=None):
    """kvc_expand_blocks: kept blocks [B][H][cap_blocks] -> token indices [B][H][cap], count [B][H]."""
    _dev(idx_blocks, "idx_blocks")
    _dev(count_blocks, "count_blocks")
    B, H, cap_blk = idx_blocks.shape
    sl = _seq_lens(seq_lens, idx_blocks.device)
    if idx is None:
        idx = torch.empty((B, H, cap), dtype=torch.int32, device=idx_blocks.device)
    if count is None:
        count = torch.empty((B, H), dtype=torch.int32, device=idx_blocks.device)
    st = lib().kvc_expand_blocks(int(B), int(H), int(s_max), _ptr(sl), int(block), int(n_keep), _ptr(idx_blocks),
                                 _ptr(count_blocks), int(cap_blk), _ptr(idx), _ptr(count), int(cap), _stream())
    _check(st, "kvc_expand_blocks")
    return idx, count
