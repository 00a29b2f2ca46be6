"""C ABI checks that need no GPU: the library loads, exports every declared symbol,
and rejects every invalid argument before any HIP call."""
import ctypes
import os
import re

import pytest
import torch

from sparse_decode_amd import kvc

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kvc.h")

BAD = 0x1000  # a non-null, 16-byte aligned address that is never dereferenced on these paths


def _declared():
    txt = open(HEADER).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(kvc_[a-z_]+)\s*\(", txt)))


def test_every_declared_symbol_is_exported():
    L = kvc.lib()
    declared = _declared()
    assert set(declared) == set(kvc.EXPORTED)
    for name in declared:
        assert hasattr(L, name), name


def test_version_and_status_strings():
    assert kvc.lib().kvc_abi_version() == 4
    seen = set()
    for s in range(5):
        txt = kvc.status_str(s)
        assert txt and txt not in seen
        seen.add(txt)
    assert kvc.status_str(99) == "unknown status"


def _dims(**kw):
    base = dict(batch=1, s_max=1024, n_h=32, n_kv=8, d_h=128, dtype_code=kvc.KVC_BF16)
    base.update(kw)
    return kvc.make_dims(base["batch"], base["s_max"], base["n_h"], base["n_kv"], base["d_h"], base["dtype_code"])


def _score(dims, w=32, **kw):
    a = dict(q=BAD, k=BAD, wic=1, n_keep=32, pool=7, scale=0.0, raw=BAD, pooled=BAD, flags=0, ws=BAD,
             ws_bytes=1 << 40)
    a.update(kw)
    return kvc.lib().kvc_score_window(ctypes.byref(dims) if dims is not None else None, a["q"], a["k"], w,
                                      a["wic"], a["n_keep"], a["pool"], a["scale"], a["raw"], a["pooled"],
                                      a["flags"], a["ws"], a["ws_bytes"], None)


def test_score_rejects_invalid_arguments():
    E, U, W = kvc.KVC_ERR_INVALID_ARG, kvc.KVC_ERR_UNSUPPORTED, kvc.KVC_ERR_WORKSPACE
    assert _score(None) == E
    assert _score(_dims(batch=0)) == E
    assert _score(_dims(s_max=0)) == E
    assert _score(_dims(n_h=30)) == E            # n_h % n_kv != 0
    assert _score(_dims(dtype_code=7)) == E
    assert _score(_dims(d_h=96)) == U
    assert _score(_dims(), w=0) == E
    assert _score(_dims(), w=2048) == E
    assert _score(_dims(), q=None) == E
    assert _score(_dims(), raw=None) == E
    assert _score(_dims(), pooled=None) == E
    assert _score(_dims(), pool=4) == E          # even pool kernel
    assert _score(_dims(), pool=0) == E
    assert _score(_dims(), n_keep=-1) == E
    assert _score(_dims(), scale=-1.0) == E
    assert _score(_dims(), scale=float("nan")) == E
    assert _score(_dims(), flags=4) == E
    assert _score(_dims(), k=BAD + 4) == E       # misaligned
    assert _score(_dims(), ws=None) == W
    need = kvc.score_window_workspace(_dims(), 32)
    assert need > 0
    assert _score(_dims(), ws_bytes=need - 1) == W


def test_workspace_queries():
    d = _dims()
    assert kvc.score_window_workspace(_dims(batch=0), 32) == 0
    small = kvc.score_window_workspace(_dims(s_max=4096), 32)
    big = kvc.score_window_workspace(_dims(s_max=131072), 32)
    assert 0 < small <= big
    gen = kvc.score_window_workspace(_dims(s_max=4096), 32, kvc.KVC_SCORE_GENERIC)
    assert kvc.score_window_workspace(_dims(s_max=(1 << 22) + 1), 32) == 0
    assert gen >= 32 * 4 * 4096 * 4 * 8     # stored logits
    plain = kvc.select_topk_workspace(d, 64, 16)
    assert plain >= 8 * 5120 * 4                  # three radix histograms (2048 + 2048 + 1024) per unit
    shared = kvc.select_topk_workspace(d, 64, 16, kvc.KVC_SELECT_SHARED_HEADS)
    assert shared >= 1024 * 4 + 5120 * 4          # head sum + one unit's histograms
    assert kvc.select_topk_workspace(_dims(s_max=131072), 1311, 32) > plain
    assert kvc.select_topk_workspace(d, -1, 16) == 0
    assert kvc.decode_attn_workspace(d, 2080) > 0
    assert kvc.decode_attn_workspace(d, 2080) <= kvc.decode_attn_workspace(d, 8192)
    assert kvc.decode_attn_workspace(d, 0) == 0


def _select(dims, k=64, n_keep=16, flags=0, scores=BAD, idx=BAD, count=BAD, ws=None, ws_bytes=0):
    return kvc.lib().kvc_select_topk(ctypes.byref(dims) if dims is not None else None, scores, k, n_keep, flags,
                                     None, idx, count, ws, ws_bytes, None)


def test_select_rejects_invalid_arguments():
    E, W = kvc.KVC_ERR_INVALID_ARG, kvc.KVC_ERR_WORKSPACE
    assert _select(None) == E
    assert _select(_dims(batch=0)) == E
    assert _select(_dims(), k=-1) == E
    assert _select(_dims(), k=0, n_keep=0) == E
    assert _select(_dims(), flags=2) == E
    assert _select(_dims(), scores=None) == E
    assert _select(_dims(), idx=None) == E
    assert _select(_dims(), count=None) == E
    assert _select(_dims()) == W                 # every selection needs its workspace
    assert _select(_dims(), flags=kvc.KVC_SELECT_SHARED_HEADS) == W
    need = kvc.select_topk_workspace(_dims(), 64, 16)
    assert _select(_dims(), ws=BAD, ws_bytes=need - 1) == W


def _gather(**kw):
    a = dict(batch=1, heads=8, s_max=1024, row_bytes=256, src0=BAD, src1=BAD, src_pos=None, idx=BAD, count=BAD,
             idx_heads=8, cap=80, dst0=BAD, dst1=BAD, pos=BAD, mask=None)
    a.update(kw)
    return kvc.lib().kvc_gather_compact(a["batch"], a["heads"], a["s_max"], a["row_bytes"], a["src0"], a["src1"],
                                        a["src_pos"], a["idx"], a["count"], a["idx_heads"], a["cap"], a["dst0"],
                                        a["dst1"], a["pos"], a["mask"], None)


def test_gather_rejects_invalid_arguments():
    E, U = kvc.KVC_ERR_INVALID_ARG, kvc.KVC_ERR_UNSUPPORTED
    assert _gather(batch=0) == E
    assert _gather(cap=0) == E
    assert _gather(idx_heads=3) == E
    assert _gather(src0=None) == E
    assert _gather(idx=None) == E
    assert _gather(dst1=None) == E              # src1 given without dst1
    assert _gather(row_bytes=8) == E
    assert _gather(row_bytes=24) == U           # not a multiple of 16
    assert _gather(row_bytes=48) == U           # 3 vectors: neither a power of two nor a multiple of 256
    assert _gather(src0=BAD + 8) == U           # misaligned


def _decode(dims, cap=80, **kw):
    a = dict(q=BAD, kc=BAD, vc=BAD, count=BAD, scale=0.0, out=BAD, lse=None, ws=BAD, ws_bytes=1 << 40)
    a.update(kw)
    return kvc.lib().kvc_decode_attn(ctypes.byref(dims) if dims is not None else None, a["q"], a["kc"], a["vc"],
                                     a["count"], cap, a["scale"], a["out"], a["lse"], a["ws"], a["ws_bytes"], None)


def test_decode_plan_query():
    # one layer of the 32-layer MHA workload after compaction (1024 + 32 tokens per head)
    mha = kvc.decode_attn_plan(_dims(batch=2, n_h=32, n_kv=32), 1056)
    assert mha["fused"] and mha["head_chunk"] == 1 and mha["n_splits"] * mha["split_tokens"] >= 1056
    # the last arrival folds up to 64 splits of one head, 8 of eight heads (a register
    # budget per thread); more splits go to the merge kernel
    assert kvc.decode_attn_plan(_dims(batch=2, n_h=4, n_kv=4), 4096) == \
        {"n_splits": 64, "split_tokens": 64, "head_chunk": 1, "fused": True}
    assert kvc.decode_attn_plan(_dims(batch=2, n_h=32, n_kv=4), 4096) == \
        {"n_splits": 64, "split_tokens": 64, "head_chunk": 8, "fused": False}
    long_few = kvc.decode_attn_plan(_dims(batch=2, n_h=8, n_kv=1), 9000)
    assert long_few["n_splits"] > 64 and not long_few["fused"]
    for p in (mha, long_few):
        assert p["split_tokens"] % 64 == 0
    out = (ctypes.c_int32 * 4)()
    E = kvc.KVC_ERR_INVALID_ARG
    assert kvc.lib().kvc_decode_attn_plan(None, 80, out) == E
    assert kvc.lib().kvc_decode_attn_plan(ctypes.byref(_dims()), 0, out) == E
    assert kvc.lib().kvc_decode_attn_plan(ctypes.byref(_dims()), 80, None) == E


def test_decode_rejects_invalid_arguments():
    E, U, W = kvc.KVC_ERR_INVALID_ARG, kvc.KVC_ERR_UNSUPPORTED, kvc.KVC_ERR_WORKSPACE
    assert _decode(None) == E
    assert _decode(_dims(n_kv=5)) == E
    assert _decode(_dims(d_h=80)) == U
    assert _decode(_dims(), cap=0) == E
    assert _decode(_dims(), q=None) == E
    assert _decode(_dims(), out=None) == E
    assert _decode(_dims(), scale=-2.0) == E
    assert _decode(_dims(), scale=float("nan")) == E
    assert _decode(_dims(), vc=BAD + 2) == E
    assert _decode(_dims(), ws=None) == W
    assert _decode(_dims(), ws_bytes=16) == W


@pytest.mark.skipif(torch.cuda.is_available(), reason="checks the error path of a host without a GPU")
def test_valid_call_without_gpu_reports_hip_error():
    # every argument passes validation, so the call reaches the HIP runtime, which has no device
    assert _gather() == kvc.KVC_ERR_HIP
    assert _select(_dims(), ws=BAD, ws_bytes=kvc.select_topk_workspace(_dims(), 64, 16)) == kvc.KVC_ERR_HIP
    assert _decode(_dims()) == kvc.KVC_ERR_HIP
    assert _score(_dims()) == kvc.KVC_ERR_HIP


def _similarity(dims, **kw):
    a = dict(q_cur=BAD, q_prev=BAD, tau=0.9, cos=BAD, refresh=BAD, keep=None)
    a.update(kw)
    return kvc.lib().kvc_query_similarity(ctypes.byref(dims) if dims is not None else None, a["q_cur"], a["q_prev"],
                                          a["tau"], a["cos"], a["refresh"], a["keep"], None)


def test_similarity_rejects_invalid_arguments():
    E, U = kvc.KVC_ERR_INVALID_ARG, kvc.KVC_ERR_UNSUPPORTED
    assert _similarity(None) == E
    assert _similarity(_dims(n_kv=5)) == E
    assert _similarity(_dims(d_h=80)) == U
    assert _similarity(_dims(), q_cur=None) == E
    assert _similarity(_dims(), refresh=None) == E
    assert _similarity(_dims(), q_prev=BAD + 4) == E
    assert _similarity(_dims(), tau=float("nan")) == E
    assert _similarity(_dims(), tau=float("inf")) == E
    # valid arguments reach the launch, which fails without a device
    assert _similarity(_dims(), tau=-3.0) == kvc.KVC_ERR_HIP


def test_shared_head_selection_takes_no_unit_mask():
    d = _dims()
    d.unit_mask = BAD
    assert kvc.select_topk_workspace(d, 64, 16, kvc.KVC_SELECT_SHARED_HEADS) == 0
    assert _select(d, flags=kvc.KVC_SELECT_SHARED_HEADS) == kvc.KVC_ERR_INVALID_ARG


def _select_core(dims, k=64, core_cap=32, n_keep=16, scores=BAD, core=BAD, idx=BAD, count=BAD, ws=BAD,
                 ws_bytes=1 << 40):
    return kvc.lib().kvc_select_core(ctypes.byref(dims) if dims is not None else None, scores, core, k, core_cap,
                                     n_keep, idx, count, ws, ws_bytes, None)


def test_select_core_rejects_invalid_arguments():
    E, W = kvc.KVC_ERR_INVALID_ARG, kvc.KVC_ERR_WORKSPACE
    assert _select_core(None) == E
    assert _select_core(_dims(batch=0)) == E
    assert _select_core(_dims(), k=-1) == E
    assert _select_core(_dims(), core_cap=-1) == E
    assert _select_core(_dims(), k=0, core_cap=0, n_keep=0) == E
    assert _select_core(_dims(), core=None) == E
    assert _select_core(_dims(), idx=None) == E
    assert _select_core(_dims(), ws=None) == W
    need = kvc.select_core_workspace(_dims(), 16)
    assert need > kvc.select_topk_workspace(_dims(), 64, 16)
    assert _select_core(_dims(), ws_bytes=need - 1) == W
    assert kvc.select_core_workspace(_dims(), -1) == 0
    # valid arguments reach the launch, which fails without a device
    assert _select_core(_dims(), ws_bytes=need) == kvc.KVC_ERR_HIP


def test_block_selection_rejects_invalid_arguments():
    E, U = kvc.KVC_ERR_INVALID_ARG, kvc.KVC_ERR_UNSUPPORTED
    L = kvc.lib()
    d = _dims()
    assert L.kvc_block_landmarks(None, BAD, 16, BAD, None) == E
    assert L.kvc_block_landmarks(ctypes.byref(d), None, 16, BAD, None) == E
    assert L.kvc_block_landmarks(ctypes.byref(d), BAD, 0, BAD, None) == E
    assert L.kvc_block_landmarks(ctypes.byref(d), BAD, 2048, BAD, None) == E     # block > s_max
    assert L.kvc_block_landmarks(ctypes.byref(_dims(d_h=80)), BAD, 16, BAD, None) == U
    assert L.kvc_block_scores(ctypes.byref(d), BAD, BAD, 16, 32, 0.0, BAD, None, None) == E   # no cand
    assert L.kvc_block_scores(ctypes.byref(d), BAD, BAD, 16, -1, 0.0, BAD, BAD, None) == E
    assert L.kvc_block_scores(ctypes.byref(d), BAD, BAD, 16, 32, float("nan"), BAD, BAD, None) == E
    assert L.kvc_expand_blocks(1, 8, 1024, None, 16, 32, BAD, BAD, 0, BAD, BAD, 80, None) == E
    assert L.kvc_expand_blocks(1, 8, 1024, None, 0, 32, BAD, BAD, 4, BAD, BAD, 80, None) == E
    assert L.kvc_expand_blocks(1, 8, 1024, None, 16, 32, None, BAD, 4, BAD, BAD, 80, None) == E
    # valid arguments reach the launch, which fails without a device
    assert L.kvc_block_landmarks(ctypes.byref(d), BAD, 16, BAD, None) == kvc.KVC_ERR_HIP
    assert L.kvc_block_scores(ctypes.byref(d), BAD, BAD, 16, 32, 0.0, BAD, BAD, None) == kvc.KVC_ERR_HIP
    assert L.kvc_expand_blocks(1, 8, 1024, None, 16, 32, BAD, BAD, 4, BAD, BAD, 80, None) == kvc.KVC_ERR_HIP


def test_score_plan_query():
    # the launch configuration depends on the shapes only (host logic, no GPU)
    E = kvc.KVC_ERR_INVALID_ARG
    cfg2_fold = kvc.score_window_plan(_dims(batch=32, s_max=32768), 32)
    assert cfg2_fold == {"mfma": True, "rt": 8, "chunk_tokens": 2048, "chunks_per_unit": 16, "single_pass": False,
                         "folded_merge": False}
    one_layer = kvc.score_window_plan(_dims(batch=1, s_max=32768), 32)
    assert one_layer["rt"] == 8 and one_layer["chunk_tokens"] == 256 and one_layer["chunks_per_unit"] == 128
    assert not one_layer["single_pass"] and not one_layer["folded_merge"]
    # 17..32 rows per KV head, up to 131072 tokens: K read once, 1024-token items
    mha = kvc.score_window_plan(_dims(batch=2, s_max=65536, n_h=32, n_kv=32), 32)
    assert mha == {"mfma": True, "rt": 2, "chunk_tokens": 1024, "chunks_per_unit": 64, "single_pass": True,
                   "folded_merge": False}
    mha_after = kvc.score_window_plan(_dims(batch=2, s_max=13140, n_h=32, n_kv=32), 32)
    assert mha_after["single_pass"] and mha_after["chunks_per_unit"] == 13
    assert kvc.score_window_plan(_dims(batch=2, s_max=131072, n_h=32, n_kv=32), 32)["single_pass"]
    assert not kvc.score_window_plan(_dims(batch=2, s_max=131073, n_h=32, n_kv=32), 32)["single_pass"]
    assert not kvc.score_window_plan(_dims(batch=2, s_max=4096, n_h=32, n_kv=32), 16)["single_pass"]   # R = 16
    # one query per head over 16 sequences: 8 items per KV head in one round of
    # work-groups, merged by the last first-pass work-group of each
    one_query = kvc.score_window_plan(_dims(batch=16, s_max=16384), 1)
    assert one_query["rt"] == 1 and not one_query["single_pass"] and one_query["chunks_per_unit"] == 8
    assert one_query["folded_merge"]
    assert not kvc.score_window_plan(_dims(batch=16, s_max=16385), 1)["folded_merge"]      # 9 items
    assert kvc.score_window_plan(_dims(dtype_code=kvc.KVC_F32), 32)["mfma"] is False
    assert kvc.score_window_plan(_dims(), 32, kvc.KVC_SCORE_GENERIC)["mfma"] is False
    assert kvc.score_window_plan(_dims(), 32, kvc.KVC_SCORE_DEFER_ALL) == kvc.score_window_plan(_dims(), 32)
    out = (ctypes.c_int32 * 6)()
    assert kvc.lib().kvc_score_window_plan(None, 32, 0, out) == E
    assert kvc.lib().kvc_score_window_plan(ctypes.byref(_dims()), 0, 0, out) == E
    assert kvc.lib().kvc_score_window_plan(ctypes.byref(_dims()), 32, 0, None) == E
    assert kvc.lib().kvc_score_window_plan(ctypes.byref(_dims()), 32, 4, out) == E


def test_decode_noalloc_rejects_invalid_arguments():
    E, W = kvc.KVC_ERR_INVALID_ARG, kvc.KVC_ERR_WORKSPACE
    L = kvc.lib()

    def call(dims, cap=2080, q=BAD, out=BAD):
        return L.kvc_decode_attn_noalloc(ctypes.byref(dims) if dims is not None else None, q, BAD, BAD, BAD, cap,
                                         0.0, out, None, None)
    assert call(None) == E
    assert call(_dims(), cap=0) == E
    assert call(_dims(), q=None) == E
    assert call(_dims(), out=BAD + 4) == E
    big = _dims(batch=1024)
    assert kvc.decode_attn_workspace(big, 128) > kvc.DECODE_NOALLOC_LIMIT
    assert call(big, cap=128) == W
