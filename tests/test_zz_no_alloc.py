"""kvc_decode_attn_noalloc, the decode entry point that allocates nothing (its split
partials live in the library's static per-GPU scratch): the same results as
kvc_decode_attn, bit for bit, on consecutive calls of different sizes, and a clear
rejection of shapes whose partials exceed the scratch."""
import ctypes
import sys

import numpy as np
import pytest
import torch

from sparse_decode_amd import kvc

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def _randn(shape, seed, dtype):
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    return torch.randn(shape, generator=g, device=DEV, dtype=torch.float32).to(dtype).contiguous()


def _case(B, n_h, n_kv, cap, d, dtype, counts, seed):
    q = _randn((B, n_h, d), seed, dtype)
    kc = _randn((B, n_kv, cap, d), seed + 1, dtype)
    vc = _randn((B, n_kv, cap, d), seed + 2, dtype)
    cnt = torch.tensor(counts, dtype=torch.int32, device=DEV).view(B, n_kv)
    return q, kc, vc, cnt


@pytest.mark.parametrize("first,second", [
    ((4, 32, 8, 2080, 128, torch.bfloat16), (1, 8, 2, 300, 128, torch.bfloat16)),
    ((2, 32, 32, 1056, 128, torch.bfloat16), (3, 4, 2, 97, 64, torch.float32)),
])
def test_noalloc_decode_matches_decode_attn(first, second):
    assert torch.cuda.is_available()
    kvc.lib()
    rng = np.random.default_rng(5)
    for i, (B, n_h, n_kv, cap, d, dtype) in enumerate((first, second)):
        _say("noalloc decode call", i, dict(B=B, n_h=n_h, n_kv=n_kv, cap=cap, d=d, dtype=str(dtype)))
        dims = kvc.make_dims(B, 1, n_h, n_kv, d, kvc.KVC_BF16 if dtype == torch.bfloat16 else kvc.KVC_F32)
        assert kvc.decode_attn_workspace(dims, cap) <= kvc.DECODE_NOALLOC_LIMIT
        counts = rng.integers(0, cap + 1, B * n_kv)
        counts[0] = cap
        counts[-1] = 0
        q, kc, vc, cnt = _case(B, n_h, n_kv, cap, d, dtype, counts.tolist(), 100 + 10 * i)
        ref, ref_lse = kvc.decode_attn(q, kc, vc, cnt)
        out = torch.full_like(ref, 7.0)
        lse = torch.full_like(ref_lse, 7.0)
        kvc.decode_attn_noalloc(q, kc, vc, cnt, out, lse)
        torch.cuda.synchronize()
        assert torch.equal(out, ref)
        assert torch.equal(lse, ref_lse)
        # a second call in a row on the same scratch
        out2 = torch.empty_like(ref)
        kvc.decode_attn_noalloc(q, kc, vc, cnt, out2)
        torch.cuda.synchronize()
        assert torch.equal(out2, ref)


def test_noalloc_decode_rejects_shapes_beyond_its_scratch():
    kvc.lib()
    big = kvc.make_dims(1024, 1, 32, 8, 128, kvc.KVC_BF16)
    assert kvc.decode_attn_workspace(big, 128) > kvc.DECODE_NOALLOC_LIMIT
    BAD = 0x1000
    st = kvc.lib().kvc_decode_attn_noalloc(ctypes.byref(big), BAD, BAD, BAD, BAD, 128, 0.0, BAD, None, None)
    assert st == kvc.KVC_ERR_WORKSPACE
