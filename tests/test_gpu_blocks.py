"""GPU parity of landmark-guided block selection (xKV section 2.3, ShadowKV-style):
landmarks and block scores bit-exact against the CPU oracle (exact products added in
the same order in double), the block top-k and its expansion exact, the attention over
the kept blocks within the decode tolerance."""
import sys

import numpy as np
import pytest
import torch

import oracle
from sparse_decode_amd import kvc, synth
from sparse_decode_amd.pipeline import BlockRetrieval
from _parity import assert_decode_close, host

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    kvc.lib()
    oracle.set_threads(0)
    yield


def _say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


@pytest.mark.parametrize("dtype,d,block", [(torch.bfloat16, 128, 16), (torch.float32, 64, 7)])
def test_landmarks_and_block_scores_bitexact(dtype, d, block):
    _say("landmarks/block scores", dtype, d, block)
    g = torch.Generator(device=DEV)
    g.manual_seed(91)
    B, n_h, n_kv, S = 3, 16, 4, 1000
    k = torch.randn((B, n_kv, S, d), generator=g, device=DEV).to(dtype)
    q = torch.randn((B, n_h, d), generator=g, device=DEV).to(dtype)
    sl = np.array([S, 513, 3], np.int32)
    lm = kvc.block_landmarks(k, block, seq_lens=sl)
    sc, cand = kvc.block_scores(q, lm, block, 32, S, seq_lens=sl)
    torch.cuda.synchronize()
    rlm = oracle.block_landmarks(host(k), block, seq_lens=sl)
    assert np.array_equal(host(lm).view(np.int32), rlm.view(np.int32))
    rsc, rcand = oracle.block_scores(host(q), rlm, block, 32, S, seq_lens=sl)
    assert np.array_equal(host(cand), rcand)
    assert np.array_equal(host(sc).view(np.int32), rsc.view(np.int32))


@pytest.mark.parametrize("steps", [2])
def test_block_retrieval_vs_oracle(steps):
    wl = synth.WORKLOADS[4]
    block, k_blocks = 16, wl.k // 16
    _say("block retrieval", wl.name, "block", block, "k_blocks", k_blocks)
    inp = synth.layer_inputs(wl, 0, device=DEV, step=0)
    k, v, sl = inp["k"], inp["v"], inp["seq_lens"]
    sl_dev = torch.from_numpy(sl).to(DEV)
    br = BlockRetrieval(wl, block, k_blocks)
    br.prepare(k, sl_dev)
    k_h, v_h = host(k), host(v)
    for i in range(steps):
        q = synth.step_query(wl, 0, i, device=DEV)
        br.step(q, k, v, sl_dev)
        torch.cuda.synchronize()
        ref = oracle.block_retrieval(host(q), k_h, v_h, k_blocks, block, wl.n_keep, seq_lens=sl)
        assert np.array_equal(host(br.bidx), ref["block_idx"]) and np.array_equal(host(br.bcount), ref["block_count"])
        assert np.array_equal(host(br.idx), ref["idx"][:, :, :br.cap]) and np.array_equal(host(br.count), ref["count"])
        want_k, _ = oracle.gather(k.view(torch.int16).cpu().numpy(), host(br.idx), host(br.count),
                                  dst=br.kc.view(torch.int16).cpu().numpy())
        assert np.array_equal(br.kc.view(torch.int16).cpu().numpy(), want_k)
        out_ref, _ = oracle.decode(host(q), host(br.kc), host(br.vc), host(br.count))
        assert_decode_close(br.out, out_ref, True, "block decode step %d" % i)
