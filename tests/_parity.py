"""Helpers shared by the GPU parity tests: host copies, tolerances and the selection
acceptance rule.  Tolerances:

* window scores (fp32): |gpu - ref| <= 1e-5 |ref| (+1e-35 absolute, which only
  matters for probabilities the GPU flushes below the fp32 normal range);
* selections and gathers: bit-exact on identical inputs; on independently computed
  scores a different selection is accepted iff every selected candidate's oracle
  score is >= every unselected candidate's oracle score times (1 - 1e-5);
* decode outputs: |gpu - ref| <= 2e-2 + 1e-2 |ref| for bf16 outputs against the
  double-precision oracle (1e-5 + 1e-5 |ref| for fp32 outputs), computed on the
  GPU's own compacted cache so that a legitimate near-tie cannot cascade.
"""
import numpy as np
import torch

SCORE_RTOL = 1e-5
SCORE_ATOL = 1e-35
SEL_RTOL = 1e-5


def host(t):
    if isinstance(t, np.ndarray):
        return t
    if t.dtype in (torch.bfloat16, torch.float16):
        t = t.float()
    return t.detach().cpu().contiguous().numpy()


def assert_scores_close(gpu, ref, what="scores"):
    gpu = host(gpu).astype(np.float64)
    ref = np.asarray(ref, np.float64)
    err = np.abs(gpu - ref)
    bound = SCORE_RTOL * np.abs(ref) + SCORE_ATOL
    bad = err > bound
    if bad.any():
        i = np.unravel_index(np.argmax(err - bound), err.shape)
        raise AssertionError("%s: %d mismatches; worst at %s gpu=%r ref=%r rel=%.3g" % (
            what, int(bad.sum()), i, gpu[i], ref[i], err[i] / max(abs(ref[i]), 1e-300)))


def decode_tol(bf16):
    return (2e-2, 1e-2) if bf16 else (1e-5, 1e-5)


def assert_decode_close(gpu, ref, bf16, what="decode"):
    atol, rtol = decode_tol(bf16)
    gpu = host(gpu).astype(np.float64)
    err = np.abs(gpu - ref)
    bad = err > atol + rtol * np.abs(ref)
    if bad.any():
        i = np.unravel_index(np.argmax(err), err.shape)
        raise AssertionError("%s: %d mismatches; worst at %s gpu=%r ref=%r" % (what, int(bad.sum()), i, gpu[i], ref[i]))


def check_selection(gpu_idx, gpu_count, ref_idx, ref_count, ref_scores, seq_lens, k, n_keep, shared=False):
    """Exact match, or the acceptance rule for near-ties.  Returns #units that differed."""
    gi, gc = host(gpu_idx), host(gpu_count)
    ri, rc = np.asarray(ref_idx), np.asarray(ref_count)
    sc = np.asarray(ref_scores)
    assert gi.shape == ri.shape and gc.shape == rc.shape
    assert np.array_equal(gc, rc), "counts differ"
    differ = 0
    B, H, cap = gi.shape
    for b in range(B):
        S = int(seq_lens[b])
        C = max(0, S - n_keep)
        k_eff = min(k, C)
        for h in range(H):
            n = int(gc[b, h])
            if np.array_equal(gi[b, h], ri[b, h]):
                continue
            differ += 1
            sel = gi[b, h, :n]
            assert np.all(np.diff(sel) > 0), "indices not strictly ascending"
            assert np.all(gi[b, h, n:] == -1)
            assert np.array_equal(sel[k_eff:], np.arange(C, S)), "window differs"
            chosen = sel[:k_eff]
            assert chosen.size == 0 or (chosen.min() >= 0 and chosen.max() < C)
            if shared:
                s = sc[b].astype(np.float64).sum(axis=0)      # the oracle's exact head sum
            else:
                s = sc[b, h]
            mask = np.zeros(C, bool)
            mask[chosen] = True
            lo = s[:C][mask].min() if mask.any() else np.inf
            hi = s[:C][~mask].max() if (~mask).any() else -np.inf
            assert lo >= hi * (1 - SEL_RTOL), "selection outside the near-tie rule (b=%d h=%d: %r < %r)" % (b, h, lo, hi)
    return differ
