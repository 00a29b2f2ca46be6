"""The seeded input generators (host logic, no GPU): lengths and planted positions stay
inside the cache whatever the token capacity asked for."""
import numpy as np
import pytest

from sparse_decode_amd import synth


@pytest.mark.parametrize("wl", list(synth.WORKLOADS.values()), ids=lambda w: w.name)
@pytest.mark.parametrize("s_max", [None, 4096, 700, 1])
def test_lengths_and_planted_positions_inside_the_cache(wl, s_max):
    S = wl.s_max if s_max is None else s_max
    sl = synth.seq_lens(wl, S)
    assert sl.dtype == np.int32 and sl.shape == (wl.batch,)
    assert (sl >= 0).all() and (sl <= S).all()
    for b, s_b in enumerate(sl):
        pos = synth.planted_positions(wl, b, int(s_b))
        assert pos.size == 0 or (0 <= pos.min() and pos.max() < max(0, int(s_b) - wl.n_keep))


def test_ragged_lengths_unchanged_at_their_own_capacity():
    # the ragged workload's lengths are its seeded draws in [4096, 16384]; a smaller
    # capacity cuts only the longer ones
    wl = synth.by_name("ragged_b16")
    full = synth.seq_lens(wl)
    assert full.min() >= wl.ragged[0] and full.max() <= wl.ragged[1] == wl.s_max
    cut = synth.seq_lens(wl, 8192)
    assert np.array_equal(cut, np.minimum(full, 8192))


def test_layer_inputs_plant_inside_a_smaller_cache():
    wl = synth.by_name("ragged_b16")
    x = synth.layer_inputs(wl, 0, device="cpu", s_max=512, batch=2)
    assert x["k"].shape[2] == 512 and (x["seq_lens"] <= 512).all()
    for pos in x["planted"]:
        assert pos.size == 0 or pos.max() < 512
