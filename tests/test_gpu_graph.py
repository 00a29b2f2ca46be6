"""The four calls captured in a HIP graph: several replays, with eager work and
synchronisations in between, each bit-identical to the eager result."""
import dataclasses

import pytest
import torch

from sparse_decode_amd import kvc, synth
from sparse_decode_amd.pipeline import LayerPath

pytestmark = pytest.mark.gpu


def _outputs(path):
    return [t.clone() for t in (path.raw, path.pooled, path.idx, path.count, path.kc, path.vc, path.pos,
                                path.out, path.lse)]


@pytest.mark.parametrize("cfg", [2, 4])
def test_graph_replays_match_eager(cfg):
    assert torch.cuda.is_available()
    kvc.lib()
    wl = synth.WORKLOADS[cfg]
    if cfg == 2:
        wl = dataclasses.replace(wl, k=512)
        s_max = 8192
    else:
        s_max = None
    print("[case] graph", wl.name, flush=True)
    layers = [synth.layer_inputs(wl, l, device="cuda", s_max=s_max) for l in range(2)]
    for inp in layers:
        inp["sl"] = torch.from_numpy(inp["seq_lens"]).cuda()
    path = LayerPath(wl, s_max=s_max)

    def step(inp):
        path.run(inp["q_win"], inp["k"], inp["v"], inp["q_dec"], inp["sl"])

    step(layers[0])
    torch.cuda.synchronize()
    eager = _outputs(path)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step(layers[0])
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(layers[0])
    for rep in range(3):
        step(layers[1])                      # eager work on other data between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = _outputs(path)
        for a, b in zip(got, eager):
            assert torch.equal(a, b), rep
