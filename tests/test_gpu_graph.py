"""moe_forward captured as a HIP graph: every replay -- with other eager
work and synchronisations between replays -- must reproduce the eager result
bitwise (the launches depend only on the shape, and the workspace's completion
counters return to zero after each call)."""
import pytest
import torch

import moe_inputs as mi
import mixture_experts_router_amd as moe
from mixture_experts_router_amd import device as dev
from gpu_helpers import say, upload

pytestmark = pytest.mark.gpu

SHAPES = {
    "few-tokens": mi.Shape(T=8, H=512, E=128, k=8, I=128),        # single-launch routing
    "many-tokens": mi.Shape(T=600, H=512, E=16, k=4, I=192),      # dense router, multi-block permutation
    "mxfp4": mi.Shape(T=40, H=512, E=16, k=4, I=128, mxfp4=True),
}


def _call(d, sh, out, ids, w, ws):
    moe.forward(sh, d["x"], d["w_router"], d["bias"], d["w_gu"], d["gu_s"], d["w_d"], d["d_s"], out, ids, w, ws)


@pytest.mark.parametrize("name", list(SHAPES))
def test_graph_replays_match_eager(gpu, name):
    s = SHAPES[name]
    say(f"graph {name}: {s}")
    d = upload(mi.make(s, seed=21))
    other = upload(mi.make(s, seed=22))
    sh = d["shape"]
    mk = lambda: (torch.empty((s.T, s.H), dtype=torch.bfloat16, device="cuda"),
                  torch.empty((s.T, s.k), dtype=torch.int32, device="cuda"),
                  torch.empty((s.T, s.k), dtype=torch.float32, device="cuda"))
    ref_out, ref_ids, ref_w = mk()
    ws_eager = dev.workspace(sh)
    _call(d, sh, ref_out, ref_ids, ref_w, ws_eager)
    torch.cuda.synchronize()

    out, ids, w = mk()
    ws = dev.workspace(sh)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        _call(d, sh, out, ids, w, ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        _call(d, sh, out, ids, w, ws)
    o2, i2, w2 = mk()
    for rep in range(4):
        out.zero_(); ids.zero_(); w.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(ids, ref_ids), f"replay {rep}: ids"
        assert torch.equal(w.view(torch.int32), ref_w.view(torch.int32)), f"replay {rep}: weights"
        assert (dev.bf16_bits(out) == dev.bf16_bits(ref_out)).all(), f"replay {rep}: out"
        _call(other, sh, o2, i2, w2, ws_eager)          # eager work between replays
        torch.cuda.synchronize()
