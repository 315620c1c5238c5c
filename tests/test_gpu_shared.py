"""moe_forward_shared: the layer plus the block's dense GEGLU MLP run as an
always-on shared expert inside the same grouped GEMM launches, against the
fp64 oracle (O10), and against moe_forward when the MLP is zero."""
import numpy as np
import pytest
import torch

import moe_inputs as mi
import oracle
import mixture_experts_router_amd as moe
from mixture_experts_router_amd import device as dev
from gpu_helpers import say, upload, run_forward, run_forward_shared, to64, check_layer

pytestmark = pytest.mark.gpu

# Row-block size from the mean rows per expert (T k / E): 16-row tiles up to
# 16, 64-row tiles up to 40, 256-row tiles above.
SMALL = {
    "tiny+mlp": mi.Shape(T=16, H=256, E=8, k=2, I=128, I_sh=192),             # mean 4: 16-row tiles
    "one-token+mlp": mi.Shape(T=1, H=256, E=8, k=2, I=128, I_sh=128),
    "mid-tiles+mlp": mi.Shape(T=150, H=512, E=16, k=4, I=192, I_sh=256),      # mean 37: 64-row tiles
    "mid-tiles-mxfp4+mlp": mi.Shape(T=150, H=512, E=16, k=4, I=192, I_sh=256, mxfp4=True),
    "ragged+mlp": mi.Shape(T=300, H=512, E=16, k=4, I=192, I_sh=320),         # mean 75: 256-row tiles
    "ragged-mxfp4+mlp": mi.Shape(T=300, H=512, E=16, k=4, I=192, I_sh=256, mxfp4=True),
    "big-tiles+mlp": mi.Shape(T=600, H=512, E=16, k=4, I=128, I_sh=512),      # mean 150: 256-row tiles
    "skew+mlp": mi.Shape(T=200, H=256, E=16, k=4, I=64, I_sh=128, skew=True),  # mean 50: 256-row tiles
}


@pytest.mark.parametrize("name", list(SMALL))
def test_forward_shared_small_full_compare(gpu, name):
    s = SMALL[name]
    say(f"forward_shared {name}: {s}")
    inp = mi.make(s, seed=3)
    out, ids, w = run_forward_shared(inp)
    ref = oracle.forward(inp)
    check_layer(to64(out), ids.cpu().numpy(), w.cpu().numpy(), ref["ids"], ref["w"], ref["out"],
                ref["margin"], name)


@pytest.mark.parametrize("name", ["tiny+mlp", "mid-tiles+mlp", "big-tiles+mlp", "ragged-mxfp4+mlp"])
def test_zero_mlp_is_bitwise_moe_forward(gpu, name):
    """A zero dense MLP adds exact zeros before the routed sum, so the result
    must be moe_forward's, bit for bit."""
    s = SMALL[name]
    inp = mi.make(s, seed=4)
    if s.mxfp4:
        inp.w_sh_gate_up = np.zeros_like(inp.w_sh_gate_up)      # codes 0 -> +0.0
    else:
        inp.w_sh_gate_up = np.zeros_like(inp.w_sh_gate_up)
    d = upload(inp)
    o1, i1, w1 = run_forward_shared(inp, d)
    o2, i2, w2 = run_forward(inp, d)
    assert torch.equal(i1, i2) and torch.equal(w1, w2)
    assert (dev.bf16_bits(o1) == dev.bf16_bits(o2)).all()


def test_forward_shared_full_size_decode(gpu):
    s = mi.CONFIGS["decode_shared"]
    say(f"forward_shared full size: {s}")
    inp = mi.make("decode_shared", seed=0)
    out, ids, w = run_forward_shared(inp)
    ref = oracle.forward_tokens(inp, np.arange(s.T))
    check_layer(to64(out), ids.cpu().numpy(), w.cpu().numpy(), ref["ids"], ref["w"], ref["out"],
                ref["margin"], "decode + dense MLP")


def test_forward_shared_graph_replay(gpu):
    s = SMALL["tiny+mlp"]
    d = upload(mi.make(s, seed=9))
    ref, _, _ = run_forward_shared(mi.make(s, seed=9), d)
    sh = d["shape"]
    out = torch.empty((s.T, s.H), dtype=torch.bfloat16, device="cuda")
    ws = dev.workspace(sh, I_sh=s.I_sh)
    call = lambda: moe.forward_shared(sh, d["x"], d["w_router"], d["bias"], d["w_gu"], d["gu_s"], d["w_d"],
                                      d["d_s"], s.I_sh, d["sh_gu"], d["sh_gu_s"], d["sh_d"], d["sh_d_s"], out,
                                      None, None, ws)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    for rep in range(3):
        out.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert (dev.bf16_bits(out) == dev.bf16_bits(ref)).all(), f"replay {rep}"
        run_forward_shared(mi.make(s, seed=10))                  # eager work between replays
