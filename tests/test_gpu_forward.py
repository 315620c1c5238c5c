"""End-to-end parity of moe_forward against the fp64 oracle.

Every problem is compared in full, token by token: small ragged shapes, and
the four Gemma-4-26B-A4B workloads (decode T=8, prefill T=2048, Zipf-skewed
T=8192, MXFP4 experts T=2048) plus a Zipf-skewed batch of 32 768 tokens, run
in the launch configuration the benchmark times."""
import numpy as np
import pytest
import torch

import moe_inputs as mi
import oracle
import mixture_experts_router_amd as moe
from mixture_experts_router_amd import device as dev
from gpu_helpers import say, upload, run_forward, to64, check_layer

pytestmark = pytest.mark.gpu


SMALL = {
    "tiny": mi.CONFIGS["tiny"],
    "ragged": mi.Shape(T=300, H=512, E=16, k=4, I=192),
    "ragged-skew": mi.Shape(T=300, H=512, E=16, k=4, I=192, skew=True),
    "ragged-mxfp4": mi.Shape(T=300, H=512, E=16, k=4, I=192, mxfp4=True),
    # 16-row tiles: 4-bit gate/up in 256-wide K steps, down (K = 704) in 64-wide ones
    "decode-like-mxfp4": mi.Shape(T=8, H=768, E=64, k=8, I=704, mxfp4=True),
    # 16-row tiles with H % 256 != 0: 64-wide steps for both GEMMs
    "k576-mxfp4": mi.Shape(T=12, H=576, E=16, k=4, I=128, mxfp4=True),
    # 16-row gate/up tiles with 256-wide steps and a partial last step
    # (1152 = 4 x 256 + 128; E8M0 scale rows of 36 bytes)
    "k1152-mxfp4": mi.Shape(T=12, H=1152, E=16, k=4, I=128, mxfp4=True),
    "one-token": mi.Shape(T=1, H=256, E=8, k=2, I=128),
    "k-equals-E": mi.Shape(T=40, H=256, E=8, k=8, I=128),
    "many-experts": mi.Shape(T=130, H=256, E=300, k=6, I=64),
    # the supported maximum of experts and of experts per token together
    "max-E-and-k": mi.Shape(T=64, H=256, E=1024, k=32, I=64),
    # one expert, top-1: the layer degenerates to a dense GEGLU FFN
    "single-expert": mi.Shape(T=50, H=256, E=1, k=1, I=128),
    # one token of the Gemma-4 layer (a single decode step)
    "one-token-model": mi.Shape(T=1, H=2816, E=128, k=8, I=704),
}


@pytest.mark.parametrize("name", list(SMALL))
def test_forward_small_full_compare(gpu, name):
    s = SMALL[name]
    say(f"forward {name}: {s}")
    inp = mi.make(s, seed=2)
    out, ids, w = run_forward(inp)
    ref = oracle.forward(inp)
    check_layer(to64(out), ids.cpu().numpy(), w.cpu().numpy(), ref["ids"], ref["w"], ref["out"],
                ref["margin"], name)


def test_forward_zero_input_is_zero(gpu):
    inp = mi.make(mi.Shape(T=50, H=256, E=8, k=2, I=128), seed=3)
    inp.x[:] = 0
    out, ids, w = run_forward(inp)
    assert (out.float() == 0).all()
    assert (ids.cpu().numpy() == np.arange(2)).all()      # all logits 0: lowest indices
    assert (w.cpu().numpy() == 0.5).all()


def test_forward_single_hot_expert(gpu):
    """A bias that sends every token to the same experts: two experts own all
    rows, the rest are empty."""
    s = mi.Shape(T=700, H=256, E=16, k=2, I=128)
    inp = mi.make(s, seed=4)
    inp.router_bias = np.full(16, -100.0, dtype=np.float32)
    inp.router_bias[[3, 11]] = 100.0
    out, ids, w = run_forward(inp)
    ref = oracle.forward(inp)
    assert set(np.unique(ids.cpu().numpy())) == {3, 11}
    check_layer(to64(out), ids.cpu().numpy(), w.cpu().numpy(), ref["ids"], ref["w"], ref["out"],
                ref["margin"], "single hot expert")


def test_forward_is_deterministic_and_reusable(gpu):
    big = mi.make(mi.Shape(T=700, H=512, E=16, k=4, I=192), seed=6)
    small = mi.make(mi.Shape(T=9, H=512, E=16, k=4, I=192), seed=6)
    db, ds = upload(big), upload(small)
    ws = dev.workspace(db["shape"])
    o1, _, _ = run_forward(big, db, ws)
    o2, _, _ = run_forward(small, ds, ws)       # same workspace, smaller T
    o3, _, _ = run_forward(big, db, ws)
    o4, _, _ = run_forward(small, ds)
    assert (dev.bf16_bits(o1) == dev.bf16_bits(o3)).all()
    assert (dev.bf16_bits(o2) == dev.bf16_bits(o4)).all()


# ---------------------------------------------------------------- full sizes
@pytest.mark.parametrize("name", ["decode", "prefill", "skew", "mxfp4"])
def test_forward_full_size(gpu, name):
    s = mi.CONFIGS[name]
    say(f"forward full size {name}: {s}")
    full_size_check(mi.make(name, seed=0), name)


def test_forward_32k_tokens(gpu):
    """The model's layer on 32 768 tokens with the skewed router bias:
    262 144 assignments (16 permutation blocks of 1024 at the hot expert
    alone), hot experts spanning dozens of 256-row tiles, and a down GEMM
    output (1.5 GB) far above the last-level cache, so its row-tile groups
    run last to first."""
    s = mi.Shape(T=32768, H=2816, E=128, k=8, I=704, skew=True)
    say(f"forward 32k tokens: {s}")
    full_size_check(mi.make(s, seed=3), "32k-skew")


def full_size_check(inp, name):
    """The whole output against the oracle's whole fp64 forward, plus the
    routing-table invariants."""
    s = inp.shape
    out, ids, w = run_forward(inp)
    ids_np, w_np = ids.cpu().numpy(), w.cpu().numpy()
    got = to64(out)
    del out
    counts = np.bincount(ids_np.reshape(-1), minlength=s.E)
    say(f"  counts min {counts.min()} max {counts.max()} empty {int((counts == 0).sum())}")
    assert counts.sum() == s.T * s.k
    assert all(len(set(r)) == s.k for r in ids_np)
    ref = oracle.forward(inp)
    check_layer(got, ids_np, w_np, ref["ids"], ref["w"], ref["out"], ref["margin"],
                f"{name} (all {s.T} tokens)")
