"""moe_forward_noalloc (the layer on the library's own per-GPU scratch, for
callers that cannot allocate) against moe_forward on a caller workspace:
the same kernels, so outputs, expert ids and weights must be bitwise equal.
Two calls in a row on the shared scratch, the second with fewer tokens."""
import numpy as np
import pytest
import torch

import moe_inputs as mi
import mixture_experts_router_amd as moe
from mixture_experts_router_amd import device as dev
from gpu_helpers import say, upload, run_forward

pytestmark = pytest.mark.gpu


def _noalloc(d, s):
    out = torch.empty((s.T, s.H), dtype=torch.bfloat16, device="cuda")
    ids = torch.empty((s.T, s.k), dtype=torch.int32, device="cuda")
    w = torch.empty((s.T, s.k), dtype=torch.float32, device="cuda")
    moe.forward_noalloc(d["shape"], d["x"], d["w_router"], d["bias"], d["w_gu"], d["gu_s"], d["w_d"], d["d_s"],
                        out, ids, w)
    return out, ids, w


@pytest.mark.parametrize("shapes", [
    # 600 tokens of the Gemma-4 layer (64-row tiles, the staged routing),
    # then 8 (single-launch routing with its completion counter)
    (mi.Shape(T=600, H=2816, E=128, k=8, I=704), mi.Shape(T=8, H=2816, E=128, k=8, I=704)),
    # MXFP4 experts, skewed router: 1000 tokens (256-row tiles) then 40
    (mi.Shape(T=1000, H=2816, E=128, k=8, I=704, mxfp4=True, skew=True),
     mi.Shape(T=40, H=2816, E=128, k=8, I=704, mxfp4=True, skew=True)),
], ids=["bf16", "mxfp4-skew"])
def test_noalloc_matches_forward(gpu, shapes):
    big, small = (mi.make(s, seed=21) for s in shapes)
    db, dsm = upload(big), upload(small)
    assert moe.workspace_bytes(db["shape"]) <= moe.NOALLOC_SCRATCH_BYTES
    say(f"noalloc: {big.shape.T} then {small.shape.T} tokens, mxfp4={big.shape.mxfp4}")
    # two calls in a row on the one scratch buffer, the second smaller
    o1, i1, w1 = _noalloc(db, big.shape)
    o2, i2, w2 = _noalloc(dsm, small.shape)
    torch.cuda.synchronize()
    r1, ri1, rw1 = run_forward(big, db)
    r2, ri2, rw2 = run_forward(small, dsm)
    for got, ref in ((o1, r1), (o2, r2)):
        assert (dev.bf16_bits(got) == dev.bf16_bits(ref)).all()
    assert torch.equal(i1, ri1) and torch.equal(i2, ri2)
    assert torch.equal(w1, rw1) and torch.equal(w2, rw2)
    # and again after the caller-workspace calls (the scratch keeps the last
    # call's contents; the completion counters must be back at zero)
    o3, i3, _ = _noalloc(dsm, small.shape)
    torch.cuda.synchronize()
    assert (dev.bf16_bits(o3) == dev.bf16_bits(r2)).all() and torch.equal(i3, ri2)


def test_noalloc_rejects_oversized_shape(gpu):
    s = moe.shape(2048, 2816, 128, 8, 704)
    assert moe.workspace_bytes(s) > moe.NOALLOC_SCRATCH_BYTES
    t = torch.empty(16, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(moe.MoeError) as e:
        moe.forward_noalloc(s, t, t, None, t, None, t, None, t)
    assert e.value.status == -5
