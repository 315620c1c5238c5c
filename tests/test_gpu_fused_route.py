"""The routing inside moe_forward -- up to 16 tokens the single-launch
routing (router chunk sums, then, in the last block to finish, top-k and
permutation), above that the staged launches -- against the stage-by-stage C
ABI path (moe_route, moe_permute, the two grouped GEMMs, moe_combine) on the
same inputs: routing, weights, the permutation tables and the output must
agree bitwise, and the completion counter must be back to zero after every
call."""
import numpy as np
import pytest
import torch

import moe_inputs as mi
import mixture_experts_router_amd as moe
from mixture_experts_router_amd import device as dev
from gpu_helpers import say, upload, run_forward

pytestmark = pytest.mark.gpu

WS_ZERO_BYTES = 256   # MOE_WS_ZERO_BYTES in include/moe.h

SHAPES = {
    "decode-like": mi.Shape(T=8, H=512, E=128, k=8, I=128),          # 64 assignments: one-wave permutation
    "one-token": mi.Shape(T=1, H=256, E=8, k=1, I=64),
    "64-tokens": mi.Shape(T=64, H=512, E=64, k=8, I=128),            # above 16 tokens: the staged routing
    "wide-experts": mi.Shape(T=2, H=256, E=1024, k=32, I=64),        # 16 logits per lane
    "odd-experts": mi.Shape(T=40, H=768, E=300, k=6, I=64),          # staged: 3 chunks of 256, partial expert block
    "odd-experts-one-launch": mi.Shape(T=12, H=768, E=300, k=6, I=64),  # A = 72: block permutation, 3 chunks
    "skew-bias": mi.Shape(T=16, H=512, E=128, k=8, I=64, skew=True),
    # one-wave permutation (A <= 64) at other expert counts
    "one-wave-odd-experts": mi.Shape(T=9, H=256, E=300, k=7, I=64),   # A = 63, five experts per lane
    "single-expert": mi.Shape(T=5, H=256, E=1, k=1, I=64),             # no id bits at all
    "one-wave-hot": mi.Shape(T=8, H=256, E=16, k=8, I=64, skew=True),  # half the experts per token, skewed
}


def _staged(d, s):
    sh = d["shape"]
    A = s.T * s.k
    i32 = dict(dtype=torch.int32, device="cuda")
    logits = torch.empty((s.T, s.E), dtype=torch.float32, device="cuda")
    ids = torch.empty((s.T, s.k), **i32)
    w = torch.empty((s.T, s.k), dtype=torch.float32, device="cuda")
    counts, offsets = torch.empty(s.E, **i32), torch.empty(s.E + 1, **i32)
    sorted_ids, inv = torch.empty(A, **i32), torch.empty(A, **i32)
    x_perm = torch.empty((A, s.H), dtype=torch.bfloat16, device="cuda")
    h = torch.empty((A, s.I), dtype=torch.bfloat16, device="cuda")
    y = torch.empty((A, s.H), dtype=torch.bfloat16, device="cuda")
    out = torch.empty((s.T, s.H), dtype=torch.bfloat16, device="cuda")
    rws = torch.empty(max(1, moe.route_workspace_bytes(sh)), dtype=torch.uint8, device="cuda")
    pws = torch.empty(max(1, moe.permute_workspace_bytes(sh)), dtype=torch.uint8, device="cuda")
    moe.route(sh, d["x"], d["w_router"], d["bias"], logits, ids, w, ws=rws)
    moe.permute(sh, ids, d["x"], counts, offsets, sorted_ids, inv, x_perm, pws)
    moe.gemm_gateup(sh, d["x"], sorted_ids, offsets, d["w_gu"], d["gu_s"], h)
    moe.gemm_down(sh, h, offsets, d["w_d"], d["d_s"], y)
    moe.combine(sh, y, inv, w, out)
    torch.cuda.synchronize()
    return out, ids, w, (counts, offsets, sorted_ids, inv)


def _ws_tables(ws, sh, s):
    """The fused kernel's counts, offsets, sorted_ids and inv inside the
    moe_forward workspace.  White-box: the offsets follow the workspace carve
    of csrc/api.hip (256-byte aligned pieces: completion counter, router
    partials, logits, ids, weights, counts, offsets, block histograms,
    sorted_ids, inv, ...)."""
    up = lambda n: (n + 255) // 256 * 256
    A = s.T * s.k
    off = WS_ZERO_BYTES + moe.route_workspace_bytes(sh)
    off += up(s.T * s.E * 4) + up(A * 4) + up(A * 4)          # logits, ids, weights
    views = []
    for n, skip in ((s.E, 0), (s.E + 1, 0), (A, moe.permute_workspace_bytes(sh)), (A, 0)):
        off += skip
        views.append(ws[off:off + 4 * n].view(torch.int32))
        off += up(4 * n)
    return views


@pytest.mark.parametrize("name", list(SHAPES))
def test_fused_routing_matches_staged_path(gpu, name):
    s = SHAPES[name]
    say(f"fused routing {name}: {s}")
    inp = mi.make(s, seed=11)
    d = upload(inp)
    ws = dev.workspace(d["shape"])
    for call in range(3):      # the counter must reset itself between calls
        out, ids, w = run_forward(inp, d, ws)
        assert int(ws[:WS_ZERO_BYTES].count_nonzero()) == 0, f"counter not reset after call {call}"
    o2, i2, w2, tables = _staged(d, s)
    # the whole permutation of the fused kernel, bitwise (moe_forward itself
    # reads only offsets and sorted_ids)
    for got, want, what in zip(_ws_tables(ws, d["shape"], s), tables, ("counts", "offsets", "sorted_ids", "inv")):
        assert torch.equal(got, want), what
    assert torch.equal(ids, i2)
    assert torch.equal(w.view(torch.int32), w2.view(torch.int32))
    assert (dev.bf16_bits(out) == dev.bf16_bits(o2)).all()
