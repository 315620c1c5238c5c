"""GPU parity of moe_route: the top-k decision bit-exact against the oracle
on the same fp32 logits, weights within fp32 rounding, and the MFMA router
GEMM within its accumulation bound."""
import numpy as np
import pytest
import torch

import moe_inputs as mi
import oracle
import mixture_experts_router_amd as moe
from mixture_experts_router_amd import device as dev
from gpu_helpers import say

pytestmark = pytest.mark.gpu


def _route_logits(gpu, L32, k):
    T, E = L32.shape
    s = moe.shape(T, 64, E, k, 64)
    logits = torch.from_numpy(np.ascontiguousarray(L32)).cuda()
    ids = torch.empty((T, k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, k), dtype=torch.float32, device="cuda")
    gpu.route(s, None, None, None, logits, ids, w)
    torch.cuda.synchronize()
    return ids.cpu().numpy(), w.cpu().numpy()


def _check_topk(gpu, L32, k, label):
    say(f"route (fp32 logits in) {label}: T={L32.shape[0]} E={L32.shape[1]} k={k}")
    ids, w = _route_logits(gpu, L32, k)
    rid, rw = oracle.topk_softmax(L32.astype(np.float64), k)
    assert (ids == rid).all(), f"{label}: ids differ at {np.argwhere(ids != rid)[:5]}"
    err = np.abs(w - rw).max()
    assert err <= 1e-6, f"{label}: weight error {err}"
    assert np.abs(w.sum(axis=1) - 1).max() <= 1e-6


@pytest.mark.parametrize("T,E,k", [(1, 8, 1), (16, 8, 2), (37, 128, 8), (300, 128, 8),
                                   (70, 100, 7), (33, 1024, 32), (20, 32, 32), (9, 5, 5)])
def test_topk_on_oracle_fp32_logits(gpu, T, E, k):
    rng = np.random.default_rng(T * 1000 + E)
    L32 = rng.standard_normal((T, E)).astype(np.float32)
    _check_topk(gpu, L32, k, "gaussian")


def test_topk_ties_lowest_index_wins(gpu):
    rng = np.random.default_rng(7)
    L32 = rng.integers(-2, 3, size=(200, 128)).astype(np.float32)   # massive ties
    _check_topk(gpu, L32, 8, "integer ties")
    L32 = np.full((5, 128), 0.25, dtype=np.float32)
    ids, w = _route_logits(gpu, L32, 8)
    assert (ids == np.arange(8)).all() and (w == np.float32(1 / 8)).all()
    L32 = np.zeros((3, 16), dtype=np.float32)
    L32[:, 3] = -0.0
    _check_topk(gpu, L32, 4, "signed zeros")


def test_topk_extremes(gpu):
    rng = np.random.default_rng(9)
    L32 = (rng.standard_normal((64, 128)) * 40).astype(np.float32)   # weights underflow to 0
    _check_topk(gpu, L32, 8, "wide logits")


def _route_x(gpu, s, x, wr, b):
    T, E, k = s.T, s.E, s.k
    logits = torch.empty((T, E), dtype=torch.float32, device="cuda")
    ids = torch.empty((T, k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, k), dtype=torch.float32, device="cuda")
    nws = moe.route_workspace_bytes(s)
    ws = torch.empty(max(nws, 1), dtype=torch.uint8, device="cuda") if nws else None
    gpu.route(s, x, wr, b, logits, ids, w, ws)
    torch.cuda.synchronize()
    return logits.cpu().numpy(), ids.cpu().numpy(), w.cpu().numpy()


@pytest.mark.parametrize("T,H,E,skew", [(8, 2816, 128, False), (64, 2816, 128, True), (300, 512, 128, False),
                                        (2048, 2816, 128, False), (999, 256, 8, True), (77, 320, 200, False)])
def test_router_gemm_and_routing(gpu, T, H, E, skew):
    say(f"router GEMM T={T} H={H} E={E} skew={skew}")
    inp = mi.make(mi.Shape(T=T, H=H, E=E, k=min(8, E), I=64, skew=skew), seed=1)
    k = inp.shape.k
    x = dev.to_device(inp.x)
    wr = dev.to_device(inp.w_router)
    b = dev.to_device(inp.router_bias) if skew else None
    s = moe.shape(T, H, E, k, 64)
    Lg, ids, w = _route_x(gpu, s, x, wr, b)
    x64 = oracle.bf16_to_f64(inp.x)
    w64 = oracle.bf16_to_f64(inp.w_router)
    L = oracle.router_logits(x64, w64, inp.router_bias)
    # Accumulation bound: fp32 sums of at most 256 exact products, 8 MFMA
    # steps each, added in fp64, one rounding: |err| <= 16 u sum|x w| + u |L|.
    u = 2.0 ** -24
    absdot = np.abs(x64) @ np.abs(w64).T
    bound = 16 * u * absdot + u * np.abs(L)
    err = np.abs(Lg.astype(np.float64) - L)
    say(f"  max |logit err| {err.max():.3e}, max err/bound {(err / bound).max():.3f}")
    assert (err <= bound).all()
    # the decision on the GPU's own fp32 logits is the oracle's decision on them
    rid, rw = oracle.topk_softmax(Lg.astype(np.float64), k)
    assert (ids == rid).all()
    assert np.abs(w - rw).max() <= 1e-6
    # against fp64 routing: differences only at near ties
    fid, _ = oracle.topk_softmax(L, k)
    margin = oracle.routing_margin(L, k)
    diff = np.array([set(a) != set(b) for a, b in zip(ids, fid)])
    say(f"  fp64-routing differences {diff.sum()}, min margin {margin.min():.3e}")
    assert (margin[diff] < 1e-6).all()


@pytest.mark.parametrize("T", [200, 8192])
def test_router_paths_agree_bitwise(gpu, T):
    """Few tokens go through the split-K router, many through the GEMM
    engine (16-token tiles; from 8192 tokens, 32-token tiles of 128
    experts); all follow one definition of the logit, so the logits of the
    same token agree bit for bit."""
    H, E = 2816, 128
    say(f"router paths T={T}")
    inp = mi.make(mi.Shape(T=T, H=H, E=E, k=8, I=64, skew=True), seed=4)
    x = dev.to_device(inp.x)
    wr = dev.to_device(inp.w_router)
    b = dev.to_device(inp.router_bias)
    L_many, _, _ = _route_x(gpu, moe.shape(T, H, E, 8, 64), x, wr, b)
    for t0 in (0, 64, 136, T - 64):
        L_few, _, _ = _route_x(gpu, moe.shape(64, H, E, 8, 64), x[t0:t0 + 64].contiguous(), wr, b)
        assert (L_few.view(np.uint32) == L_many[t0:t0 + 64].view(np.uint32)).all()
