"""W4A4 (MOE_W_MXFP4_A4): the MXFP4 activation quantiser bit for bit against
the oracle's (O11), and moe_forward with MXFP4 weights and activations on
the gfx950 block-scaled FP4 matrix instructions against the fp64 oracle."""
import numpy as np
import pytest
import torch

import moe_inputs as mi
import oracle
import mixture_experts_router_amd as moe
from mixture_experts_router_amd import device as dev
from gpu_helpers import say, run_forward, to64, check_layer

pytestmark = pytest.mark.gpu


def _quantize_gpu(bits):
    src = dev.to_device(bits)
    rows, K = bits.shape
    codes = torch.empty((rows, K // 2), dtype=torch.uint8, device="cuda")
    scales = torch.empty((rows, K // 32), dtype=torch.uint8, device="cuda")
    moe.quantize_mx(src, codes, scales)
    torch.cuda.synchronize()
    return codes.cpu().numpy(), scales.cpu().numpy()


def _oracle_packed(bits):
    c, s = oracle.mx_quantize(oracle.bf16_to_f64(bits))
    return (c[:, 0::2] | (c[:, 1::2] << 4)).astype(np.uint8), s


@pytest.mark.parametrize("rows,K,seed", [(1, 32, 0), (7, 96, 1), (300, 2816, 2), (64, 704, 3)])
def test_quantizer_matches_oracle_bitwise(gpu, rows, K, seed):
    rng = np.random.default_rng(seed)
    v = rng.standard_normal((rows, K)) * np.exp(rng.uniform(-8, 8, (rows, 1)))
    bits = mi.f32_to_bf16_bits(v.astype(np.float32))
    codes, scales = _quantize_gpu(bits)
    rc, rs = _oracle_packed(bits)
    assert (scales == rs).all()
    assert (codes == rc).all()


def test_quantizer_special_values(gpu):
    """Zeros, negative zeros, bf16 subnormals, every E2M1 midpoint (ties to
    even) and saturation, huge and tiny blocks."""
    rows = []
    z = np.zeros(32, dtype=np.float32)
    rows.append(z)
    nz = z.copy(); nz[::2] = -0.0; nz[5] = 1e-40; rows.append(nz)            # -0 and a subnormal
    sub = np.full(32, 2.0 ** -130, dtype=np.float32); sub[3] = -2.0 ** -128; rows.append(sub)
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 7.9, 4.0, 6.0, 5.9, 0.0] * 3, dtype=np.float32)[:32]
    rows.append(mids); rows.append(-mids); rows.append(mids * 2.0 ** 20); rows.append(mids * 2.0 ** -30)
    huge = np.full(32, 3.0e38, dtype=np.float32); huge[0] = -3.3e38; rows.append(huge)
    bits = mi.f32_to_bf16_bits(np.stack(rows))
    codes, scales = _quantize_gpu(bits)
    rc, rs = _oracle_packed(bits)
    assert (scales == rs).all()
    assert (codes == rc).all()


A4 = {
    "tiny-a4": mi.Shape(T=16, H=256, E=8, k=2, I=128, mxfp4=True, a4=True),          # down K: half a step
    "mid-tiles-a4": mi.Shape(T=120, H=512, E=16, k=4, I=192, mxfp4=True, a4=True),    # mean 30: 64-row tiles
    "ragged-a4": mi.Shape(T=300, H=512, E=16, k=4, I=192, mxfp4=True, a4=True),      # mean 75: 256-row tiles
    "big-tiles-a4": mi.Shape(T=600, H=512, E=16, k=4, I=320, mxfp4=True, a4=True),   # 256-row tiles
    # 256-row tiles with half a 256-wide K step in all (K = 128) and a gate/up
    # that ends in a half step (H = 576)
    "short-k-a4": mi.Shape(T=400, H=128, E=8, k=2, I=64, mxfp4=True, a4=True),       # mean 100
    "odd-k-a4": mi.Shape(T=600, H=576, E=16, k=4, I=320, mxfp4=True, a4=True),
    "decode-like-a4": mi.Shape(T=8, H=768, E=64, k=8, I=704, mxfp4=True, a4=True),   # the model's I
    # the Gemma-4 layer at 300 tokens (mean 19): 64-row tiles with the model's
    # K (gate/up 2816 = 11 steps of 256, down 704 = 2.75 steps)
    "model-mid-tiles-a4": mi.Shape(T=300, H=2816, E=128, k=8, I=704, mxfp4=True, a4=True),
    "skew-a4": mi.Shape(T=200, H=256, E=16, k=4, I=64, mxfp4=True, a4=True, skew=True),
}


@pytest.mark.parametrize("name", list(A4))
def test_forward_w4a4_small_full_compare(gpu, name):
    s = A4[name]
    say(f"forward w4a4 {name}: {s}")
    inp = mi.make(s, seed=5)
    out, ids, w = run_forward(inp)
    ref = oracle.forward(inp)
    check_layer(to64(out), ids.cpu().numpy(), w.cpu().numpy(), ref["ids"], ref["w"], ref["out"],
                ref["margin"], name)


def test_forward_w4a4_differs_from_w4a16(gpu):
    """The activations really are quantised: W4A4 and W4A16 outputs differ by
    about the activation quantisation error, and W4A4 matches its oracle."""
    s = A4["ragged-a4"]
    inp = mi.make(s, seed=6)
    o4, _, _ = run_forward(inp)
    import dataclasses
    inp16 = dataclasses.replace(inp, shape=dataclasses.replace(s, a4=False))
    o16, _, _ = run_forward(inp16)
    d = to64(o4) - to64(o16)
    rel = np.linalg.norm(d) / np.linalg.norm(to64(o16))
    say(f"w4a4 vs w4a16 rel difference {rel:.3e}")
    assert 1e-2 < rel < 0.5


def test_forward_w4a4_full_size(gpu):
    """The W4A4 prefill workload (2048 tokens), every token against the
    oracle's whole forward."""
    s = mi.CONFIGS["w4a4"]
    say(f"forward w4a4 full size: {s}")
    inp = mi.make("w4a4", seed=0)
    out, ids, w = run_forward(inp)
    ref = oracle.forward(inp)
    check_layer(to64(out), ids.cpu().numpy(), w.cpu().numpy(), ref["ids"], ref["w"], ref["out"],
                ref["margin"], f"w4a4 (all {s.T} tokens)")
