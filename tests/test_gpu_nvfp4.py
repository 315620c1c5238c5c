"""NVFP4 expert weights (MOE_W_NVFP4: E2M1 codes, an E4M3 scale per 16 K
values, an fp32 scale per expert matrix; bf16 activations) through
moe_forward and the per-step grouped GEMMs, against the fp64 oracle (O12)."""
import numpy as np
import pytest
import torch

import moe_inputs as mi
import oracle
import mixture_experts_router_amd as moe
from mixture_experts_router_amd import device as dev
from gpu_helpers import say, run_forward, upload, to64, check_layer

pytestmark = pytest.mark.gpu

NV = {
    "tiny-nv": mi.Shape(T=16, H=256, E=8, k=2, I=128, nvfp4=True),
    "mid-tiles-nv": mi.Shape(T=150, H=512, E=16, k=4, I=192, nvfp4=True),     # mean 37: 64-row tiles
    "ragged-nv": mi.Shape(T=300, H=512, E=16, k=4, I=192, nvfp4=True),        # mean 75: 256-row tiles, ragged tails
    "big-tiles-nv": mi.Shape(T=600, H=512, E=16, k=4, I=320, nvfp4=True),     # 256-row tiles
    "decode-like-nv": mi.Shape(T=8, H=768, E=64, k=8, I=704, nvfp4=True),     # 16-row tiles, the model's I
    "skew-nv": mi.Shape(T=200, H=256, E=16, k=4, I=64, nvfp4=True, skew=True),
    "k576-nv": mi.Shape(T=12, H=576, E=16, k=4, I=128, nvfp4=True),            # H % 256 != 0
    # 16-row gate/up tiles with 256-wide steps straight to LDS and a partial
    # last step (1088 = 4 x 256 + 64)
    "k1088-nv": mi.Shape(T=12, H=1088, E=16, k=4, I=128, nvfp4=True),
}


@pytest.mark.parametrize("name", list(NV))
def test_forward_nvfp4_small_full_compare(gpu, name):
    s = NV[name]
    say(f"forward nvfp4 {name}: {s}")
    inp = mi.make(s, seed=7)
    out, ids, w = run_forward(inp)
    ref = oracle.forward(inp)
    check_layer(to64(out), ids.cpu().numpy(), w.cpu().numpy(), ref["ids"], ref["w"], ref["out"],
                ref["margin"], name)


def test_forward_nvfp4_decode_full_size(gpu):
    s = mi.CONFIGS["nvfp4_decode"]
    say(f"forward nvfp4 decode full size: {s}")
    inp = mi.make("nvfp4_decode", seed=0)
    out, ids, w = run_forward(inp)
    ref = oracle.forward(inp)
    check_layer(to64(out), ids.cpu().numpy(), w.cpu().numpy(), ref["ids"], ref["w"], ref["out"],
                ref["margin"], "nvfp4 decode")


@pytest.mark.parametrize("rows_per_expert", [3, 40, 300])
def test_nvfp4_grouped_gemms_step_by_step(gpu, rows_per_expert):
    """moe_grouped_gemm_gateup / _down with NVFP4 weights on pre-grouped
    rows, each tile size, against the oracle's GEGLU and down projection on
    the decoded weights (h compared after the kernel's own bf16 rounding)."""
    E, H, I = 6, 512, 192
    s = mi.Shape(T=rows_per_expert * E, H=H, E=E, k=1, I=I, nvfp4=True)
    inp = mi.make(s, seed=11)
    d = upload(inp)
    A = s.T
    x = d["x"]
    offsets = torch.arange(E + 1, dtype=torch.int32, device="cuda") * rows_per_expert
    h = torch.empty((A, I), dtype=torch.bfloat16, device="cuda")
    y = torch.empty((A, H), dtype=torch.bfloat16, device="cuda")
    moe.gemm_gateup(d["shape"], x, None, offsets, d["w_gu"], d["gu_s"], h)
    moe.gemm_down(d["shape"], h, offsets, d["w_d"], d["d_s"], y)
    torch.cuda.synchronize()
    x64 = oracle.bf16_to_f64(inp.x)
    h_got, y_got = to64(h), to64(y)
    for e in range(E):
        r = slice(e * rows_per_expert, (e + 1) * rows_per_expert)
        wgu, wd = oracle.expert_weights(inp, e)
        h_ref = oracle.gateup_geglu(x64[r], wgu)
        y_ref = oracle.down_proj(h_got[r], wd)        # down on the kernel's own bf16 h
        rel_h = np.linalg.norm(h_got[r] - h_ref) / np.linalg.norm(h_ref)
        rel_y = np.linalg.norm(y_got[r] - y_ref) / np.linalg.norm(y_ref)
        assert rel_h < 1e-2 and rel_y < 1e-2, (e, rel_h, rel_y)
    say(f"nvfp4 gemms, {rows_per_expert} rows/expert: last expert rel h {rel_h:.2e}, y {rel_y:.2e}")


def test_nvfp4_expert_scale_is_applied_per_expert(gpu):
    """Scaling one expert's fp32 matrix scale by 2 doubles exactly that
    expert's gate/up output (before the GEGLU: h = gelu(2g) * 2u), and leaves
    the others bitwise unchanged."""
    E, H, I, R = 4, 256, 128, 16
    s = mi.Shape(T=R * E, H=H, E=E, k=1, I=I, nvfp4=True)
    inp = mi.make(s, seed=12)
    d = upload(inp)
    offsets = torch.arange(E + 1, dtype=torch.int32, device="cuda") * R
    h1 = torch.empty((s.T, I), dtype=torch.bfloat16, device="cuda")
    h2 = torch.empty_like(h1)
    moe.gemm_gateup(d["shape"], d["x"], None, offsets, d["w_gu"], d["gu_s"], h1)
    g2 = inp.gu_global.copy()
    g2[2] *= 2
    s2 = dev.to_device(moe.nvfp4_scale_buffer(g2, inp.gu_scales))
    moe.gemm_gateup(d["shape"], d["x"], None, offsets, d["w_gu"], s2, h2)
    torch.cuda.synchronize()
    a, b = to64(h1), to64(h2)
    other = np.r_[0:2 * R, 3 * R:4 * R]
    assert (a[other] == b[other]).all()
    x64 = oracle.bf16_to_f64(inp.x)[2 * R:3 * R]
    wgu, _ = oracle.expert_weights(inp, 2)
    ref = oracle.gateup_geglu(x64, 2 * wgu)
    rel = np.linalg.norm(b[2 * R:3 * R] - ref) / np.linalg.norm(ref)
    assert rel < 1e-2


# ------------------------------------------------------------ NVFP4 activations
def _quantize_nv_gpu(bits, g):
    src = dev.to_device(bits)
    rows, K = bits.shape
    gs = torch.tensor([g], dtype=torch.float32, device="cuda")
    codes = torch.empty((rows, K // 2), dtype=torch.uint8, device="cuda")
    scales = torch.empty((rows, K // 16), dtype=torch.uint8, device="cuda")
    moe.quantize_nv(src, gs, codes, scales)
    torch.cuda.synchronize()
    return codes.cpu().numpy(), scales.cpu().numpy()


def _oracle_nv_packed(bits, g):
    c, s = oracle.nv_quantize(oracle.bf16_to_f64(bits), g)
    return (c[:, 0::2] | (c[:, 1::2] << 4)).astype(np.uint8), s


@pytest.mark.parametrize("rows,K,g,seed", [(1, 16, 2.0 ** -8, 0), (9, 48, 0.0037, 1), (300, 2816, 2.0 ** -8, 2),
                                           (64, 704, 1.0, 3), (33, 704, 2.0 ** -8, 4)])
def test_nv_quantizer_matches_oracle_bitwise(gpu, rows, K, g, seed):
    rng = np.random.default_rng(seed)
    v = rng.standard_normal((rows, K)) * np.exp(rng.uniform(-7, 4, (rows, 1)))
    bits = mi.f32_to_bf16_bits(v.astype(np.float32))
    codes, scales = _quantize_nv_gpu(bits, g)
    rc, rs = _oracle_nv_packed(bits, g)
    assert (scales == rs).all()
    assert (codes == rc).all()


def test_nv_quantizer_special_values(gpu):
    """Zeros and negative zeros, bf16 subnormals, E2M1 midpoints of the step
    (ties to even), E4M3 midpoints of the block scale, saturation of the
    scale at 448 and of the codes at 6."""
    g = 2.0 ** -8
    rows = [np.zeros(16, np.float32)]
    nz = np.zeros(16, np.float32); nz[::2] = -0.0; nz[5] = 1e-40; rows.append(nz)
    rows.append(np.full(16, 2.0 ** -130, np.float32))
    step = 2.0 * g
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0, -0.25, -5.0, 0, 0, 0, 0, 0, 0], np.float32) * step
    rows.append(mids)
    grid = oracle.e4m3_to_f64(np.arange(127))
    for m in ((grid[:-1] + grid[1:]) / 2)[::9]:        # block amax whose amax / (6 g) is an E4M3 midpoint
        r = np.full(16, 0.1, np.float32) * np.float32(m * 6 * g)
        r[0] = np.float32(m * 6 * g)
        rows.append(r)
    big = np.full(16, 1e4 * g, np.float32); big[0] = -3e4 * g; rows.append(big)
    bits = mi.f32_to_bf16_bits(np.stack(rows).astype(np.float32))
    codes, scales = _quantize_nv_gpu(bits, g)
    rc, rs = _oracle_nv_packed(bits, g)
    assert (scales == rs).all()
    assert (codes == rc).all()


NV_A4 = {
    "tiny-nva4": mi.Shape(T=16, H=256, E=8, k=2, I=128, nvfp4=True, nv_a4=True),
    "mid-tiles-nva4": mi.Shape(T=150, H=512, E=16, k=4, I=192, nvfp4=True, nv_a4=True),       # 64-row tiles
    "big-tiles-nva4": mi.Shape(T=600, H=512, E=16, k=4, I=320, nvfp4=True, nv_a4=True),       # 256-row tiles
    "decode-like-nva4": mi.Shape(T=8, H=768, E=64, k=8, I=704, nvfp4=True, nv_a4=True),       # the model's I
    "skew-nva4": mi.Shape(T=200, H=256, E=16, k=4, I=64, nvfp4=True, nv_a4=True, skew=True),
    "k1088-nva4": mi.Shape(T=12, H=1088, E=16, k=4, I=128, nvfp4=True, nv_a4=True),           # partial last step
}


@pytest.mark.parametrize("name", list(NV_A4))
def test_forward_nvfp4_a4_small_full_compare(gpu, name):
    s = NV_A4[name]
    say(f"forward nvfp4 w4a4 {name}: {s}")
    inp = mi.make(s, seed=8)
    out, ids, w = run_forward(inp)
    ref = oracle.forward(inp)
    check_layer(to64(out), ids.cpu().numpy(), w.cpu().numpy(), ref["ids"], ref["w"], ref["out"],
                ref["margin"], name)


@pytest.mark.parametrize("name", ["nvfp4_a4_decode", "nvfp4_a4"])
def test_forward_nvfp4_a4_full_size(gpu, name):
    """The Gemma-4 layer with NVFP4 weights and activations at decode (8
    tokens) and prefill (2048 tokens) size, every token against the oracle's
    whole forward."""
    s = mi.CONFIGS[name]
    say(f"forward nvfp4 w4a4 full size: {s}")
    inp = mi.make(name, seed=0)
    out, ids, w = run_forward(inp)
    ref = oracle.forward(inp)
    check_layer(to64(out), ids.cpu().numpy(), w.cpu().numpy(), ref["ids"], ref["w"], ref["out"],
                ref["margin"], f"{name} (all {s.T} tokens)")


def test_forward_nvfp4_a4_differs_from_weight_only(gpu):
    """The activations really are quantised: NVFP4 W4A4 and NVFP4 weights
    with bf16 activations differ by about the activation quantisation error."""
    import dataclasses
    s = NV_A4["mid-tiles-nva4"]
    inp = mi.make(s, seed=9)
    o4, _, _ = run_forward(inp)
    o16, _, _ = run_forward(dataclasses.replace(inp, shape=dataclasses.replace(s, nv_a4=False)))
    rel = np.linalg.norm(to64(o4) - to64(o16)) / np.linalg.norm(to64(o16))
    say(f"nvfp4 w4a4 vs weight-only rel difference {rel:.3e}")
    assert 1e-2 < rel < 0.5
