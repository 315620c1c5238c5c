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
