"""Helpers shared by the GPU parity tests: upload generator inputs, run the
C ABI, compare against the oracle."""
import sys

import numpy as np
import torch

import moe_inputs as mi
import mixture_experts_router_amd as moe
from mixture_experts_router_amd import device as dev

# Output tolerance of the layer (bf16 in/out, fp32 accumulation).
REL_L2 = 1e-2
MAX_ABS = 3e-2
# Tokens whose oracle routing margin (k-th minus (k+1)-th logit) is below
# this are near ties: counted and excluded from the output comparison.
TIE_MARGIN = 1e-6


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def upload(inp):
    d = dict(
        x=dev.to_device(inp.x),
        w_router=dev.to_device(inp.w_router),
        bias=dev.to_device(inp.router_bias) if inp.router_bias is not None else None,
        w_gu=dev.to_device(inp.w_gate_up),
        w_d=dev.to_device(inp.w_down),
        gu_s=dev.to_device(inp.gu_scales) if inp.gu_scales is not None else None,
        d_s=dev.to_device(inp.d_scales) if inp.d_scales is not None else None,
    )
    s = inp.shape
    if s.nvfp4:   # one scale buffer per matrix: fp32 expert scales (+ input scale), then E4M3 codes
        gi = inp.gu_input_scale if s.nv_a4 else 1.0
        di = inp.d_input_scale if s.nv_a4 else 1.0
        d["gu_s"] = dev.to_device(moe.nvfp4_scale_buffer(inp.gu_global, inp.gu_scales, gi))
        d["d_s"] = dev.to_device(moe.nvfp4_scale_buffer(inp.d_global, inp.d_scales, di))
    d["shape"] = moe.shape(s.T, s.H, s.E, s.k, s.I, mxfp4=s.mxfp4, a4=s.a4, nvfp4=s.nvfp4, nv_a4=s.nv_a4)
    if s.I_sh > 0:
        d["sh_gu"] = dev.to_device(inp.w_sh_gate_up)
        d["sh_d"] = dev.to_device(inp.w_sh_down)
        d["sh_gu_s"] = dev.to_device(inp.sh_gu_scales) if inp.sh_gu_scales is not None else None
        d["sh_d_s"] = dev.to_device(inp.sh_d_scales) if inp.sh_d_scales is not None else None
    return d


def run_forward_shared(inp, d=None, ws=None):
    """moe_forward_shared on generator inputs whose shape has I_sh > 0."""
    d = d or upload(inp)
    s = inp.shape
    sh = d["shape"]
    out = torch.empty((s.T, s.H), dtype=torch.bfloat16, device="cuda")
    ids = torch.empty((s.T, s.k), dtype=torch.int32, device="cuda")
    w = torch.empty((s.T, s.k), dtype=torch.float32, device="cuda")
    ws = ws if ws is not None else dev.workspace(sh, I_sh=s.I_sh)
    moe.forward_shared(sh, d["x"], d["w_router"], d["bias"], d["w_gu"], d["gu_s"], d["w_d"], d["d_s"], s.I_sh,
                       d["sh_gu"], d["sh_gu_s"], d["sh_d"], d["sh_d_s"], out, ids, w, ws)
    torch.cuda.synchronize()
    return out, ids, w


def run_forward(inp, d=None, ws=None):
    d = d or upload(inp)
    s = inp.shape
    sh = d["shape"]
    out = torch.empty((s.T, s.H), dtype=torch.bfloat16, device="cuda")
    ids = torch.empty((s.T, s.k), dtype=torch.int32, device="cuda")
    w = torch.empty((s.T, s.k), dtype=torch.float32, device="cuda")
    ws = ws if ws is not None else dev.workspace(sh)
    moe.forward(sh, d["x"], d["w_router"], d["bias"], d["w_gu"], d["gu_s"], d["w_d"], d["d_s"],
                out, ids, w, ws)
    torch.cuda.synchronize()
    return out, ids, w


def to64(t):
    return t.float().cpu().numpy().astype(np.float64)


def compare_out(got, ref, keep):
    """rel-L2 and max-abs over the kept tokens."""
    d = got[keep] - ref[keep]
    rel = np.linalg.norm(d) / max(np.linalg.norm(ref[keep]), 1e-300)
    mx = float(np.abs(d).max()) if d.size else 0.0
    return rel, mx


def check_layer(got_out, got_ids, got_w, ref_ids, ref_w, ref_out, margin, label):
    """The layer's acceptance: routing equal outside near ties, output within
    tolerance over the tokens that are not near ties."""
    keep = margin >= TIE_MARGIN
    ties = int((~keep).sum())
    same_set = np.array([set(a) == set(b) for a, b in zip(got_ids, ref_ids)])
    flips = int((~same_set & keep).sum())
    rel, mx = compare_out(got_out, ref_out, keep)
    wsum = np.abs(got_w.sum(axis=1) - 1).max()
    say(f"{label}: near-tie tokens {ties}, routing flips outside ties {flips}, "
        f"rel_l2 {rel:.3e}, max_abs {mx:.3e}, max|sum w - 1| {wsum:.2e}")
    assert flips == 0, f"{label}: {flips} routing differences at margin >= {TIE_MARGIN}"
    assert rel <= REL_L2 and mx <= MAX_ABS, f"{label}: rel {rel} max {mx}"
    assert wsum <= 1e-6
    return rel, mx
