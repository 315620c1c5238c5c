"""The bounds-checked build (libmoe_debug.so, include/moe_debug.h) run over
the shapes the parity tests use -- every entry point, every tile size and
weight format, the full-size workloads -- must record no out-of-range
address.  A positive control feeds the combine one row index past the end
of y (into slack rows of the same allocation) and must see it recorded.
Runs in a child process so that the debug library is the only one loaded."""
import ctypes
import os
import subprocess
import sys

import pytest

from mixture_experts_router_amd import build as b

pytestmark = pytest.mark.gpu
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CHILD = r'''
import ctypes, sys
import numpy as np, torch
sys.path.insert(0, "tests")
import moe_inputs as mi
import mixture_experts_router_amd as moe
from mixture_experts_router_amd import device as dev
lib = moe.load(sys.argv[1])
lib.moe_debug_bounds.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
from gpu_helpers import upload, run_forward, run_forward_shared

def bounds(label):
    v, w = ctypes.c_uint32(), ctypes.c_uint32()
    assert lib.moe_debug_bounds(ctypes.byref(v), ctypes.byref(w)) == 0
    print(f"{label}: violations {v.value} first at {w.value}", flush=True)
    return v.value, w.value

S = mi.Shape
FORWARD = [S(T=16, H=256, E=8, k=2, I=128), S(T=300, H=512, E=16, k=4, I=192),
           S(T=150, H=512, E=16, k=4, I=192, mxfp4=True), S(T=1200, H=512, E=16, k=4, I=192, mxfp4=True),
           S(T=12, H=1152, E=16, k=4, I=128, mxfp4=True), S(T=130, H=256, E=300, k=6, I=64),
           S(T=700, H=512, E=16, k=4, I=192, skew=True), S(T=1, H=256, E=8, k=2, I=128),
           S(T=40, H=256, E=8, k=8, I=128),
           S(T=120, H=512, E=16, k=4, I=192, mxfp4=True, a4=True), S(T=600, H=512, E=16, k=4, I=320, mxfp4=True, a4=True),
           S(T=300, H=2816, E=128, k=8, I=704, mxfp4=True, a4=True),
           S(T=150, H=512, E=16, k=4, I=192, nvfp4=True), S(T=600, H=512, E=16, k=4, I=320, nvfp4=True),
           S(T=12, H=1088, E=16, k=4, I=128, nvfp4=True, nv_a4=True), S(T=600, H=512, E=16, k=4, I=320, nvfp4=True, nv_a4=True)]
for s in FORWARD:
    run_forward(mi.make(s, seed=1))
    assert bounds(f"forward {s}")[0] == 0
for name in ["decode", "prefill", "skew", "mxfp4", "w4a4", "nvfp4_decode", "nvfp4_a4"]:
    run_forward(mi.make(name, seed=0))
    assert bounds(f"forward {name}")[0] == 0
for s in [S(T=16, H=256, E=8, k=2, I=128, I_sh=192), S(T=150, H=512, E=16, k=4, I=192, I_sh=256),
          S(T=300, H=512, E=16, k=4, I=192, I_sh=256, mxfp4=True), S(T=8, H=2816, E=128, k=8, I=704, I_sh=2112)]:
    run_forward_shared(mi.make(s, seed=2))
    assert bounds(f"forward_shared {s}")[0] == 0
# the no-alloc variant, and the step entry points with a gathered copy of x
inp = mi.make(S(T=40, H=512, E=16, k=4, I=192), seed=3)
d = upload(inp)
s, sh = inp.shape, d["shape"]
out = torch.empty((s.T, s.H), dtype=torch.bfloat16, device="cuda")
moe.forward_noalloc(sh, d["x"], d["w_router"], None, d["w_gu"], None, d["w_d"], None, out)
A = s.T * s.k
i32 = dict(dtype=torch.int32, device="cuda")
logits = torch.empty((s.T, s.E), dtype=torch.float32, device="cuda")
ids, w = torch.empty((s.T, s.k), **i32), torch.empty((s.T, s.k), dtype=torch.float32, device="cuda")
rws = torch.empty(max(1, moe.route_workspace_bytes(sh)), dtype=torch.uint8, device="cuda")
moe.route(sh, d["x"], d["w_router"], None, logits, ids, w, ws=rws)
moe.route(sh, None, None, None, logits, ids, w)
counts, offsets = torch.empty(s.E, **i32), torch.empty(s.E + 1, **i32)
sid, inv = torch.empty(A, **i32), torch.empty(A, **i32)
xp = torch.empty((A, s.H), dtype=torch.bfloat16, device="cuda")
pws = torch.empty(moe.permute_workspace_bytes(sh), dtype=torch.uint8, device="cuda")
moe.permute(sh, ids, d["x"], counts, offsets, sid, inv, xp, pws)
h = torch.empty((A, s.I), dtype=torch.bfloat16, device="cuda")
y = torch.empty((A, s.H), dtype=torch.bfloat16, device="cuda")
moe.gemm_gateup(sh, d["x"], sid, offsets, d["w_gu"], None, h)
moe.gemm_gateup(sh, xp, None, offsets, d["w_gu"], None, h)
moe.gemm_down(sh, h, offsets, d["w_d"], None, y)
moe.combine(sh, y, inv, w, out)
codes = torch.empty((A, s.I // 2), dtype=torch.uint8, device="cuda")
moe.quantize_mx(h, codes, torch.empty((A, s.I // 32), dtype=torch.uint8, device="cuda"))
g = torch.tensor([2.0 ** -8], dtype=torch.float32, device="cuda")
moe.quantize_nv(h, g, codes, torch.empty((A, s.I // 16), dtype=torch.uint8, device="cuda"))
assert bounds("noalloc, route, permute, step GEMMs, combine, quantisers")[0] == 0
# positive control: one token's first slot points one row past y's A rows
# (y has slack rows, so the unchecked address would still be in the buffer)
y_slack = torch.zeros((A + 16, s.H), dtype=torch.bfloat16, device="cuda")
bad = inv.clone()
bad[0] = A + 3
moe.combine(sh, y_slack[:A], bad, w, out)
v, where = bounds("combine with an index past the end of y")
assert v == s.H // 8 and where // 100000 == 4, (v, where)
print("__DEBUG_BOUNDS_OK__", flush=True)
'''


def test_debug_build_records_no_out_of_range_access():
    if not os.path.exists(b.DEBUG_LIB):
        pytest.fail(f"{b.DEBUG_LIB} is missing: build it with build(debug=True)")
    r = subprocess.run([sys.executable, "-u", "-c", CHILD, b.DEBUG_LIB], cwd=ROOT, capture_output=True, text=True,
                       timeout=900)
    print(r.stdout[-6000:])
    assert r.returncode == 0 and "__DEBUG_BOUNDS_OK__" in r.stdout, r.stdout[-3000:] + r.stderr[-3000:]
