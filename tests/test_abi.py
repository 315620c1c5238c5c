"""The C ABI on the CPU: the library loads, exports every entry point of
include/moe.h, and rejects bad arguments on the host before any HIP call.
Every call here fails validation, so nothing is launched."""
import ctypes
import os
import re

import pytest

import mixture_experts_router_amd as moe
from mixture_experts_router_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")
FAKE = 0x100000          # a 256-byte aligned non-NULL address that is never dereferenced
MIS = FAKE + 2            # misaligned


@pytest.fixture(scope="module")
def lib():
    # MOE_TEST_LIB: run these checks against another build of the library
    # (the host-sanitised one, from test_sanitizers.py)
    return moe.load(os.environ.get("MOE_TEST_LIB", _lib.LIB_PATH))


def declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(moe_\w+)\s*\(", text, re.M)))


def test_header_declares_the_exports(lib):
    names = declared()
    assert set(names) == set(_lib.EXPORTS)
    for n in names:
        assert hasattr(lib, n)


def test_single_hip_runtime_in_process(lib):
    maps = [l.split()[-1] for l in open("/proc/self/maps") if "libamdhip64" in l]
    assert len(set(maps)) == 1


def test_status_strings(lib):
    for st, name in [(0, "ok"), (-1, "invalid"), (-2, "unsupported"), (-3, "workspace"), (-4, "HIP")]:
        assert name in lib.moe_status_string(st).decode()
    assert lib.moe_status_string(7) is not None


def S(T=16, H=256, E=8, k=2, I=128, f=0):
    return _lib.MoeShape(T, H, E, k, I, f)


@pytest.mark.parametrize("s,expect", [
    (S(T=0), -1), (S(H=0), -1), (S(E=0), -1), (S(k=0), -1), (S(I=0), -1), (S(k=9), -1),
    (S(H=96), -2), (S(I=100), -2), (S(E=2000, k=8), -2), (S(E=64, k=33), -2), (S(f=5), -2),
    (S(T=1 << 28, k=8), -2),
])
def test_bad_shapes_rejected_everywhere(lib, s, expect):
    b = ctypes.byref(s)
    F = FAKE
    assert lib.moe_route(b, F, F, None, F, F, F, F, 1 << 30, None) == expect
    assert lib.moe_permute(b, F, None, F, F, F, F, None, F, 1 << 30, None) == expect
    assert lib.moe_grouped_gemm_gateup(b, F, F, F, F, None, F, None) == expect
    assert lib.moe_grouped_gemm_down(b, F, F, F, None, F, None) == expect
    assert lib.moe_combine(b, F, F, F, F, None) == expect
    assert lib.moe_forward(b, F, F, None, F, None, F, None, F, None, None, F, 1 << 40, None, None) == expect
    assert lib.moe_workspace_bytes(b) == 0 and lib.moe_permute_workspace_bytes(b) == 0
    assert lib.moe_route_workspace_bytes(b) == 0
    assert lib.moe_route(None, F, F, None, F, F, F, F, 1 << 30, None) == -1


def test_null_and_misaligned_pointers(lib):
    s = S()
    b = ctypes.byref(s)
    F = FAKE
    assert lib.moe_route(b, F, None, None, F, F, F, F, 1 << 20, None) == -1        # x without router weight
    assert lib.moe_route(b, MIS, F, None, F, F, F, F, 1 << 20, None) == -1         # misaligned x
    assert lib.moe_route(b, None, None, None, None, F, F, None, 0, None) == -1     # no logits
    need_r = lib.moe_route_workspace_bytes(b)
    assert need_r > 0                                                             # T=16: split-K router
    assert lib.moe_route(b, F, F, None, F, F, F, None, 0, None) == -3
    assert lib.moe_route(b, F, F, None, F, F, F, F, need_r - 4, None) == -3
    assert lib.moe_permute(b, None, None, F, F, F, F, None, F, 1 << 20, None) == -1
    assert lib.moe_permute(b, F, F, F, F, F, F, None, F, 1 << 20, None) == -1   # x without x_perm
    assert lib.moe_permute(b, F, None, F, F, F, F, None, None, 1 << 20, None) == -3
    assert lib.moe_permute(b, F, None, F, F, F, F, None, F, 4, None) == -3
    assert lib.moe_grouped_gemm_gateup(b, F, None, F, F, F, F, None) == -1     # bf16 with scales
    assert lib.moe_grouped_gemm_gateup(b, F, None, F, MIS, None, F, None) == -1
    mx = S(f=1)
    assert lib.moe_grouped_gemm_gateup(ctypes.byref(mx), F, None, F, F, None, F, None) == -1  # mx without scales
    assert lib.moe_grouped_gemm_down(b, F, F, None, None, F, None) == -1
    assert lib.moe_combine(b, F, F, F, MIS, None) == -1
    need = lib.moe_workspace_bytes(b)
    assert need > 0
    assert lib.moe_forward(b, F, F, None, F, None, F, None, F, None, None, F, need - 1, None, None) == -3
    assert lib.moe_forward(b, F, F, None, F, None, F, None, F, None, None, None, need, None, None) == -3
    ev = (ctypes.c_void_p * 6)(F, F, F, None, F, F)
    assert lib.moe_forward(b, F, F, None, F, None, F, None, F, None, None, F, need,
                           None, ctypes.cast(ev, ctypes.c_void_p)) == -1


def test_route_workspace(lib):
    small = _lib.MoeShape(8, 2816, 128, 8, 704, 0)
    big = _lib.MoeShape(2048, 2816, 128, 8, 704, 0)
    # few tokens: fp32 partial sums of 11 chunks of 256; many tokens: none
    assert lib.moe_route_workspace_bytes(ctypes.byref(small)) >= 11 * 8 * 128 * 4
    assert lib.moe_route_workspace_bytes(ctypes.byref(big)) == 0


def test_workspace_monotone_in_T(lib):
    prev = 0
    for T in (1, 7, 8, 100, 2048, 8192):
        s = _lib.MoeShape(T, 2816, 128, 8, 704, 0)
        n = lib.moe_workspace_bytes(ctypes.byref(s))
        assert n > prev and n % 256 == 0
        prev = n
    s = _lib.MoeShape(2048, 2816, 128, 8, 704, 0)
    # h and y dominate: T*k*(I + H) bf16
    assert lib.moe_workspace_bytes(ctypes.byref(s)) >= 2048 * 8 * (704 + 2816) * 2


def test_missing_library_fails_loudly(tmp_path):
    with pytest.raises(RuntimeError, match="missing"):
        _lib.load.__wrapped__(str(tmp_path / "nope.so")) if hasattr(_lib.load, "__wrapped__") else \
            _load_fresh(str(tmp_path / "nope.so"))


def _load_fresh(path):
    saved = _lib._lib
    _lib._lib = None
    try:
        return _lib.load(path)
    finally:
        _lib._lib = saved


def test_forward_shared_argument_checks(lib):
    s = S()
    b = ctypes.byref(s)
    F = FAKE
    big = 1 << 40
    args = lambda I_sh, gu=F, d=F, gus=None, ds=None: (b, F, F, None, F, None, F, None, I_sh, gu, gus, d, ds,
                                                         F, None, None, F, big, None, None)
    assert lib.moe_forward_shared(*args(0)) == -1            # no dense MLP: use moe_forward
    assert lib.moe_forward_shared(*args(-64)) == -1
    assert lib.moe_forward_shared(*args(100)) == -2          # not a multiple of 64
    assert lib.moe_forward_shared(*args(128, gu=None)) == -1
    assert lib.moe_forward_shared(*args(128, d=MIS)) == -1   # bf16 weights must be 16-byte aligned
    assert lib.moe_forward_shared(*args(128, gus=F)) == -1   # bf16 weights come without scales
    small = (b, F, F, None, F, None, F, None, 128, F, None, F, None, F, None, None, F, 64, None, None)
    assert lib.moe_forward_shared(*small) == -3


def test_shared_workspace_sizes(lib):
    s = S(T=16)
    base = lib.moe_workspace_bytes(ctypes.byref(s))
    a = lib.moe_workspace_shared_bytes(ctypes.byref(s), 128)
    b2 = lib.moe_workspace_shared_bytes(ctypes.byref(s), 256)
    assert base < a < b2
    assert a - base >= 16 * 128 * 2 + 16 * 256 * 2       # h and output rows of the dense MLP
    assert lib.moe_workspace_shared_bytes(ctypes.byref(s), 0) == 0
    assert lib.moe_workspace_shared_bytes(ctypes.byref(s), 100) == 0
    assert lib.moe_workspace_shared_bytes(ctypes.byref(S(T=0)), 128) == 0


def test_w4a4_argument_checks(lib):
    s = S(f=2)
    b = ctypes.byref(s)
    F = FAKE
    # the per-step GEMM entry points do not take W4A4
    assert lib.moe_grouped_gemm_gateup(b, F, F, F, F, F, F, None) == -2
    assert lib.moe_grouped_gemm_down(b, F, F, F, F, F, None) == -2
    # W4A4 weight codes must be 16-byte aligned (plain MXFP4 needs 4)
    big = 1 << 40
    assert lib.moe_forward(b, F, F, None, F + 4, F, F, F, F, None, None, F, big, None, None) == -1
    # no dense MLP with W4A4
    assert lib.moe_forward_shared(b, F, F, None, F, F, F, F, 128, F, F, F, F, F, None, None, F, big, None,
                                  None) == -2
    # quantiser: K a positive multiple of 32, aligned pointers
    assert lib.moe_quantize_mx(F, 4, 48, F, F, None) == -2
    assert lib.moe_quantize_mx(F, 4, 0, F, F, None) == -1
    assert lib.moe_quantize_mx(F, -1, 64, F, F, None) == -1
    assert lib.moe_quantize_mx(MIS, 4, 64, F, F, None) == -1
    assert lib.moe_quantize_mx(None, 0, 64, None, None, None) == 0     # nothing to do


def test_nvfp4_argument_checks(lib):
    s = S(f=3)
    b = ctypes.byref(s)
    F = FAKE
    big = 1 << 40
    # NVFP4 needs a scale buffer, 4-byte aligned (fp32 header, 32-bit scale loads)
    assert lib.moe_forward(b, F, F, None, F, None, F, F, F, None, None, F, big, None, None) == -1
    assert lib.moe_forward(b, F, F, None, F, F + 2, F, F, F, None, None, F, big, None, None) == -1
    assert lib.moe_grouped_gemm_gateup(b, F, F, F, F, F + 2, F, None) == -1
    assert lib.moe_grouped_gemm_down(b, F, F, F, None, F, None) == -1
    # codes 4-byte aligned
    assert lib.moe_forward(b, F, F, None, F + 2, F, F, F, F, None, None, F, big, None, None) == -1
    # no dense MLP with NVFP4 experts
    assert lib.moe_forward_shared(b, F, F, None, F, F, F, F, 128, F, F, F, F, F, None, None, F, big, None,
                                  None) == -2
    # same workspace as bf16 (the weights are read in place)
    assert lib.moe_workspace_bytes(b) == lib.moe_workspace_bytes(ctypes.byref(S(f=0)))


def test_nvfp4_header_size():
    text = open(HEADER).read()
    assert "#define MOE_NVFP4_HEADER_BYTES(E)" in text
    # E matrix scales and the activation input scale, padded to 256
    for E, n in [(1, 256), (8, 256), (63, 256), (64, 512), (65, 512), (128, 768), (1024, 4352)]:
        assert moe.nvfp4_header_bytes(E) == n
    import numpy as np
    buf = moe.nvfp4_scale_buffer(np.array([1.5, -2.0], np.float32), np.arange(6, dtype=np.uint8).reshape(2, 1, 3),
                                 0.25)
    assert buf.size == 256 + 6
    assert buf[:12].view(np.float32).tolist() == [1.5, -2.0, 0.25]
    assert (buf[12:256] == 0).all() and buf[256:].tolist() == list(range(6))
    assert moe.nvfp4_scale_buffer(np.ones(2, np.float32), np.zeros(3, np.uint8))[8:12].view(np.float32)[0] == 1.0


def test_forward_noalloc_argument_checks(lib):
    """moe_forward_noalloc checks its arguments like moe_forward, and rejects
    shapes whose workspace exceeds its built-in scratch, before any launch."""
    F = FAKE
    call = lambda s, x=F, wr=F, gu=F, gus=None, d=F, ds=None, out=F: lib.moe_forward_noalloc(
        ctypes.byref(s), x, wr, None, gu, gus, d, ds, out, None, None, None)
    assert call(S(T=0)) == -1
    assert call(S(H=96)) == -2
    assert call(S(), x=None) == -1
    assert call(S(), out=MIS) == -1
    assert call(S(), gus=F) == -1                         # bf16 weights come without scales
    assert call(S(f=1)) == -1                             # MXFP4 weights need scales
    text = open(HEADER).read()
    assert "#define MOE_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)" in text
    assert _lib.NOALLOC_SCRATCH_BYTES == 64 << 20
    fits = _lib.MoeShape(1000, 2816, 128, 8, 704, 0)
    too_big = _lib.MoeShape(2048, 2816, 128, 8, 704, 0)
    assert lib.moe_workspace_bytes(ctypes.byref(fits)) <= _lib.NOALLOC_SCRATCH_BYTES
    assert lib.moe_workspace_bytes(ctypes.byref(too_big)) > _lib.NOALLOC_SCRATCH_BYTES
    assert call(too_big) == -5
    assert call(_lib.MoeShape(2048, 2816, 128, 8, 704, 1), gus=F, ds=F) == -5
    assert "scratch" in lib.moe_status_string(-5).decode()


def test_nvfp4_activation_checks(lib):
    """MOE_W_NVFP4_A4 runs through moe_forward only, without a dense MLP;
    moe_quantize_nv wants K % 16 == 0 and aligned pointers."""
    s = S(f=4)
    b = ctypes.byref(s)
    F = FAKE
    big = 1 << 40
    assert lib.moe_grouped_gemm_gateup(b, F, F, F, F, F, F, None) == -2
    assert lib.moe_grouped_gemm_down(b, F, F, F, F, F, None) == -2
    assert lib.moe_forward(b, F, F, None, F, None, F, F, F, None, None, F, big, None, None) == -1   # scales
    assert lib.moe_forward_shared(b, F, F, None, F, F, F, F, 128, F, F, F, F, F, None, None, F, big, None,
                                  None) == -2
    # the workspace adds the quantised x: T*H bf16
    assert lib.moe_workspace_bytes(b) >= lib.moe_workspace_bytes(ctypes.byref(S(f=3))) + 16 * 256 * 2
    assert lib.moe_quantize_nv(F, 4, 24, F, F, F, None) == -2
    assert lib.moe_quantize_nv(F, 4, 0, F, F, F, None) == -1
    assert lib.moe_quantize_nv(F, -1, 32, F, F, F, None) == -1
    assert lib.moe_quantize_nv(MIS, 4, 32, F, F, F, None) == -1
    assert lib.moe_quantize_nv(F, 4, 32, None, F, F, None) == -1
    assert lib.moe_quantize_nv(F, 4, 32, F, F + 4, F, None) == -1     # codes 8-byte aligned
    assert lib.moe_quantize_nv(None, 0, 32, None, None, None, None) == 0


def test_debug_header_and_exports():
    """include/moe_debug.h declares the query of the bounds-checked build:
    libmoe_debug.so exports it (and every moe.h entry point), the release
    library does not."""
    import subprocess
    from mixture_experts_router_amd import build as b
    text = open(os.path.join(ROOT, "include", "moe_debug.h")).read()
    assert re.findall(r"^\s*int\s+(moe_\w+)\s*\(", text, re.M) == ["moe_debug_bounds"]
    if not os.path.exists(b.DEBUG_LIB):
        pytest.skip("libmoe_debug.so not built")
    names = lambda path: set(subprocess.run(["nm", "-D", "--defined-only", path], capture_output=True, text=True,
                                            check=True).stdout.split())
    dbg, rel = names(b.DEBUG_LIB), names(_lib.LIB_PATH)
    assert "moe_debug_bounds" in dbg and "moe_debug_bounds" not in rel
    assert set(_lib.EXPORTS) <= dbg


def test_probe_header_and_exports():
    """include/moe_probe.h declares the streaming probes of libmoe_probe.so:
    the library exports exactly those, names and sizes every kind, and
    rejects bad arguments before any HIP call."""
    from mixture_experts_router_amd import build as b
    text = open(os.path.join(ROOT, "include", "moe_probe.h")).read()
    decl = sorted(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(moe_\w+)\s*\(", text, re.M))
    assert decl == ["moe_probe_bytes", "moe_probe_count", "moe_probe_footprint", "moe_probe_launch",
                    "moe_probe_name"]
    if not os.path.exists(b.PROBE_LIB):
        pytest.skip("libmoe_probe.so not built")
    p = ctypes.CDLL(b.PROBE_LIB)
    for n in decl:
        assert hasattr(p, n)
    p.moe_probe_name.restype = ctypes.c_char_p
    p.moe_probe_bytes.restype = ctypes.c_size_t
    p.moe_probe_footprint.restype = ctypes.c_size_t
    p.moe_probe_launch.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p,
                                   ctypes.c_void_p]
    n = p.moe_probe_count()
    assert n >= 1
    for k in range(n):
        assert p.moe_probe_name(k) and p.moe_probe_bytes(k) >= p.moe_probe_footprint(k)
        assert p.moe_probe_bytes(k) > 0
    assert p.moe_probe_name(n) is None and p.moe_probe_bytes(n) == 0 and p.moe_probe_bytes(-1) == 0
    assert p.moe_probe_footprint(n) == 0
    big = p.moe_probe_footprint(0)
    assert big == p.moe_probe_bytes(0)
    assert p.moe_probe_launch(n, FAKE, big, FAKE, None) == -1          # unknown kind
    assert p.moe_probe_launch(0, None, big, FAKE, None) == -1          # no buffer
    assert p.moe_probe_launch(0, FAKE, big, None, None) == -1          # no sink
    assert p.moe_probe_launch(0, FAKE, big - 1, FAKE, None) == -1      # short buffer
    assert p.moe_probe_launch(0, MIS, big, FAKE, None) == -1           # misaligned buffer
    # the layer library does not carry the probes
    rel = ctypes.CDLL(_lib.LIB_PATH)
    assert not hasattr(rel, "moe_probe_launch")
