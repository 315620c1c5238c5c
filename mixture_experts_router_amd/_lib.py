"""ctypes binding of libmoe.so (include/moe.h).  Argument marshalling only:
every step of the layer runs in the library's HIP kernels.  torch provides
device memory and the current stream."""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmoe.so")

MOE_W_BF16, MOE_W_MXFP4, MOE_W_MXFP4_A4, MOE_W_NVFP4, MOE_W_NVFP4_A4 = 0, 1, 2, 3, 4
MOE_FORWARD_STAGES = 5
STATUS = {0: "MOE_OK", -1: "MOE_ERR_INVALID_ARGUMENT", -2: "MOE_ERR_UNSUPPORTED",
          -3: "MOE_ERR_WORKSPACE", -4: "MOE_ERR_HIP", -5: "MOE_ERR_SCRATCH_TOO_SMALL"}
# MOE_NOALLOC_SCRATCH_BYTES: the scratch moe_forward_noalloc holds per GPU.
NOALLOC_SCRATCH_BYTES = 64 << 20

# Entry points declared in include/moe.h.
EXPORTS = ("moe_route", "moe_permute", "moe_grouped_gemm_gateup", "moe_grouped_gemm_down",
           "moe_combine", "moe_forward", "moe_forward_shared", "moe_workspace_bytes",
           "moe_workspace_shared_bytes", "moe_route_workspace_bytes", "moe_permute_workspace_bytes",
           "moe_quantize_mx", "moe_quantize_nv", "moe_forward_noalloc", "moe_status_string")


class MoeShape(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int32), ("H", ctypes.c_int32), ("E", ctypes.c_int32),
                ("k", ctypes.c_int32), ("I", ctypes.c_int32), ("w_format", ctypes.c_int32)]

    def __repr__(self):
        return (f"MoeShape(T={self.T}, H={self.H}, E={self.E}, k={self.k}, I={self.I}, "
                f"w_format={self.w_format})")


class MoeError(RuntimeError):
    def __init__(self, fn, status, msg):
        super().__init__(f"{fn} failed: {STATUS.get(status, status)} ({msg})")
        self.status = status


_lib = None
_P = ctypes.c_void_p
_S = ctypes.POINTER(MoeShape)


def load(path: str = LIB_PATH):
    """Load libmoe.so.  torch is imported first so that the library binds to
    the HIP runtime torch already uses (one runtime per process)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with mixture_experts_router_amd.build.build()")
    import torch  # noqa: F401  (loads torch's libamdhip64 before ours)
    lib = ctypes.CDLL(path)
    c_int, c_size = ctypes.c_int, ctypes.c_size_t
    sig = {
        "moe_route": [_S, _P, _P, _P, _P, _P, _P, _P, c_size, _P],
        "moe_permute": [_S, _P, _P, _P, _P, _P, _P, _P, _P, c_size, _P],
        "moe_grouped_gemm_gateup": [_S, _P, _P, _P, _P, _P, _P, _P],
        "moe_grouped_gemm_down": [_S, _P, _P, _P, _P, _P, _P],
        "moe_combine": [_S, _P, _P, _P, _P, _P],
        "moe_forward": [_S, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, c_size, _P, _P],
        "moe_forward_noalloc": [_S, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P],
        "moe_forward_shared": [_S, _P, _P, _P, _P, _P, _P, _P, ctypes.c_int32, _P, _P, _P, _P, _P, _P, _P, _P,
                               c_size, _P, _P],
    }
    for name, args in sig.items():
        f = getattr(lib, name)
        f.argtypes = args
        f.restype = c_int
    for name in ("moe_workspace_bytes", "moe_route_workspace_bytes", "moe_permute_workspace_bytes"):
        f = getattr(lib, name)
        f.argtypes = [_S]
        f.restype = c_size
    lib.moe_quantize_mx.argtypes = [_P, ctypes.c_int64, ctypes.c_int32, _P, _P, _P]
    lib.moe_quantize_mx.restype = c_int
    lib.moe_quantize_nv.argtypes = [_P, ctypes.c_int64, ctypes.c_int32, _P, _P, _P, _P]
    lib.moe_quantize_nv.restype = c_int
    lib.moe_workspace_shared_bytes.argtypes = [_S, ctypes.c_int32]
    lib.moe_workspace_shared_bytes.restype = c_size
    lib.moe_status_string.argtypes = [c_int]
    lib.moe_status_string.restype = ctypes.c_char_p
    _lib = lib
    return lib


def shape(T, H, E, k, I, mxfp4=False, a4=False, nvfp4=False, nv_a4=False) -> MoeShape:
    if nvfp4:
        fmt = MOE_W_NVFP4_A4 if nv_a4 else MOE_W_NVFP4
    else:
        fmt = MOE_W_MXFP4_A4 if a4 else (MOE_W_MXFP4 if mxfp4 else MOE_W_BF16)
    return MoeShape(T, H, E, k, I, fmt)


def nvfp4_header_bytes(E: int) -> int:
    """MOE_NVFP4_HEADER_BYTES(E): bytes of the E fp32 matrix scales and the
    fp32 activation input scale, padded to 256, in front of the E4M3 codes of
    an NVFP4 scale buffer."""
    return ((E + 1) * 4 + 255) // 256 * 256


def nvfp4_scale_buffer(matrix_scales, block_scales, input_scale=1.0):
    """Host bytes of one NVFP4 scale argument: the E fp32 matrix scales and
    the activation input scale (read with NVFP4 activations only), padded to
    nvfp4_header_bytes(E), followed by the E4M3 codes [E][rows][K/16] (numpy
    arrays in, a flat uint8 numpy array out)."""
    import numpy as np
    g = np.concatenate([np.ascontiguousarray(matrix_scales, dtype=np.float32).reshape(-1),
                        np.array([input_scale], dtype=np.float32)])
    head = np.zeros(nvfp4_header_bytes(g.size - 1), dtype=np.uint8)
    head[:g.size * 4] = g.view(np.uint8)
    return np.concatenate([head, np.ascontiguousarray(block_scales, dtype=np.uint8).reshape(-1)])


def _ptr(t):
    """Device address of a contiguous CUDA tensor (None -> NULL)."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not t.is_cuda:
        raise ValueError("expected a device tensor")
    if not t.is_contiguous():
        raise ValueError("expected a contiguous tensor")
    return t.data_ptr()


def _stream(stream):
    import torch
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _check(fn, st):
    if st != 0:
        raise MoeError(fn, st, _lib.moe_status_string(st).decode())


def workspace_bytes(s: MoeShape) -> int:
    return load().moe_workspace_bytes(ctypes.byref(s))


def workspace_shared_bytes(s: MoeShape, I_sh: int) -> int:
    return load().moe_workspace_shared_bytes(ctypes.byref(s), I_sh)


def route_workspace_bytes(s: MoeShape) -> int:
    return load().moe_route_workspace_bytes(ctypes.byref(s))


def permute_workspace_bytes(s: MoeShape) -> int:
    return load().moe_permute_workspace_bytes(ctypes.byref(s))


def route(s, x, w_router, router_bias, logits, topk_ids, topk_w, ws=None, stream=None):
    lib = load()
    nbytes = ws.numel() * ws.element_size() if ws is not None else 0
    _check("moe_route", lib.moe_route(ctypes.byref(s), _ptr(x), _ptr(w_router), _ptr(router_bias),
                                      _ptr(logits), _ptr(topk_ids), _ptr(topk_w), _ptr(ws), nbytes,
                                      _stream(stream)))


def permute(s, topk_ids, x, counts, offsets, sorted_ids, inv, x_perm, ws, stream=None):
    lib = load()
    nbytes = ws.numel() * ws.element_size() if ws is not None else 0
    _check("moe_permute", lib.moe_permute(ctypes.byref(s), _ptr(topk_ids), _ptr(x), _ptr(counts),
                                          _ptr(offsets), _ptr(sorted_ids), _ptr(inv), _ptr(x_perm),
                                          _ptr(ws), nbytes, _stream(stream)))


def gemm_gateup(s, x, sorted_ids, offsets, w_gate_up, gu_scales, h, stream=None):
    lib = load()
    _check("moe_grouped_gemm_gateup",
           lib.moe_grouped_gemm_gateup(ctypes.byref(s), _ptr(x), _ptr(sorted_ids), _ptr(offsets),
                                       _ptr(w_gate_up), _ptr(gu_scales), _ptr(h), _stream(stream)))


def gemm_down(s, h, offsets, w_down, d_scales, y, stream=None):
    lib = load()
    _check("moe_grouped_gemm_down",
           lib.moe_grouped_gemm_down(ctypes.byref(s), _ptr(h), _ptr(offsets), _ptr(w_down),
                                     _ptr(d_scales), _ptr(y), _stream(stream)))


def combine(s, y, inv, topk_w, out, stream=None):
    lib = load()
    _check("moe_combine", lib.moe_combine(ctypes.byref(s), _ptr(y), _ptr(inv), _ptr(topk_w),
                                          _ptr(out), _stream(stream)))


def forward(s, x, w_router, router_bias, w_gate_up, gu_scales, w_down, d_scales, out,
            topk_ids_out=None, topk_w_out=None, ws=None, stream=None, stage_events=None):
    """stage_events: None or a ctypes array of MOE_FORWARD_STAGES + 1 hipEvent_t handles."""
    lib = load()
    nbytes = ws.numel() * ws.element_size() if ws is not None else 0
    ev = ctypes.cast(stage_events, _P) if stage_events is not None else None
    _check("moe_forward",
           lib.moe_forward(ctypes.byref(s), _ptr(x), _ptr(w_router), _ptr(router_bias), _ptr(w_gate_up),
                           _ptr(gu_scales), _ptr(w_down), _ptr(d_scales), _ptr(out), _ptr(topk_ids_out),
                           _ptr(topk_w_out), _ptr(ws), nbytes, _stream(stream), ev))


def forward_noalloc(s, x, w_router, router_bias, w_gate_up, gu_scales, w_down, d_scales, out,
                    topk_ids_out=None, topk_w_out=None, stream=None):
    """moe_forward_noalloc: moe_forward on the library's own per-GPU scratch
    (no workspace argument; calls on one GPU must not overlap)."""
    lib = load()
    _check("moe_forward_noalloc",
           lib.moe_forward_noalloc(ctypes.byref(s), _ptr(x), _ptr(w_router), _ptr(router_bias), _ptr(w_gate_up),
                                   _ptr(gu_scales), _ptr(w_down), _ptr(d_scales), _ptr(out), _ptr(topk_ids_out),
                                   _ptr(topk_w_out), _stream(stream)))


def forward_shared(s, x, w_router, router_bias, w_gate_up, gu_scales, w_down, d_scales, I_sh, w_sh_gate_up,
                   sh_gu_scales, w_sh_down, sh_d_scales, out, topk_ids_out=None, topk_w_out=None, ws=None,
                   stream=None, stage_events=None):
    """moe_forward_shared: the layer plus a dense GEGLU MLP (intermediate I_sh) on every token."""
    lib = load()
    nbytes = ws.numel() * ws.element_size() if ws is not None else 0
    ev = ctypes.cast(stage_events, _P) if stage_events is not None else None
    _check("moe_forward_shared",
           lib.moe_forward_shared(ctypes.byref(s), _ptr(x), _ptr(w_router), _ptr(router_bias), _ptr(w_gate_up),
                                  _ptr(gu_scales), _ptr(w_down), _ptr(d_scales), I_sh, _ptr(w_sh_gate_up),
                                  _ptr(sh_gu_scales), _ptr(w_sh_down), _ptr(sh_d_scales), _ptr(out),
                                  _ptr(topk_ids_out), _ptr(topk_w_out), _ptr(ws), nbytes, _stream(stream), ev))


def quantize_nv(src, input_scale, codes, scales, stream=None):
    """moe_quantize_nv: NVFP4 codes [rows][K/2] and E4M3 scales [rows][K/16]
    of bf16 rows src [rows][K] relative to input_scale (a one-element fp32
    device tensor)."""
    lib = load()
    rows, K = src.shape
    _check("moe_quantize_nv", lib.moe_quantize_nv(_ptr(src), rows, K, _ptr(input_scale), _ptr(codes),
                                                  _ptr(scales), _stream(stream)))


def quantize_mx(src, codes, scales, stream=None):
    """moe_quantize_mx: MXFP4 codes [rows][K/2] and scales [rows][K/32] of bf16 rows src [rows][K]."""
    lib = load()
    rows, K = src.shape
    _check("moe_quantize_mx", lib.moe_quantize_mx(_ptr(src), rows, K, _ptr(codes), _ptr(scales), _stream(stream)))
