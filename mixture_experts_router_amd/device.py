"""Device plumbing around the C ABI: uploading host arrays into torch device
tensors, workspace allocation and HIP events for stage timing.  No layer
arithmetic happens here."""
from __future__ import annotations

import ctypes

import numpy as np

from . import _lib


def to_device(a: np.ndarray, device="cuda"):
    """Copy a host array to the device: uint16 bf16 bits become a bfloat16
    tensor, other dtypes keep theirs."""
    import torch
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(a).to(device)


def bf16_bits(t) -> np.ndarray:
    """uint16 bit patterns of a bfloat16 device tensor, on the host."""
    import torch
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def workspace(s, device="cuda", I_sh: int = 0):
    """moe_forward (I_sh = 0) or moe_forward_shared workspace, zero-filled:
    its leading MOE_WS_ZERO_BYTES hold completion counters that must start at
    zero (each call leaves them zero)."""
    import torch
    n = _lib.workspace_shared_bytes(s, I_sh) if I_sh else _lib.workspace_bytes(s)
    return torch.zeros(n, dtype=torch.uint8, device=device)


_hip = None


def _hiprt():
    """The HIP runtime already loaded by torch (same soname)."""
    global _hip
    if _hip is None:
        import torch  # noqa: F401
        _hip = ctypes.CDLL("libamdhip64.so.7")
        _hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        _hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        _hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        _hip.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        _hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
    return _hip


class StageEvents:
    """MOE_FORWARD_STAGES + 1 hipEvents per call, for `n_calls` calls, that
    moe_forward records on its stream between its stages."""

    def __init__(self, n_calls: int):
        hip = _hiprt()
        n = _lib.MOE_FORWARD_STAGES + 1
        self.arrays = []
        for _ in range(n_calls):
            arr = (ctypes.c_void_p * n)()
            for i in range(n):
                ev = ctypes.c_void_p()
                if hip.hipEventCreate(ctypes.byref(ev)) != 0:
                    raise RuntimeError("hipEventCreate failed")
                arr[i] = ev
            self.arrays.append(arr)

    def stage_ms(self, call: int):
        """Per-stage milliseconds of one call (after the stream is synchronised)."""
        hip = _hiprt()
        arr = self.arrays[call]
        out = []
        for i in range(len(arr) - 1):
            ms = ctypes.c_float()
            if hip.hipEventElapsedTime(ctypes.byref(ms), arr[i], arr[i + 1]) != 0:
                raise RuntimeError("hipEventElapsedTime failed")
            out.append(ms.value)
        return out

    def close(self):
        hip = _hiprt()
        for arr in self.arrays:
            for ev in arr:
                hip.hipEventDestroy(ev)
        self.arrays = []
