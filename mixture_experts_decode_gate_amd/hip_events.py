"""hipEvent_t handles for timing work on a given stream (plain HIP runtime calls).

torch.cuda.Event only records on torch's current stream; these events are
recorded by libmoe itself (moe_forward_timed) or by the caller on any stream.
The HIP runtime used is the one torch loaded, found by its soname.
"""

from __future__ import annotations

import ctypes

_hip = None


def _rt():
    global _hip
    if _hip is None:
        import torch  # noqa: F401  (loads the HIP runtime)
        _hip = ctypes.CDLL("libamdhip64.so.7")
        _hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        _hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        _hip.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        _hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        _hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
    return _hip


class HipEvent:
    def __init__(self):
        h = ctypes.c_void_p()
        err = _rt().hipEventCreate(ctypes.byref(h))
        if err != 0:
            raise RuntimeError(f"hipEventCreate failed: {err}")
        self.handle = h.value

    def record(self, stream: int) -> None:
        err = _rt().hipEventRecord(self.handle, ctypes.c_void_p(int(stream)))
        if err != 0:
            raise RuntimeError(f"hipEventRecord failed: {err}")

    def synchronize(self) -> None:
        _rt().hipEventSynchronize(self.handle)

    def elapsed_ms(self, end: "HipEvent") -> float:
        ms = ctypes.c_float()
        err = _rt().hipEventElapsedTime(ctypes.byref(ms), self.handle, end.handle)
        if err != 0:
            raise RuntimeError(f"hipEventElapsedTime failed: {err}")
        return float(ms.value)

    def __del__(self):
        if _hip is not None and getattr(self, "handle", None):
            _hip.hipEventDestroy(self.handle)
            self.handle = None
