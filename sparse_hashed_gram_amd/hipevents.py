"""Minimal HIP event timing through the HIP runtime (ctypes).

torch.cuda.Event only sees work recorded through torch; these raw hipEvent_t
handles can be handed to libngram's profiling hook so that events are
recorded on the same stream right around one kernel group."""
from __future__ import annotations

import ctypes

_hip = None


def _rt():
    global _hip
    if _hip is None:
        h = ctypes.CDLL("libamdhip64.so")
        h.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        h.hipEventDestroy.argtypes = [ctypes.c_void_p]
        h.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        h.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        h.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                          ctypes.c_void_p]
        _hip = h
    return _hip


class Event:
    def __init__(self):
        self.h = ctypes.c_void_p()
        rc = _rt().hipEventCreate(ctypes.byref(self.h))
        if rc != 0:
            raise RuntimeError(f"hipEventCreate failed ({rc})")

    @property
    def handle(self) -> int:
        return self.h.value

    def record(self, stream: int):
        _rt().hipEventRecord(self.h, ctypes.c_void_p(stream))

    def synchronize(self):
        _rt().hipEventSynchronize(self.h)

    def elapsed_ms(self, later: "Event") -> float:
        ms = ctypes.c_float()
        rc = _rt().hipEventElapsedTime(ctypes.byref(ms), self.h, later.h)
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return float(ms.value)

    def __del__(self):
        try:
            if self.h.value:
                _rt().hipEventDestroy(self.h)
        except Exception:
            pass
