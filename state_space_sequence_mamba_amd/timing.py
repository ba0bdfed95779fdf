"""Raw HIP event handles for the library's per-kernel timing entry point.

The handles are created with the HIP runtime that torch already loaded (same library,
looked up by its soname) and passed to the *_ex entry points.  Measurement plumbing only: nothing
here takes part in the scan.
"""
import ctypes

import torch


class HipEvents:
    def __init__(self):
        h = ctypes.CDLL("libamdhip64.so.7")
        vp = ctypes.c_void_p
        h.hipEventCreate.argtypes = [ctypes.POINTER(vp)]
        h.hipEventCreate.restype = ctypes.c_int
        h.hipEventDestroy.argtypes = [vp]
        h.hipEventDestroy.restype = ctypes.c_int
        h.hipEventRecordWithFlags.argtypes = [vp, vp, ctypes.c_uint]
        h.hipEventRecordWithFlags.restype = ctypes.c_int
        h.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), vp, vp]
        h.hipEventElapsedTime.restype = ctypes.c_int
        self.h = h
        self.events = []

    def create(self):
        ev = ctypes.c_void_p()
        if self.h.hipEventCreate(ctypes.byref(ev)) != 0:
            raise RuntimeError("hipEventCreate failed")
        self.events.append(ev.value)
        return ev.value

    def record(self, ev, stream=None):
        """Record on `stream` (default: torch's current stream)."""
        s = (stream or torch.cuda.current_stream()).cuda_stream
        if self.h.hipEventRecordWithFlags(ev, s, 0) != 0:
            raise RuntimeError("hipEventRecordWithFlags failed")

    def elapsed_ms(self, a, b):
        ms = ctypes.c_float()
        if self.h.hipEventElapsedTime(ctypes.byref(ms), a, b) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value

    def close(self):
        for ev in self.events:
            self.h.hipEventDestroy(ev)
        self.events = []
