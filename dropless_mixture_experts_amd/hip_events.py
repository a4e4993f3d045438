"""Raw HIP events for per-kernel timing through the *_timed entry points.

torch's own events only time torch's streams from Python; these are plain
hipEvent_t handles that the library records on the stream it launches on.
"""
from __future__ import annotations

import ctypes
import ctypes.util

_hip = None


def _lib():
    global _hip
    if _hip is None:
        name = ctypes.util.find_library("amdhip64") or "libamdhip64.so"
        try:
            _hip = ctypes.CDLL(name)
        except OSError:
            _hip = ctypes.CDLL("/opt/rocm/lib/libamdhip64.so")
        _hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        _hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        _hip.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        _hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float),
                                             ctypes.c_void_p, ctypes.c_void_p]
        _hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
    return _hip


class EventArray:
    """n hipEvent_t handles, created on the current device.  only: if given,
    the indices that get an event; the other entries are NULL, and the
    library skips those records (so that timing one kernel costs two
    records, not one per kernel)."""

    def __init__(self, n: int, only=None):
        lib = _lib()
        self._arr = (ctypes.c_void_p * n)()
        for i in range(n):
            if only is not None and i not in only:
                continue
            h = ctypes.c_void_p()
            rc = lib.hipEventCreate(ctypes.byref(h))
            if rc != 0:
                raise RuntimeError(f"hipEventCreate failed ({rc})")
            self._arr[i] = h.value

    def __len__(self):
        return len(self._arr)

    def pointer(self):
        return ctypes.cast(self._arr, ctypes.c_void_p)

    def record(self, i: int, stream) -> None:
        """Record event i on a torch stream (hipEventRecord)."""
        rc = _lib().hipEventRecord(self._arr[i], ctypes.c_void_p(stream.cuda_stream))
        if rc != 0:
            raise RuntimeError(f"hipEventRecord failed ({rc})")

    def elapsed_ms(self, i: int, j: int) -> float:
        lib = _lib()
        out = ctypes.c_float()
        lib.hipEventSynchronize(self._arr[j])
        rc = lib.hipEventElapsedTime(ctypes.byref(out), self._arr[i], self._arr[j])
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return float(out.value)

    def close(self):
        lib = _lib()
        for i in range(len(self._arr)):
            if self._arr[i]:
                lib.hipEventDestroy(self._arr[i])
                self._arr[i] = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
