"""HIP events for ordering and timing work on the compute and copy streams.

Stream plumbing beside the C ABI: the events are created through the HIP
runtime that libra.so is linked against (the same runtime instance torch uses
in this process), with the system-scope fence turned off.  Both streams live
on one GPU, so the device-scope release/acquire that remains is what orders
the staging copy's writes before the step that reads them; the system-scope
fence would additionally write back and invalidate the caches for the host and
other devices, which costs several microseconds between every two launches.
"""
from __future__ import annotations

import ctypes

from . import _lib

_HIP_EVENT_DISABLE_TIMING = 0x2
_HIP_EVENT_DISABLE_SYSTEM_FENCE = 0x20000000

_hip = None


def _runtime() -> ctypes.CDLL:
    global _hip
    if _hip is None:
        h = _lib.lib()   # symbol lookup through libra.so reaches its HIP runtime
        vp = ctypes.c_void_p
        h.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(vp), ctypes.c_uint]
        h.hipEventRecord.argtypes = [vp, vp]
        h.hipStreamWaitEvent.argtypes = [vp, vp, ctypes.c_uint]
        h.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), vp, vp]
        h.hipEventSynchronize.argtypes = [vp]
        h.hipEventDestroy.argtypes = [vp]
        for f in ("hipEventCreateWithFlags", "hipEventRecord", "hipStreamWaitEvent",
                  "hipEventElapsedTime", "hipEventSynchronize", "hipEventDestroy"):
            getattr(h, f).restype = ctypes.c_int
        _hip = h
    return _hip


def _check(err: int, what: str) -> None:
    if err != 0:
        raise RuntimeError(f"{what} failed with HIP error {err}")


def _handle(stream) -> ctypes.c_void_p:
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else stream)


class Event:
    """A HIP event without the system-scope fence; `timing` enables timestamps."""

    def __init__(self, timing: bool = False):
        h = _runtime()
        self._ev = ctypes.c_void_p()
        flags = _HIP_EVENT_DISABLE_SYSTEM_FENCE | (0 if timing else _HIP_EVENT_DISABLE_TIMING)
        _check(h.hipEventCreateWithFlags(ctypes.byref(self._ev), flags), "hipEventCreateWithFlags")

    @property
    def handle(self) -> int:
        """The hipEvent_t, for the library's timed entry points."""
        return self._ev.value

    def record(self, stream) -> None:
        _check(_runtime().hipEventRecord(self._ev, _handle(stream)), "hipEventRecord")

    def wait(self, stream) -> None:
        """Make `stream` wait for the work this event was last recorded after."""
        _check(_runtime().hipStreamWaitEvent(_handle(stream), self._ev, 0), "hipStreamWaitEvent")

    def synchronize(self) -> None:
        _check(_runtime().hipEventSynchronize(self._ev), "hipEventSynchronize")

    def elapsed_time(self, end: "Event") -> float:
        """Milliseconds from this event to `end` (both timing events, both complete)."""
        ms = ctypes.c_float()
        _check(_runtime().hipEventElapsedTime(ctypes.byref(ms), self._ev, end._ev), "hipEventElapsedTime")
        return ms.value

    def __del__(self):
        if getattr(self, "_ev", None) and _hip is not None:
            _hip.hipEventDestroy(self._ev)
            self._ev = None
