"""Minimal HIP runtime plumbing through ctypes: stream capture into a graph,
graph replay, timing events (including event-record nodes inside a graph)
and cross-stream waits (a fork and join inside a capture).  No compute; used by the benchmark and the graph-replay test.
"""
from __future__ import annotations

import ctypes as C

_hip = C.CDLL("libamdhip64.so")
_vp = C.c_void_p

hipStreamCaptureModeRelaxed = 2
hipEventRecordExternal = 1

_hip.hipStreamBeginCapture.argtypes = [_vp, C.c_int]
_hip.hipStreamEndCapture.argtypes = [_vp, C.POINTER(_vp)]
_hip.hipGraphInstantiate.argtypes = [C.POINTER(_vp), _vp, _vp, _vp, C.c_size_t]
_hip.hipGraphLaunch.argtypes = [_vp, _vp]
_hip.hipGraphExecDestroy.argtypes = [_vp]
_hip.hipGraphDestroy.argtypes = [_vp]
_hip.hipEventCreate.argtypes = [C.POINTER(_vp)]
_hip.hipEventRecordWithFlags.argtypes = [_vp, _vp, C.c_uint]
_hip.hipEventRecord.argtypes = [_vp, _vp]
_hip.hipEventElapsedTime.argtypes = [C.POINTER(C.c_float), _vp, _vp]
_hip.hipEventDestroy.argtypes = [_vp]
_hip.hipEventSynchronize.argtypes = [_vp]
_hip.hipStreamSynchronize.argtypes = [_vp]
_hip.hipStreamWaitEvent.argtypes = [_vp, _vp, C.c_uint]
_hip.hipGetErrorString.argtypes = [C.c_int]
_hip.hipGetErrorString.restype = C.c_char_p


class HipError(RuntimeError):
    pass


def _ok(rc, what):
    if rc != 0:
        raise HipError(f"{what}: {_hip.hipGetErrorString(rc).decode()} ({rc})")


class Event:
    def __init__(self):
        self.h = _vp()
        _ok(_hip.hipEventCreate(C.byref(self.h)), "hipEventCreate")

    def record(self, stream: int, external: bool = False):
        if external:
            _ok(_hip.hipEventRecordWithFlags(self.h, _vp(stream), hipEventRecordExternal),
                "hipEventRecordWithFlags")
        else:
            _ok(_hip.hipEventRecord(self.h, _vp(stream)), "hipEventRecord")

    def synchronize(self):
        _ok(_hip.hipEventSynchronize(self.h), "hipEventSynchronize")

    def elapsed_ms(self, later: "Event") -> float:
        ms = C.c_float()
        _ok(_hip.hipEventElapsedTime(C.byref(ms), self.h, later.h), "hipEventElapsedTime")
        return ms.value

    def __del__(self):
        try:
            _hip.hipEventDestroy(self.h)
        except Exception:
            pass


class Graph:
    """Capture everything enqueued on `stream` inside the with-block."""

    def __init__(self, stream: int):
        self.stream = stream
        self.graph = _vp()
        self.exec = _vp()

    def __enter__(self):
        _ok(_hip.hipStreamBeginCapture(_vp(self.stream), hipStreamCaptureModeRelaxed),
            "hipStreamBeginCapture")
        return self

    def __exit__(self, et, ev, tb):
        rc = _hip.hipStreamEndCapture(_vp(self.stream), C.byref(self.graph))
        if et is None:
            _ok(rc, "hipStreamEndCapture")
            _ok(_hip.hipGraphInstantiate(C.byref(self.exec), self.graph, None, None, 0),
                "hipGraphInstantiate")
        return False

    def launch(self):
        _ok(_hip.hipGraphLaunch(self.exec, _vp(self.stream)), "hipGraphLaunch")

    def __del__(self):
        try:
            if self.exec:
                _hip.hipGraphExecDestroy(self.exec)
            if self.graph:
                _hip.hipGraphDestroy(self.graph)
        except Exception:
            pass


def stream_synchronize(stream: int):
    _ok(_hip.hipStreamSynchronize(_vp(stream)), "hipStreamSynchronize")


def stream_wait_event(stream: int, event: Event):
    """Work enqueued on `stream` after this waits for `event`'s last record."""
    _ok(_hip.hipStreamWaitEvent(_vp(stream), event.h, 0), "hipStreamWaitEvent")
