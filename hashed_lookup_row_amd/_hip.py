"""Raw HIP events and stream waits (ctypes over libamdhip64), for ordering work between streams.

Events are created without timing and without the system-scope fence: they order work between
streams of one GPU, for which the device-scope release and acquire of the packets suffice, and a
system-scope fence would write back the L2 caches at every record.  Timing events keep timing on.
"""
from __future__ import annotations

import ctypes

_DISABLE_TIMING = 0x2
_DISABLE_SYSTEM_FENCE = 0x20000000


class _Hip:
    def __init__(self):
        self.lib = ctypes.CDLL("libamdhip64.so")
        self.lib.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        self.lib.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.lib.hipStreamWaitEvent.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_uint]
        self.lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.lib.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.lib.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self.lib.hipMemcpyAsync.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int,
                                            ctypes.c_void_p]
        self.lib.hipStreamBeginCapture.argtypes = [ctypes.c_void_p, ctypes.c_int]
        self.lib.hipStreamEndCapture.argtypes = [ctypes.c_void_p, ctypes.POINTER(ctypes.c_void_p)]
        self.lib.hipGraphInstantiate.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_void_p, ctypes.c_void_p,
                                                 ctypes.c_char_p, ctypes.c_size_t]
        self.lib.hipGraphLaunch.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.lib.hipGraphExecDestroy.argtypes = [ctypes.c_void_p]
        self.lib.hipGraphDestroy.argtypes = [ctypes.c_void_p]

    def event(self, timing: bool = False) -> ctypes.c_void_p:
        e = ctypes.c_void_p()
        flags = _DISABLE_SYSTEM_FENCE | (0 if timing else _DISABLE_TIMING)
        rc = self.lib.hipEventCreateWithFlags(ctypes.byref(e), flags)
        if rc != 0:
            raise RuntimeError(f"hipEventCreateWithFlags failed ({rc})")
        return e

    def record(self, e, stream: int):
        rc = self.lib.hipEventRecord(e, ctypes.c_void_p(stream))
        if rc != 0:
            raise RuntimeError(f"hipEventRecord failed ({rc})")

    def wait(self, stream: int, e):
        rc = self.lib.hipStreamWaitEvent(ctypes.c_void_p(stream), e, 0)
        if rc != 0:
            raise RuntimeError(f"hipStreamWaitEvent failed ({rc})")

    def copy_d2d(self, dst: int, src: int, nbytes: int, stream: int):
        rc = self.lib.hipMemcpyAsync(ctypes.c_void_p(dst), ctypes.c_void_p(src), nbytes, 3, ctypes.c_void_p(stream))
        if rc != 0:
            raise RuntimeError(f"hipMemcpyAsync failed ({rc})")

    # Stream capture into a HIP graph (relaxed mode: other threads may keep using the runtime).
    def begin_capture(self, stream: int):
        rc = self.lib.hipStreamBeginCapture(ctypes.c_void_p(stream), 2)
        if rc != 0:
            raise RuntimeError(f"hipStreamBeginCapture failed ({rc})")

    def end_capture(self, stream: int) -> ctypes.c_void_p:
        g = ctypes.c_void_p()
        rc = self.lib.hipStreamEndCapture(ctypes.c_void_p(stream), ctypes.byref(g))
        if rc != 0:
            raise RuntimeError(f"hipStreamEndCapture failed ({rc})")
        return g

    def instantiate(self, graph) -> ctypes.c_void_p:
        x = ctypes.c_void_p()
        rc = self.lib.hipGraphInstantiate(ctypes.byref(x), graph, None, None, 0)
        if rc != 0:
            raise RuntimeError(f"hipGraphInstantiate failed ({rc})")
        return x

    def launch_graph(self, graph_exec, stream: int):
        rc = self.lib.hipGraphLaunch(graph_exec, ctypes.c_void_p(stream))
        if rc != 0:
            raise RuntimeError(f"hipGraphLaunch failed ({rc})")

    def destroy_graph(self, graph, graph_exec):
        if graph_exec:
            self.lib.hipGraphExecDestroy(graph_exec)
        if graph:
            self.lib.hipGraphDestroy(graph)

    def synchronize(self, e):
        rc = self.lib.hipEventSynchronize(e)
        if rc != 0:
            raise RuntimeError(f"hipEventSynchronize failed ({rc})")

    def elapsed_s(self, a, b) -> float:
        ms = ctypes.c_float()
        rc = self.lib.hipEventElapsedTime(ctypes.byref(ms), a, b)
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return ms.value * 1e-3


_hip = None


def hip() -> _Hip:
    global _hip
    if _hip is None:
        _hip = _Hip()
    return _hip
