"""Minimal HIP graph plumbing (ctypes on the process's HIP runtime): capture
the launches a Python callable enqueues on one stream, instantiate, count the
kernel nodes, and replay.  Used to run the chained per-layer launch sequence
as one graph launch."""
import ctypes

import memory_bound_amd as fr

_hip = ctypes.CDLL(fr.hip_runtimes()[0])

_P = ctypes.c_void_p
_hip.hipStreamBeginCapture.argtypes = [_P, ctypes.c_int]
_hip.hipStreamEndCapture.argtypes = [_P, ctypes.POINTER(_P)]
_hip.hipGraphInstantiate.argtypes = [ctypes.POINTER(_P), _P, _P, _P, ctypes.c_size_t]
_hip.hipGraphLaunch.argtypes = [_P, _P]
_hip.hipGraphGetNodes.argtypes = [_P, _P, ctypes.POINTER(ctypes.c_size_t)]
_hip.hipGraphNodeGetType.argtypes = [_P, ctypes.POINTER(ctypes.c_int)]
_hip.hipGraphExecDestroy.argtypes = [_P]
_hip.hipGraphDestroy.argtypes = [_P]
for _f in ("hipStreamBeginCapture", "hipStreamEndCapture", "hipGraphInstantiate",
           "hipGraphLaunch", "hipGraphGetNodes", "hipGraphNodeGetType",
           "hipGraphExecDestroy", "hipGraphDestroy"):
    getattr(_hip, _f).restype = ctypes.c_int

CAPTURE_MODE_RELAXED = 2
NODE_TYPE_KERNEL = 0


def _ok(err, what):
    if err != 0:
        raise RuntimeError(f"{what} failed with hipError {err}")


class HipGraph:
    """Capture `fn()` (which must enqueue work only on `stream`) into a graph."""

    def __init__(self, stream, fn):
        self.stream = stream
        h = _P(stream.cuda_stream)
        _ok(_hip.hipStreamBeginCapture(h, CAPTURE_MODE_RELAXED), "hipStreamBeginCapture")
        graph = _P()
        try:
            fn()
        except BaseException:
            # end the capture so the stream is usable again, drop the partial
            # graph, and let the callable's own error through
            _hip.hipStreamEndCapture(h, ctypes.byref(graph))
            if graph:
                _hip.hipGraphDestroy(graph)
            raise
        _ok(_hip.hipStreamEndCapture(h, ctypes.byref(graph)), "hipStreamEndCapture")
        self.graph = graph
        self.exec = _P()
        _ok(_hip.hipGraphInstantiate(ctypes.byref(self.exec), graph, None, None, 0),
            "hipGraphInstantiate")

    def nodes(self):
        n = ctypes.c_size_t(0)
        _ok(_hip.hipGraphGetNodes(self.graph, None, ctypes.byref(n)), "hipGraphGetNodes")
        arr = (_P * n.value)()
        _ok(_hip.hipGraphGetNodes(self.graph, arr, ctypes.byref(n)), "hipGraphGetNodes")
        return list(arr)

    def kernel_node_count(self):
        count = 0
        for node in self.nodes():
            t = ctypes.c_int(-1)
            _ok(_hip.hipGraphNodeGetType(node, ctypes.byref(t)), "hipGraphNodeGetType")
            count += t.value == NODE_TYPE_KERNEL
        return count

    def launch(self):
        _ok(_hip.hipGraphLaunch(self.exec, _P(self.stream.cuda_stream)), "hipGraphLaunch")

    def __del__(self):
        try:
            if getattr(self, "exec", None):
                _hip.hipGraphExecDestroy(self.exec)
            if getattr(self, "graph", None):
                _hip.hipGraphDestroy(self.graph)
        except Exception:
            pass
