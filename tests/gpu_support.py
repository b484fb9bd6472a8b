"""Build and load the test and measurement support library
(tests/gpu_support.hip): the matrix-instruction probe the GEMM parity tests
use, and the plain streaming copy the benchmark reports as its achievable
reference.  Built by ``__graft_entry__.build()`` next to this file."""
import ctypes
import os
import subprocess

_HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(_HERE, "gpu_support.hip")
LIB = os.path.join(_HERE, "libfrsupport.so")


def build():
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    cmd = [hipcc, "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           SRC, "-o", LIB + ".tmp"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed:\n{res.stderr}")
    os.replace(LIB + ".tmp", LIB)
    return LIB


def load():
    import torch  # noqa: F401  (binds the probe to torch's HIP runtime)
    if not os.path.exists(LIB):
        raise ImportError(f"{LIB} is not built (run __graft_entry__.build())")
    lib = ctypes.CDLL(LIB)
    lib.mfma_probe_e4m3.argtypes = [ctypes.c_void_p] * 3 + [ctypes.c_int, ctypes.c_int,
                                                            ctypes.c_void_p]
    lib.mfma_probe_e4m3.restype = ctypes.c_int
    lib.stream_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_long, ctypes.c_int,
                                ctypes.c_void_p]
    lib.stream_copy.restype = ctypes.c_int
    return lib
