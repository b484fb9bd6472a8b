"""Compile the HIP library libfrhip.so in-tree for gfx950.

    python memory_bound_amd/build.py

(run by path: importing the package loads the library being rebuilt)
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libfrhip.so")
SOURCES = ["fr_api.hip", "fr_norm.hip", "fr_qkv.hip", "fr_act.hip", "fr_gemm.hip",
           "fr_chain.hip", "fr_qknorm.hip"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-fvisibility=hidden",
    # keep the compiler from forming packed fp32 (v_pk_*_f32) instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # matrix-core results in ordinary VGPRs: the GEMM's per-block scale fold
    # then reads them without accumulator-register copies
    "-mllvm", "-amdgpu-mfma-vgpr-form=1",
    "-Wall", "-Wno-unused-result",
]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{err}")
    if err.strip() and verbose:
        print(err, file=sys.stderr)


def build(verbose=False):
    """Compile every source to an object in parallel (one hipcc per file),
    then link the shared library; the objects go to _build/ (not tracked)."""
    from concurrent.futures import ThreadPoolExecutor
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    obj_dir = os.path.join(HERE, "_build")
    os.makedirs(obj_dir, exist_ok=True)
    compile_flags = [f for f in HIPCC_FLAGS if f != "-shared"]
    objs = [os.path.join(obj_dir, s.replace(".hip", ".o")) for s in SOURCES]
    cmds = [[hipcc, *compile_flags, "-c", "-I", os.path.join(ROOT, "include"), "-I", CSRC,
             os.path.join(CSRC, s), "-o", o] for s, o in zip(SOURCES, objs)]
    jobs = max(1, min(len(cmds), os.cpu_count() or 1, 16))
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        for f in [ex.submit(_run, c, verbose) for c in cmds]:
            f.result()
    tmp = LIB + ".tmp"
    _run([hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp], verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
