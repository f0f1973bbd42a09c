"""Builds libq4moe.so (gfx950) in-tree with hipcc.

Each source is compiled to its own object in parallel (a temporary directory), then
the objects are linked into the shared library.  No source calls a device function
of another, so no relocatable device code is needed.

Usage: ``python int4_group_quantized_g128_amd/build.py`` (by path, so that a stale
library is not loaded first) or ``__graft_entry__.build()``.
"""
import os
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libq4moe.so")
SOURCES = ["api.hip", "quantize.hip", "router.hip", "permute.hip", "gemm.hip", "gemm_prefill.hip", "lora.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wno-unused-function",
    # packed fp32 arithmetic off in device code (v_pk_* fp32 forms are avoided)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA results in VGPRs (the per-group scaling reads them with VALU right away)
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-fvisibility=hidden",
]


def _run(cmd):
    res = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in res.stderr.splitlines() if "packed-fp32-ops" not in l)
    return res.returncode, err


def build(verbose=False, jobs=None):
    jobs = jobs or min(len(SOURCES), max(1, len(os.sched_getaffinity(0))))
    with tempfile.TemporaryDirectory(prefix="q4moe_build_") as tmpdir:
        objs, cmds = [], []
        for s in SOURCES:
            obj = os.path.join(tmpdir, os.path.splitext(s)[0] + ".o")
            objs.append(obj)
            cmds.append([HIPCC] + FLAGS + ["-c", "-o", obj, os.path.join(CSRC, s)])
        if verbose:
            for c in cmds:
                print(" ".join(c), flush=True)
        with ThreadPoolExecutor(jobs) as ex:
            results = list(ex.map(_run, cmds))
        for (rc, err), s in zip(results, SOURCES):
            if rc != 0:
                raise RuntimeError(f"hipcc failed on {s} ({rc}):\n{err}")
            if verbose and err.strip():
                print(err, file=sys.stderr)
        tmp = LIB + ".tmp"
        link = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs
        if verbose:
            print(" ".join(link), flush=True)
        rc, err = _run(link)
        if rc != 0:
            raise RuntimeError(f"link failed ({rc}):\n{err}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
