"""Build libdsq.so (gfx950 only) in-tree with hipcc.

    python -m group_quantized_moe_dsq_amd.build

Every source compiles to its own object (in parallel) under _build/, then one
link step makes the shared library.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OBJ = os.path.join(os.path.dirname(HERE), "_build")
LIB = os.path.join(HERE, "libdsq.so")
SOURCES = ["api.hip", "pack.hip", "gemv.hip", "gemv_sb4.hip", "decode.hip", "route.hip",
           "gemm_mfma.hip", "gmm.hip", "head.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    # IEEE fp32 division and sqrt: the quantizer's codes depend on it
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-fno-fast-math",
    # no packed fp32 instructions anywhere in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
]
LINK = [
    "--offload-arch=gfx950",
    "-shared",
    # every symbol must resolve at link time: a kernel whose host stub was not
    # emitted fails the build here instead of at load time
    "-Wl,-z,defs",
]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("hipcc failed: " + " ".join(cmd[-3:]))
    return r


def build(verbose: bool = False, extra=(), out: str = None, objdir: str = None,
          csrc: str = None) -> str:
    """Compile every source and link the library (to `out`, default the
    in-tree libdsq.so); `extra` adds compiler flags (e.g. -D overrides of
    the launch-shape macros)."""
    obj = objdir or OBJ
    os.makedirs(obj, exist_ok=True)
    objs = [os.path.join(obj, os.path.splitext(s)[0] + ".o") for s in SOURCES]
    src = csrc or CSRC
    cmds = [[HIPCC, *FLAGS, *extra, "-c", os.path.join(src, s), "-o", o]
            for s, o in zip(SOURCES, objs)]
    workers = max(1, min(len(cmds), os.cpu_count() or 1, 16))
    with cf.ThreadPoolExecutor(workers) as ex:
        for f in [ex.submit(_run, c, verbose) for c in cmds]:
            f.result()
    dst = out or LIB
    tmp = dst + ".tmp"
    _run([HIPCC, *LINK, *objs, "-o", tmp], verbose)
    os.replace(tmp, dst)
    return dst


if __name__ == "__main__":
    print(build(verbose=True))
