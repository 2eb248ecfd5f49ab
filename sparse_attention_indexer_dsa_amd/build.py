"""Build libdsaidx.so (the HIP kernels and the C ABI) in-tree for gfx950.

Each source is compiled to its own object in parallel (every kernel is
launched from the file that defines it, so no relocatable device code is
needed), then the objects are linked into the shared library.
"""
from __future__ import annotations

import os
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libdsaidx.so")
SOURCES = ["api.cpp", "scan_topk.hip", "dense_topk.hip", "decode.hip", "group_pool.hip", "mtp.hip", "calib.hip",
           "group_query.hip", "probe.hip", "noalloc.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
INCLUDE = os.path.join(os.path.dirname(HERE), "include")

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    # no packed-fp32 instructions anywhere in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def _clean(text: str) -> str:
    return "\n".join(l for l in text.splitlines() if "packed-fp32-ops" not in l and l.strip())


def _run(cmd):
    res = subprocess.run(cmd, cwd=CSRC, capture_output=True, text=True)
    return res.returncode, _clean(res.stdout + res.stderr)


def build(verbose: bool = False) -> str:
    """Compile every HIP source into libdsaidx.so (always recompiles)."""
    srcs = [s for s in SOURCES if os.path.exists(os.path.join(CSRC, s))]
    jobs = min(len(srcs), max(1, min(16, os.cpu_count() or 1)))
    with tempfile.TemporaryDirectory(prefix="dsaidx_build_") as tmpdir:
        objs = [os.path.join(tmpdir, os.path.splitext(s)[0] + ".o") for s in srcs]
        cmds = [[HIPCC, *FLAGS, "-I", INCLUDE, "-c", "-o", o, os.path.join(CSRC, s)] for s, o in zip(srcs, objs)]
        if verbose:
            for c in cmds:
                print(" ".join(c), flush=True)
        with ThreadPoolExecutor(jobs) as ex:
            results = list(ex.map(_run, cmds))
        for (rc, out), s in zip(results, srcs):
            if rc != 0:
                raise RuntimeError(f"hipcc failed on {s} ({rc}):\n{out}")
            if verbose and out:
                print(out, flush=True)
        tmp = LIB + ".tmp"
        link = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
        rc, out = _run(link)
        if rc != 0:
            raise RuntimeError(f"link failed ({rc}):\n{out}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    print(LIB)
    sys.exit(0)
