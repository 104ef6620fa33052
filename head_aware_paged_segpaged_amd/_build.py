"""Compiles libsegpaged.so for gfx950 with hipcc (in-tree, next to this file)."""

from __future__ import annotations

import os
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libsegpaged.so")
# (source, extra flags). The kernels never produce or test NaNs, so they are compiled without
# NaN semantics: max/min then map to plain v_max/v_max3 without canonicalising every input.
SOURCES = [("api.cpp", []), ("planner.cpp", []), ("kernels.hip", ["-fno-honor-nans"])]

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    # Packed fp32 VALU forms stay off; the compiler would otherwise emit them from scalar code.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-mcode-object-version=5",
    "-Wno-unused-command-line-argument",
]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    path = os.path.join(rocm, "bin", "hipcc")
    return path if os.path.exists(path) else "hipcc"


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(line for line in res.stderr.splitlines() if noise not in line)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed (%d):\n%s" % (res.returncode, err))
    if verbose and err.strip():
        print(err, file=sys.stderr)


def build(verbose: bool = False) -> str:
    """Compile every source and link libsegpaged.so; returns the library path."""
    with tempfile.TemporaryDirectory(prefix="segpaged_build_") as tmpdir:
        objs = []
        procs = []
        for src, extra in SOURCES:
            obj = os.path.join(tmpdir, src + ".o")
            cmd = [hipcc(), *HIPCC_FLAGS, *extra, "-I", INCLUDE, "-I", CSRC, "-c",
                   os.path.join(CSRC, src), "-o", obj]
            if verbose:
                print(" ".join(cmd), flush=True)
            procs.append((cmd, subprocess.Popen(cmd, stdout=subprocess.PIPE,
                                                stderr=subprocess.PIPE, text=True)))
            objs.append(obj)
        for cmd, proc in procs:
            _, err = proc.communicate()
            noise = "is not a recognized feature for this target"
            err = "\n".join(line for line in err.splitlines() if noise not in line)
            if proc.returncode != 0:
                raise RuntimeError("hipcc failed (%d): %s\n%s"
                                   % (proc.returncode, " ".join(cmd), err))
            if verbose and err.strip():
                print(err, file=sys.stderr)
        tmp = LIB + ".tmp%d" % os.getpid()
        _run([hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", "-pthread", *objs, "-o", tmp],
             verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
