"""Build libs4dplr.so in-tree with hipcc for gfx950.

    python structured_state_space_dplr_amd/build.py

(run as a file so that the stale library is not loaded by the package import)
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libs4dplr.so")
SOURCES = ["kernels.hip", "big.hip", "recurrent.hip", "backward.hip", "vandermonde.hip", "block.hip",
           "noalloc.hip", "rank.hip", "api.cpp"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (looked in $HIPCC, /opt/rocm/bin, PATH)")


OBJDIR = os.path.join(PKG, "_build")


def flags() -> list[str]:
    return [
        f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
        "-Wall", "-Wno-unused-function",
        # packed fp32 VALU forms are kept out of the generated code
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I", os.path.join(ROOT, "include"), "-I", CSRC,
    ]


def command(out: str = LIB) -> list[str]:
    """The whole build as one hipcc command (same flags as ``build``)."""
    return [hipcc(), *flags(), "-shared", *[os.path.join(CSRC, s) for s in SOURCES], "-o", out]


def _run(cmd: list[str], verbose: bool) -> None:
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed with exit code {res.returncode}: {' '.join(cmd)}")
    if verbose:
        noisy = [l for l in (res.stdout + res.stderr).splitlines()
                 if "packed-fp32-ops" not in l]
        if noisy:
            print("\n".join(noisy))


def build(verbose: bool = False) -> str:
    """Compile every source to an object in parallel, then link the library."""
    os.makedirs(OBJDIR, exist_ok=True)
    cc = hipcc()
    objs = [os.path.join(OBJDIR, os.path.splitext(s)[0] + ".o") for s in SOURCES]
    jobs = [[cc, *flags(), "-c", os.path.join(CSRC, s), "-o", o] for s, o in zip(SOURCES, objs)]
    workers = max(1, min(len(jobs), int(os.environ.get("MAX_JOBS", os.cpu_count() or 1))))
    with ThreadPoolExecutor(workers) as ex:
        list(ex.map(lambda c: _run(c, verbose), jobs))
    tmp = LIB + ".tmp"
    _run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp], verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
