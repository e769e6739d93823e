"""Build libtokenselect.so (HIP, gfx950) in the package directory.

Every kernel source under csrc/ is compiled by hipcc into one shared library
exporting the C ABI declared in include/tokenselect.h. Two measurement-only
libraries are built beside it: the streaming-bandwidth probe under csrc/probe/
(declared in csrc/probe/ts_stream_probe.h, outside the method's ABI directory
include/) into libts_stream_probe.so, and the same kernel sources with the per-wave
timeline of csrc/timeline.h compiled in (-DTS_TIMELINE) into
libtokenselect_timeline.so. The three compiles run in parallel.
"""
from __future__ import annotations

import glob
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
LIB = os.path.join(PKG, "libtokenselect.so")
PROBE_LIB = os.path.join(PKG, "libts_stream_probe.so")
TIMELINE_LIB = os.path.join(PKG, "libtokenselect_timeline.so")
ARCH = "gfx950"

# Packed fp32 VALU forms are turned off: the compiler would otherwise emit them
# from ordinary float code.
HIP_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (set HIPCC or install ROCm)")


def sources():
    return sorted(glob.glob(os.path.join(PKG, "csrc", "*.hip")))


def _start(out: str, srcs, verbose: bool, extra_inc=(), defines=()):
    tmp = out + ".tmp"
    inc = [os.path.join(ROOT, "include"), os.path.join(PKG, "csrc"), *extra_inc]
    cmd = [hipcc(), *HIP_FLAGS, *[f"-D{d}" for d in defines], *[a for d in inc for a in ("-I", d)],
           "-o", tmp, *srcs]
    if verbose:
        print(" ".join(cmd), flush=True)
    return out, tmp, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True)


def _finish(job, verbose: bool) -> str:
    out, tmp, proc = job
    _, stderr = proc.communicate()
    noise = "is not a recognized feature for this target"
    errs = "\n".join(l for l in stderr.splitlines() if noise not in l)
    if proc.returncode != 0:
        raise RuntimeError(f"hipcc failed for {os.path.basename(out)} ({proc.returncode}):\n{errs}")
    if verbose and errs.strip():
        print(errs, file=sys.stderr)
    os.replace(tmp, out)
    return out


def build(verbose: bool = False) -> str:
    """Compile every HIP source into libtokenselect.so (and the bandwidth probe into
    libts_stream_probe.so, the timeline build into libtokenselect_timeline.so);
    returns the main library path."""
    probe = os.path.join(PKG, "csrc", "probe")
    jobs = [_start(LIB, sources(), verbose),
            _start(PROBE_LIB, sorted(glob.glob(os.path.join(probe, "*.hip"))), verbose, extra_inc=(probe,)),
            _start(TIMELINE_LIB, sources(), verbose, defines=("TS_TIMELINE",))]
    for job in jobs:
        _finish(job, verbose)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
