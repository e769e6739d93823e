"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

Builds every HIP source with the sanitizers on the host side only (the gfx950 device
code is built as usual and never runs here), links the C driver tests/abi_host_check.c
against it, and runs the driver on this machine, which needs no GPU: every call in the
driver fails validation before any launch. The sanitizers watch the workspace size
arithmetic over extreme shapes, the argument checks and the error formatting of every
entry point. Skipped where hipcc or gcc is missing.
"""
import os
import shutil
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "token_level_sparse_amd", "csrc")
HIPCC = "/opt/rocm/bin/hipcc"


def _run(cmd, **kw):
    res = subprocess.run(cmd, capture_output=True, text=True, **kw)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
    return res.returncode, res.stdout, err


@pytest.mark.timeout(600)
def test_abi_host_code_under_asan_and_ubsan():
    if not os.path.exists(HIPCC) or shutil.which("gcc") is None:
        pytest.skip("hipcc or gcc not available")
    srcs = sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]
    with tempfile.TemporaryDirectory() as tmp:
        rc, _, err = _run([HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17",
                           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", *san,
                           "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-c", *srcs], cwd=tmp)
        assert rc == 0, err
        drv = os.path.join(tmp, "abi_host_check.o")
        rc, _, err = _run(["gcc", "-c", "-g", "-Wall", "-Werror", "-D__HIP_PLATFORM_AMD__",
                           "-I", os.path.join(ROOT, "include"), "-I", "/opt/rocm/include",
                           os.path.join(ROOT, "tests", "abi_host_check.c"), "-o", drv])
        assert rc == 0, err
        objs = sorted(os.path.join(tmp, f) for f in os.listdir(tmp) if f.endswith(".o"))
        exe = os.path.join(tmp, "abi_host_check")
        rc, _, err = _run([HIPCC, "--offload-arch=gfx950", *san[:4], *objs, "-o", exe])
        assert rc == 0, err
        env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=0",
                   UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
        rc, out, err = _run([exe], env=env, timeout=300)
    assert "AddressSanitizer" not in err and "runtime error" not in err, err[-4000:]
    assert rc == 0, out[-4000:] + err[-2000:]
    assert out.strip().endswith("0 failures"), out[-2000:]
