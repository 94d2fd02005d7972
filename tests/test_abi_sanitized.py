"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

tests/abi_checks.cpp drives every host-side argument check of the C ABI
(the calls test_abi.py makes from Python, plus the no-allocation verify and
the decision kernels' shape checks); here it is linked with all library
sources, the host pass of each built with -fsanitize=address,undefined (the
device code is built as usual, without sanitizers), and run on the CPU: no
call reaches a device.  Any sanitizer report aborts the run.
"""

import glob
import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

from block_diffusion_speculative_kv_amd import build as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.slow
def test_abi_host_checks_under_sanitizers(tmp_path):
    hipcc = B.hipcc()
    if shutil.which(hipcc) is None and not os.path.exists(hipcc):
        pytest.skip("hipcc not available")
    exe = str(tmp_path / "abi_checks")
    srcs = [os.path.join(B.CSRC, s) for s in B.SOURCES] + [os.path.join(ROOT, "tests", "abi_checks.cpp")]
    flags = [f for f in B.FLAGS if f not in ("-shared", "-fPIC", "-O3")]
    san = ["-O1", "-g", "-fno-omit-frame-pointer",
           "-Xarch_host", "-fsanitize=address",
           "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all"]
    inc = ["-I", os.path.join(ROOT, "include")]

    def compile_one(src):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        r = subprocess.run([hipcc, *flags, *san, *inc, "-c", src, "-o", obj],
                           capture_output=True, text=True)
        return obj, r
    with ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        built = list(ex.map(compile_one, srcs))
    for obj, r in built:
        assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    res = subprocess.run([hipcc, *flags, *san, *[o for o, _ in built], "-o", exe],
                         capture_output=True, text=True)
    assert res.returncode == 0, res.stdout[-3000:] + res.stderr[-3000:]
    # the sanitizer runtimes are in the executable
    syms = subprocess.run(["nm", exe], capture_output=True, text=True).stdout
    assert "__asan_init" in syms and "__ubsan_handle" in syms
    env = dict(os.environ,
               ASAN_OPTIONS="detect_leaks=1:halt_on_error=1:abort_on_error=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1",
               HIP_VISIBLE_DEVICES="")
    run = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    out = run.stdout + run.stderr
    assert run.returncode == 0, out[-4000:]
    assert "all passed" in out
    assert "ERROR: AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
