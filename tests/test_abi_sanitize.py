"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

Builds the library with both sanitizers on its host code (the device code
is built as usual and never launched: the driver makes no HIP call), links
it with tests/abi_host_sanitize.c and runs the driver: argument validation, size arithmetic and T = 0 of every entry
point.  Any sanitizer report aborts the driver.  CPU only.
"""
import importlib
import os
import subprocess

import pytest

# the module (the package also exports a function named build)
B = importlib.import_module("sparse_moe_transformer_sigmoid_amd.build")

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
DRIVER = os.path.join(ROOT, "tests", "abi_host_sanitize.c")
# host-side sanitizers only (each flag applies to the host compilation)
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]


def _hipcc():
    try:
        return B.hipcc()
    except RuntimeError:
        return None


@pytest.mark.skipif(_hipcc() is None, reason="hipcc not available")
def test_abi_host_paths_under_sanitizers(tmp_path):
    cc = _hipcc()
    procs, objs = [], []
    for src in B.SOURCES:
        obj = str(tmp_path / src.replace(".hip", ".o"))
        cmd = [cc, *B.compile_flags(), "-O1", "-g", *SAN,
               "-c", os.path.join(B.CSRC, src), "-o", obj]
        procs.append((subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE,
                                       text=True), src))
        objs.append(obj)
    for p, src in procs:
        _, err = p.communicate()
        assert p.returncode == 0, f"{src}: {err[-2000:]}"
    drv = str(tmp_path / "driver.o")
    r = subprocess.run([cc, "-O1", "-g", *SAN, "-I", B.INCLUDE, "-c", DRIVER, "-o", drv],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    exe = str(tmp_path / "abi_host_sanitize")
    r = subprocess.run([cc, *SAN, drv, *objs, "-o", exe], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, (r.stdout + r.stderr)[-4000:]
    assert r.stdout.startswith("ok "), r.stdout
