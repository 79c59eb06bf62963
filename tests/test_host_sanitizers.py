"""Host ASan + UBSan and bounds-assert build of the C ABI, exercised on the
CPU.

`delta_rule_recurrence_amd.build.build_sanitized()` compiles the host code
with AddressSanitizer and UndefinedBehaviorSanitizer (every finding fatal)
and with the launchers' host-side bounds model (FALCON_BOUNDS_CHECK): before
a fast kernel is launched, its grid decomposition, workspace layout and every
workgroup's workspace, flag and output ranges are checked against the
buffers.  A child process with the ASan runtime preloaded and no visible
device then drives every entry point on fake device addresses
(tests/host_abi_driver.py): thousands of shapes, variants, chunk sizes,
dtypes and optional-argument combinations, the noalloc grouping, decode, the
backward, and invalid arguments.  Launches fail for want of a device; every
host-side step before them runs sanitised.  Never run where a GPU is present:
fake addresses must not reach a device."""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
from delta_rule_recurrence_amd import build as B  # noqa: E402


def _stale(lib):
    if not os.path.exists(lib):
        return True
    t = os.path.getmtime(lib)
    srcs = [os.path.join(B.CSRC, f) for f in os.listdir(B.CSRC)] + [os.path.join(B.INCLUDE, f)
                                                                  for f in os.listdir(B.INCLUDE)]
    return any(os.path.getmtime(s) > t for s in srcs)


@pytest.fixture(scope="module")
def san_lib():
    if os.path.exists("/dev/kfd"):
        pytest.skip("a GPU is present: the fake-address driver runs on CPU-only machines")
    lib = B.LIB_SAN
    if _stale(lib):
        B.build_sanitized(verbose=False)
    return lib


def test_sanitized_build_is_instrumented(san_lib):
    syms = subprocess.run(["nm", "-D", san_lib], capture_output=True, text=True, check=True).stdout
    assert "__asan_report_load" in syms, "no AddressSanitizer instrumentation"
    assert "__ubsan_handle_" in syms, "no UndefinedBehaviorSanitizer instrumentation"
    syms_all = subprocess.run(["nm", "-C", san_lib], capture_output=True, text=True, check=True).stdout
    assert "falcon::host_check_failed" in syms_all, "bounds checks not compiled in"


def test_abi_under_host_sanitizers(san_lib):
    env = dict(os.environ)
    env.update(HIP_VISIBLE_DEVICES="", ROCR_VISIBLE_DEVICES="", CUDA_VISIBLE_DEVICES="",
               LD_PRELOAD=B.asan_runtime(), ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    res = subprocess.run([sys.executable, os.path.join(ROOT, "tests", "host_abi_driver.py"), san_lib],
                         env=env, capture_output=True, text=True, timeout=600)
    assert res.returncode == 0, f"driver failed ({res.returncode}):\n{res.stdout[-2000:]}\n{res.stderr[-6000:]}"
    assert "calls checked" in res.stdout
