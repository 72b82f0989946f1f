"""Host-side sanitizer builds (CPU only; no kernel is ever launched).

* The oracle (oracle/oracle.c) built with gcc -fsanitize=address,undefined and driven through
  every function on small seeded inputs and its argument rejections
  (tests/sanitize/oracle_driver.c).
* The host side of libqpg (the C ABI's validation and launch code, csrc/*.hip) and of
  libqpg_calib built with hipcc, address and undefined-behaviour sanitizers on the host pass
  only (the gfx950 device code is compiled as usual), driven through every entry point with
  arguments the validation must reject (tests/sanitize/abi_driver.cpp); on a machine without
  a GPU also with valid arguments, which must report QPG_EDEVICE.
A sanitizer finding aborts the driver with a report, which fails the test.
"""
import os
import shutil
import subprocess

import pytest

from quantized_prefill_gemm_amd import build as qbuild

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1", UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")


def _has_gpu():
    try:
        import torch
        return torch.cuda.device_count() > 0
    except Exception:
        return False


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_under_asan_ubsan(tmp_path):
    exe = tmp_path / "oracle_driver"
    subprocess.run(["gcc", "-std=c11", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=undefined", "-o", str(exe), os.path.join(HERE, "oracle_driver.c"),
                    os.path.join(ROOT, "oracle", "oracle.c"), "-lm", "-lpthread"], check=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, env=ENV, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "oracle driver: ok" in r.stdout


@pytest.mark.skipif(not os.path.exists(qbuild.hipcc()), reason="hipcc not available")
def test_c_abi_host_side_under_asan_ubsan(tmp_path):
    exe = tmp_path / "abi_driver"
    cmd = [qbuild.hipcc(), *qbuild.DEVICE_FLAGS, "-Wno-unused-command-line-argument",
           "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer", "-g",
           "-o", str(exe), *qbuild.SOURCES, *qbuild.CALIB_SOURCES, os.path.join(HERE, "abi_driver.cpp")]
    b = subprocess.run(cmd, capture_output=True, text=True)
    assert b.returncode == 0, b.stdout + b.stderr
    args = [] if _has_gpu() else ["nodevice"]
    r = subprocess.run([str(exe), *args], capture_output=True, text=True, env=ENV, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "abi driver: ok" in r.stdout
