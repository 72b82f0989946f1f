"""Build libqpg.so (all HIP sources of csrc/) and the measurement helper libqpg_calib.so
(csrc/calib/) for gfx950 with hipcc, in-tree."""
from __future__ import annotations

import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "libqpg.so")
SOURCES = sorted(glob.glob(os.path.join(HERE, "csrc", "*.hip")))
CALIB_LIB = os.path.join(HERE, "libqpg_calib.so")
CALIB_SOURCES = sorted(glob.glob(os.path.join(HERE, "csrc", "calib", "*.hip")))

# Device-code flags. "-target-feature -packed-fp32-ops" removes the packed f32 VALU forms
# (v_pk_add_f32 / v_pk_mul_f32 / v_pk_fma_f32) from the gfx950 code: without it hipcc -O3
# forms them from plain f32 code. The feature is a gfx950 one, so the x86 host pass of the
# same hipcc line reports it as unknown and ignores it; the device pass applies it, which
# tests/test_isa.py checks on the assembly of every source. Correctly rounded f32 division
# is required by the q8_1 scale (d = amax / 127, 1/d).
DEVICE_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fhip-fp32-correctly-rounded-divide-sqrt", "-fno-fast-math",
    # keep MFMA results in arch VGPRs: the fold reads every accumulator with VALU ops
    "-mllvm", "-amdgpu-mfma-vgpr-form",
]
HIPCC_FLAGS = DEVICE_FLAGS + ["-fPIC", "-shared", "-Wno-unused-command-line-argument"]

# The one line the host pass prints for the gfx950-only feature above (see DEVICE_FLAGS).
HOST_FEATURE_NOTE = "'-packed-fp32-ops' is not a recognized feature for this target"


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def _compile(sources: list[str], out: str, extra: list[str] | None, verbose: bool) -> str:
    cmd = [hipcc(), *HIPCC_FLAGS, *(extra or []), "-o", out + ".tmp", *sources]
    res = subprocess.run(cmd, capture_output=True, text=True)
    msgs = (res.stdout + res.stderr).splitlines()
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    if verbose and msgs:
        # every message is shown; the host pass's note on the gfx950 feature once per line
        # of output it produced, collapsed to a count
        host_notes = sum(HOST_FEATURE_NOTE in m for m in msgs)
        other = [m for m in msgs if HOST_FEATURE_NOTE not in m]
        if other:
            print("\n".join(other), file=sys.stderr)
        if host_notes:
            print(f"hipcc host pass: {host_notes} x \"{HOST_FEATURE_NOTE}\" (expected: the feature is "
                  f"applied to the gfx950 device code only)", file=sys.stderr)
    os.replace(out + ".tmp", out)
    return out


def device_asm(source: str, out: str) -> str:
    """gfx950 assembly of one source with the library's device flags (for ISA checks)."""
    cmd = [hipcc(), *DEVICE_FLAGS, "--cuda-device-only", "-S", "-Wno-unused-command-line-argument",
           "-o", out, source]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + res.stdout + res.stderr)
    return out


def build(extra: list[str] | None = None, out: str = LIB, verbose: bool = False) -> str:
    _compile(SOURCES, out, extra, verbose)
    if out == LIB:
        _compile(CALIB_SOURCES, CALIB_LIB, extra, verbose)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
