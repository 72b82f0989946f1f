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

# -packed-fp32-ops: no v_pk_{add,mul,fma}_f32 (packed fp32 forms are kept out of the code).
# Correctly rounded f32 division is required by the q8_1 scale (d = amax / 127, 1/d).
HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fhip-fp32-correctly-rounded-divide-sqrt", "-fno-fast-math",
    "-Wno-unused-command-line-argument",
    # keep MFMA results in arch VGPRs: the fold reads every accumulator with VALU ops
    "-mllvm", "-amdgpu-mfma-vgpr-form",
]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def _compile(sources: list[str], out: str, extra: list[str] | None, verbose: bool) -> str:
    cmd = [hipcc(), *HIPCC_FLAGS, *(extra or []), "-o", out + ".tmp", *sources]
    res = subprocess.run(cmd, capture_output=True, text=True)
    msgs = [l for l in (res.stdout + res.stderr).splitlines() if "packed-fp32-ops" not in l]
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs), file=sys.stderr)
    os.replace(out + ".tmp", out)
    return out


def build(extra: list[str] | None = None, out: str = LIB, verbose: bool = False) -> str:
    _compile(SOURCES, out, extra, verbose)
    if out == LIB:
        _compile(CALIB_SOURCES, CALIB_LIB, extra, verbose)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
