"""ISA census of our own gfx950 build (CPU only: hipcc cross-compiles to assembly here).

* No packed f32 VALU forms (v_pk_add_f32 / v_pk_mul_f32 / v_pk_fma_f32) anywhere in the
  library's device code. The build excludes them with a target feature that only the
  device pass knows (the host pass prints a harmless note); a positive control shows that
  the same flags remove them from code where hipcc -O3 would otherwise form them.
* The production instantiations of the MMQ kernels keep everything in registers (no
  scratch), at the occupancy their launch bounds ask for.
"""
import os
import re
import shutil
import subprocess

import pytest

from quantized_prefill_gemm_amd import build as qbuild

PACKED_F32 = re.compile(r"\bv_pk_(add|mul|fma)_f32\b")

pytestmark = pytest.mark.skipif(shutil.which(qbuild.hipcc()) is None and not os.path.exists(qbuild.hipcc()),
                                reason="hipcc not available")


@pytest.fixture(scope="module")
def asm_texts(tmp_path_factory):
    d = tmp_path_factory.mktemp("asm")
    out = {}
    for src in qbuild.SOURCES + qbuild.CALIB_SOURCES:
        name = os.path.basename(src)
        out[name] = open(qbuild.device_asm(src, str(d / (name + ".s")))).read()
    return out


def test_no_packed_f32_in_device_code(asm_texts):
    bad = {name: sorted(set(m.group(0) for m in PACKED_F32.finditer(t))) for name, t in asm_texts.items()}
    bad = {k: v for k, v in bad.items() if v}
    assert not bad, f"packed f32 VALU forms in the gfx950 code: {bad}"


def test_packed_f32_flag_is_what_removes_them(tmp_path):
    """Positive control: float2 multiply-adds that hipcc -O3 turns into v_pk_fma_f32 without
    the feature flag, and into none with the library's device flags."""
    src = tmp_path / "pk.hip"
    src.write_text(
        "#include <hip/hip_runtime.h>\n"
        "typedef float f2 __attribute__((ext_vector_type(2)));\n"
        "__global__ void k(f2* a, const f2* b, const f2* c) {\n"
        "  int i = threadIdx.x; f2 x = a[i];\n"
        "  for (int t = 0; t < 8; ++t) x = x * b[i + t] + c[i + t];\n"
        "  a[i] = x; }\n")
    without = [f for f in qbuild.DEVICE_FLAGS]
    j = without.index("-packed-fp32-ops")
    del without[j - 3:j + 1]                      # drop "-Xclang -target-feature -Xclang -packed-fp32-ops"
    assert "-packed-fp32-ops" not in without and len(without) == len(qbuild.DEVICE_FLAGS) - 4
    outs = {}
    for tag, flags in (("without", without), ("with", qbuild.DEVICE_FLAGS)):
        o = tmp_path / f"pk_{tag}.s"
        subprocess.run([qbuild.hipcc(), *flags, "--cuda-device-only", "-S", "-Wno-unused-command-line-argument",
                        "-o", str(o), str(src)], check=True, capture_output=True)
        outs[tag] = len(PACKED_F32.findall(o.read_text()))
    assert outs["without"] > 0, "control did not produce packed forms: the check would be vacuous"
    assert outs["with"] == 0


def _kernel_meta(text: str):
    """(kernel symbol -> (private segment bytes, vgpr count)) from the amdhsa directives."""
    meta = {}
    for m in re.finditer(r"\.amdhsa_kernel (\S+)(.*?)\.end_amdhsa_kernel", text, re.S):
        body = m.group(2)
        priv = int(re.search(r"\.amdhsa_private_segment_fixed_size (\d+)", body).group(1))
        vg = int(re.search(r"\.amdhsa_next_free_vgpr (\d+)", body).group(1))
        meta[m.group(1)] = (priv, vg)
    return meta


# production instantiations (fold, not the integer-sum witness): symbol prefix -> source
PRODUCTION = {
    "mmq_q4k.hip": [r"mmq_q4K_kernelILb0E"],
    "mmq_q6k.hip": [r"mmq_q6K_kernelILb0E"],
    "mmq_q6k_exp.hip": [r"mmq_q6K_exp_kernelILb0E"],
}


def test_production_kernels_do_not_spill(asm_texts):
    seen = 0
    for name, pats in PRODUCTION.items():
        meta = _kernel_meta(asm_texts[name])
        for sym, (priv, vg) in meta.items():
            if any(re.search(p, sym) for p in pats):
                seen += 1
                assert priv == 0, f"{sym}: {priv} bytes of scratch per lane"
                assert vg <= 168, f"{sym}: {vg} VGPRs (three waves per SIMD need <= 168)"
    assert seen >= 6
