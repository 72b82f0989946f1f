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


def _occupancy(lds: int, vgpr: int, waves_per_wg: int):
    """Workgroups per CU and waves per SIMD of one instantiation on gfx950: 160 KiB of LDS per
    CU, 512 VGPRs per SIMD lane (allocated in granules of 8), at most 8 waves per SIMD, four
    SIMDs per CU, a workgroup's waves spread over the four."""
    per_simd = min(8, 512 // (-(-vgpr // 8) * 8))
    by_lds = 163840 // lds if lds else 1 << 30
    by_waves = (per_simd * 4) // waves_per_wg
    wgs = min(by_lds, by_waves)
    return wgs, wgs * waves_per_wg // 4


# production instantiations -> (waves per workgroup, workgroups per CU, waves per SIMD) the
# designs rest on
OCCUPANCY = [
    ("mmq_q4k.hip", r"mmq_q4K_kernelILb0ELi1ELi2E", 4, 3, 3),     # 64-token tiles
    ("mmq_q4k.hip", r"mmq_q4K_kernelILb0ELi1ELi1E", 4, 4, 4),     # 32-token tiles
    ("mmq_q4k.hip", r"mmq_q4K_kernelILb0ELi3ELi2E", 12, 1, 3),    # three groups per workgroup
    ("mmq_q4k.hip", r"mmq_q4K_kernelILb0ELi3ELi1E", 12, 1, 3),
    ("mmq_q6k.hip", r"mmq_q6K_kernelILb0ELi1ELb0E", 4, 3, 3),     # raw blocks
    ("mmq_q6k.hip", r"mmq_q6K_kernelILb0ELi1ELb1E", 4, 3, 3),     # prepared
    ("mmq_q6k.hip", r"mmq_q6K_kernelILb0ELi3ELb0E", 12, 1, 3),
    ("mmq_q6k.hip", r"mmq_q6K_kernelILb0ELi3ELb1E", 12, 1, 3),
    ("mmq_q6k_exp.hip", r"mmq_q6K_exp_kernelILb0ELi1ELi2E", 8, 2, 4),   # eight waves per tile
    ("mmq_q6k_exp.hip", r"mmq_q6K_exp_kernelILb0ELi3ELi1E", 12, 1, 3),
]


@pytest.mark.parametrize("src,pat,waves,wgs,per_simd", OCCUPANCY)
def test_production_occupancy(asm_texts, src, pat, waves, wgs, per_simd):
    """The LDS and VGPR budgets of each production kernel give the occupancy its design
    assumes (a change that silently costs a workgroup per CU fails here)."""
    text = asm_texts[src]
    hits = [m for m in re.finditer(r"\.amdhsa_kernel (\S+)(.*?)\.end_amdhsa_kernel", text, re.S)
            if re.search(pat, m.group(1))]
    assert len(hits) == 1, pat
    body = hits[0].group(2)
    lds = int(re.search(r"\.amdhsa_group_segment_fixed_size (\d+)", body).group(1))
    vgpr = int(re.search(r"\.amdhsa_next_free_vgpr (\d+)", body).group(1))
    assert _occupancy(lds, vgpr, waves) == (wgs, per_simd), (pat, lds, vgpr)
