"""The gfx950 assembly of every HIP source has no unprotected hazard around
its hand-written memory instructions (see asm_hazards.py): the kernels are
compiled to assembly here (hipcc cross-compiles without a GPU) and scanned."""
import glob
import os
import shutil
import subprocess

import pytest

import asm_hazards as ah

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "head_latent_attention_cache_amd", "csrc")


def test_scanner_flags_a_restored_base_and_an_early_m0():
    bad = "\n".join([
        "\tv_readlane_b32 s0, v255, 9",
        "\tv_readlane_b32 s1, v255, 10",
        "\t;;#ASMSTART",
        "\tglobal_load_lds_dwordx4 v177, s[0:1]",
        "\t;;#ASMEND",
        "\ts_mov_b32 m0, s3",
        "\t;;#ASMSTART",
        "\tglobal_load_lds_dwordx4 v2, off",
        "\t;;#ASMEND",
    ])
    found = ah.scan(bad)
    assert len(found) == 2 and "VALU" in found[0][2] and "M0" in found[1][2]
    good = "\n".join([
        "\tv_readlane_b32 s0, v255, 9",
        "\tv_readlane_b32 s1, v255, 10",
        "\t;;#ASMSTART",
        "\ts_nop 4",
        "\tglobal_load_lds_dwordx4 v177, s[0:1]",
        "\t;;#ASMEND",
    ])
    assert ah.scan(good) == []


def test_scanner_flags_an_early_read_of_an_asm_mfma_result():
    bad = "\n".join([
        "\t;;#ASMSTART",
        "\tv_mfma_f32_32x32x16_bf16 v[16:31], v[2:5], v[6:9], v[16:31]",
        "\t;;#ASMEND",
        "\tv_mov_b64_e32 v[0:1], v[16:17]",
    ])
    found = ah.scan(bad)
    assert len(found) == 1 and "MFMA result" in found[0][2]
    good = "\n".join([
        "\t;;#ASMSTART",
        "\tv_mfma_f32_32x32x16_bf16 v[16:31], v[2:5], v[6:9], v[16:31]",
        "\ts_nop 15",
        "\ts_nop 3",
        "\t;;#ASMEND",
        "\tv_mov_b64_e32 v[0:1], v[16:17]",
    ])
    assert ah.scan(good) == []
    chain = "\n".join([
        "\t;;#ASMSTART",
        "\tv_mfma_f32_32x32x16_bf16 v[16:31], v[2:5], v[6:9], v[16:31]",
        "\t;;#ASMEND",
        "\tv_mfma_f32_32x32x16_bf16 a[0:15], v[10:13], v[6:9], a[0:15]",
        "\t;;#ASMSTART",
        "\tv_mfma_f32_32x32x16_bf16 v[16:31], v[2:5], v[6:9], v[16:31]",
        "\ts_nop 15",
        "\ts_nop 3",
        "\t;;#ASMEND",
    ])
    assert ah.scan(chain) == []


@pytest.mark.parametrize("src", sorted(os.path.basename(p) for p in glob.glob(os.path.join(CSRC, "*.hip"))))
def test_kernel_assembly_has_no_hand_written_load_hazard(src, tmp_path):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available")
    out = tmp_path / (src + ".s")
    cmd = [hipcc, "--offload-arch=gfx950", "-O3", "-std=c++17", "-Xclang", "-target-feature", "-Xclang",
           "-packed-fp32-ops", "--cuda-device-only", "-S", os.path.join(CSRC, src), "-o", str(out)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    found = ah.scan(out.read_text())
    assert found == [], found[:10]
