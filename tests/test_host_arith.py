"""Host-side checks of arithmetic shortcuts in the GPU encoders (no GPU).

The NVFP4 encoders compute a block's scale byte from (amax_block / 6) * S
(page "Thinking Machines Details End-to-End 4-Bit Training for Inkling 2
Small", section "Background": an E4M3 scale per 16 values under an fp32
tensor scale). On the GPU the quotient is one multiply and one FMA
correction instead of an IEEE division; tests/div6_exhaustive.c checks on
every fp32 input that this changes no scale byte (same IEEE fp32 multiply and
FMA as the GPU's, denormals kept)."""
import os
import shutil
import subprocess
import tempfile

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_fma_quotient_by_six_is_exact():
    with tempfile.TemporaryDirectory() as d:
        exe = os.path.join(d, "div6")
        # no contraction: the reference quotient and products stay single roundings
        subprocess.run(["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
                        os.path.join(HERE, "div6_exhaustive.c"), "-o", exe, "-lm"], check=True)
        out = subprocess.run([exe], capture_output=True, text=True, timeout=600)
    assert out.returncode == 0, out.stdout + out.stderr
    assert out.stdout.strip() == "mismatches 0 small_bad 0", out.stdout
