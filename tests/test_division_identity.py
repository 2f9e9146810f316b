"""The encoders divide by a group's scale with one correctly rounded
reciprocal and one FMA residual correction instead of an IEEE division per
element.  This pins that the two agree wherever the quotient can decide a
code (C model of the device sequence, compiled with gcc; CPU only)."""

import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_fma_corrected_division_matches_ieee(tmp_path):
    exe = str(tmp_path / "div_identity")
    # -ffp-contract=off: every operation rounds exactly as written
    subprocess.check_call(["gcc", "-O2", "-ffp-contract=off", "-o", exe, os.path.join(HERE, "div_identity.c"), "-lm"])
    out = subprocess.run([exe], capture_output=True, text=True, timeout=300)
    assert out.returncode == 0, out.stdout + out.stderr
    assert " 0 disagreements" in out.stdout
