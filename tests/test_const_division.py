"""The row scale s' = m / r of the int4, int6 and int8 classes is computed in
the step kernel as a product and two fused multiply-adds (Markstein's
correction step with the rounded reciprocal of r) instead of an IEEE
division.  The scale must equal the oracle's correctly rounded quotient bit
for bit, so the replacement is checked here on the host for every finite
non-negative fp32 m and each r in {7, 31, 127} (tests/host/const_div_check.c,
built with gcc; the host's fused multiply-add and division are IEEE)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_row_scale_division_is_exact_for_every_fp32(tmp_path):
    exe = tmp_path / "const_div_check"
    src = os.path.join(ROOT, "tests", "host", "const_div_check.c")
    cmd = ["gcc", "-O2", "-mfma", "-ffp-contract=off", "-fopenmp", src, "-o", str(exe), "-lm"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=900)
    assert r.returncode == 0 and "const div ok" in r.stdout, (r.stdout, r.stderr[-2000:])
