"""The register-path top-k finds the crossing bucket's members by two compares
on the bucket's fma result instead of recomputing the clamped bucket.  This
checks that identity in float32 arithmetic on the CPU (C, correctly rounded
fmaf, truncating conversion, as the GPU's v_fma_f32 and v_cvt_i32_f32)."""
from __future__ import annotations

import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_bucket_interval_identity(tmp_path):
    exe = str(tmp_path / "bucket_interval")
    subprocess.run(["gcc", "-O2", "-ffp-contract=off", "-o", exe, os.path.join(HERE, "bucket_interval.c"), "-lm"],
                   check=True)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "mismatches 0" in r.stdout
    # the unclamped bucket does go below 1 on these rows: the clamp is needed
    below = int(r.stdout.strip().rsplit(" ", 1)[1])
    assert below > 0
