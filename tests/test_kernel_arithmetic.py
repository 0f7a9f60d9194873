"""Host proofs of the arithmetic shortcuts the GPU kernels take where floating point decides an
integer code, so that the kernels' codes equal the oracle's for every input and not only for the
sampled ones the GPU parity tests see."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_int4_scale_and_reciprocal_shortcuts_are_exact(tmp_path):
    """Exhaustive over every finite fp32 group maximum and every bf16 scale: the activation
    kernel's fma-corrected amax/7 and its one-step reciprocal give exactly the IEEE results the
    oracle's quantizer uses (tests/kernel_division_check.c)."""
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not available")
    exe = str(tmp_path / "divcheck")
    src = os.path.join(ROOT, "tests", "kernel_division_check.c")
    cmd = [gcc, "-O2", "-mfma", "-ffp-contract=off", "-fopenmp", src, "-o", exe, "-lm"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:   # no OpenMP runtime: build it single-threaded
        res = subprocess.run([c for c in cmd if c != "-fopenmp"], capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-2000:]
    run = subprocess.run([exe], capture_output=True, text=True, timeout=600,
                         env=dict(os.environ, OMP_NUM_THREADS=str(min(8, os.cpu_count() or 1))))
    assert run.returncode == 0, run.stdout + run.stderr
    assert "scale: 0 mismatches" in run.stdout and "reciprocal: 0 of" in run.stdout
