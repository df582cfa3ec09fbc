"""The FP8 row quantizer's division, checked exhaustively on the CPU.

The quantizer's E4M3 code is RNE(fl32(x / s)) with the row scale s = fl32(amax / 448)
(page "WaveSpeedAI X DataCrunch", engine list: FP8 with per-row scales).  For rows
whose largest magnitude is at least 2^-60 the kernel forms the quotient from one
reciprocal per row and one FMA correction instead of a division per element.
tests/csrc/fp8_row_division_check.c replays that formula for every bf16 amax >= 2^-60
and every bf16 x with |x| <= amax (about 10^9 pairs, a few seconds on 8 cores) and
requires the IEEE quotient bit for bit wherever |x / s| >= 2^-10, and otherwise a
quotient of magnitude <= 2^-10 with the sign of x (both round to the same signed E4M3
zero).  The GPU parity tests then compare the kernel's codes with the oracle's.
"""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_rcp_correction_equals_ieee_division_for_every_bf16_pair(tmp_path):
    exe = tmp_path / "fp8_row_division_check"
    src = os.path.join(HERE, "csrc", "fp8_row_division_check.c")
    # no contraction: every multiply and FMA rounds exactly where the formula says
    flags = ["-O2", "-ffp-contract=off", "-fopenmp"]
    r = subprocess.run(["gcc", *flags, src, "-o", str(exe), "-lm"], capture_output=True, text=True)
    if r.returncode != 0:   # no OpenMP runtime: the same check on one thread
        r = subprocess.run(["gcc", "-O2", "-ffp-contract=off", src, "-o", str(exe), "-lm"], capture_output=True,
                           text=True)
    assert r.returncode == 0, r.stderr
    run = subprocess.run([str(exe)], capture_output=True, text=True, timeout=600)
    assert run.returncode == 0, run.stdout + run.stderr
    assert "mismatches 0" in run.stdout
