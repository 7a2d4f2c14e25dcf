"""Exhaustive CPU check of the fp32-quotient identity used by the quantizer kernels
(every bf16 (x, amax) pair): the kernels form fl32(x / s) as fl32(x * fl64(1/s)), which
must equal the IEEE fp32 division the oracle performs, and |x / s| must stay below 464
so the hardware E4M3 conversion rounds the top values to 448 rather than NaN."""

import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_fp64_reciprocal_quotient_is_exact_for_all_bf16_pairs(tmp_path):
    exe = tmp_path / "quotient_check"
    subprocess.run(["gcc", "-O2", "-fopenmp", "-ffp-contract=off", os.path.join(HERE, "lemma", "quotient_check.c"),
                    "-o", str(exe), "-lm"], check=True)
    out = subprocess.run([str(exe)], capture_output=True, text=True, timeout=600)
    fields = out.stdout.split()
    pairs, bad, maxabs = int(fields[1]), int(fields[3]), float(fields[5])
    assert pairs == 1065402238          # 2 * sum over the 32639 positive amax of (#bf16 <= amax)
    assert bad == 0 and out.returncode == 0
    assert maxabs < 464.0
