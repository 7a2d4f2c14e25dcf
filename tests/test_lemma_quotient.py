"""Exhaustive CPU checks of the arithmetic the quantizer kernels use instead of a division
per value (every bf16 (x, amax) pair):
- fl32(x * fl64(1/s)) equals the IEEE fp32 division fl32(x / s) the oracle performs (the
  kernels' form for a subnormal s);
- for a normal s, q = fl32(x h + fl32(x l)) with h = 1/s rounded toward zero and
  l = fl32((1 - h s) h) has the same E4M3 value, sign of zero included, as fl32(x / s) (the
  kernels' form for every other fp32 scale); the one-multiply form fl32(x h) does not;
- |q| stays below 464, so the hardware E4M3 conversion rounds the top values to 448
  rather than NaN."""

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


def _run_code_check(tmp_path, *defines):
    exe = tmp_path / ("code_check" + "".join(defines))
    subprocess.run(["gcc", "-O2", "-fopenmp", "-ffp-contract=off", *defines,
                    os.path.join(HERE, "lemma", "code_check.c"), "-o", str(exe), "-lm"], check=True)
    out = subprocess.run([str(exe)], capture_output=True, text=True, timeout=600)
    fields = out.stdout.split()
    return int(fields[1]), int(fields[3]), float(fields[5])


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_double_float_quotient_gives_the_oracle_codes_for_all_bf16_pairs(tmp_path):
    pairs, bad, maxabs = _run_code_check(tmp_path)
    assert pairs == 1063843488          # the pairs above whose amax >= 448 * 2^-126
    assert bad == 0
    assert maxabs < 449.0
    # control: dropping the low part of the reciprocal changes codes on exact ties
    pairs, bad, _ = _run_code_check(tmp_path, "-DDROP_LOW_PART")
    assert pairs == 1063843488 and bad > 0
