"""The build-time bf16(silu(g)) table of the HIP path (csrc/gen_silu_lut.py, fp64 libm) equals
the oracle's 60-digit decimal values for every entry. The two computations share no code;
this is a host-side check of the table the kernels read."""

import importlib.util
import os

import numpy as np

from oracle import producers as P

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_generated_silu_table_matches_oracle():
    spec = importlib.util.spec_from_file_location(
        "gen_silu_lut", os.path.join(ROOT, "fp8_block_scaled_quant_amd", "csrc", "gen_silu_lut.py"))
    gen = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(gen)
    table = np.array(gen.table(), dtype=np.uint32)
    pats = np.concatenate([np.arange(gen.LO, gen.HI), np.arange(gen.LO, gen.HI) | 0x8000])
    ref = P.silu_bf16_table()[pats].view(np.uint32) >> 16
    assert table.shape == ref.shape
    assert np.array_equal(table, ref)
