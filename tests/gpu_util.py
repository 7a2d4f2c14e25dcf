"""Helpers for the GPU parity tests: host<->device moves and the comparison rules.

Rules (from the method's contract): quantized bytes and scales are compared bit for
bit; fp32 GEMM outputs must satisfy max|y_gpu - y_oracle| <= 2e-3 * RMS(y_oracle); bf16
GEMM outputs must equal the RNE bf16 rounding of the same kernel's fp32 output, and lie
within that tolerance plus half a bf16 ulp of the oracle."""

import numpy as np
import torch

GEMM_TOL = 2e-3


def dev():
    return torch.device("cuda", 0)


def bf16_dev(a32: np.ndarray) -> torch.Tensor:
    """float32 array of bf16-exact values -> bf16 tensor on the GPU."""
    return torch.from_numpy(np.ascontiguousarray(a32, dtype=np.float32)).to(torch.bfloat16).to(dev())


def u8_dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).to(dev())


def f32_dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev())


def host(t: torch.Tensor) -> np.ndarray:
    torch.cuda.synchronize()
    if t.dtype == torch.bfloat16:
        return t.float().cpu().numpy()
    return t.cpu().numpy()


def assert_bytes_equal(gpu: torch.Tensor, ref: np.ndarray, what: str):
    g = host(gpu)
    assert g.shape == ref.shape, (what, g.shape, ref.shape)
    if g.dtype == np.float32:
        g, ref = g.view(np.uint32), np.asarray(ref, np.float32).view(np.uint32)
    bad = np.argwhere(g != ref)
    assert len(bad) == 0, f"{what}: {len(bad)} mismatches, first at {bad[:5].tolist()}"


def assert_gemm_close(y_gpu_f32: np.ndarray, y_ref: np.ndarray, what: str, rms=None):
    rms = float(np.sqrt(np.mean(np.square(y_ref)))) if rms is None else rms
    err = float(np.max(np.abs(y_gpu_f32.astype(np.float64) - y_ref))) if y_ref.size else 0.0
    assert err <= GEMM_TOL * rms, f"{what}: max|err| {err:.3e} > {GEMM_TOL} * RMS {rms:.3e}"
    return err / rms if rms else 0.0


def assert_bf16_consistent(y_bf16: torch.Tensor, y_f32: torch.Tensor, y_ref: np.ndarray, what: str, rms=None):
    """bf16 output == RNE(fp32 output of the same kernel), bitwise; and close to the oracle."""
    torch.cuda.synchronize()
    rounded = y_f32.to(torch.bfloat16)
    same = torch.equal(y_bf16.view(torch.int16), rounded.view(torch.int16))
    assert same, f"{what}: bf16 output is not the RNE rounding of the fp32 output"
    yb = host(y_bf16).astype(np.float64)
    rms = float(np.sqrt(np.mean(np.square(y_ref)))) if rms is None else rms
    half_ulp = np.ldexp(1.0, np.frexp(np.abs(yb))[1] - 9)    # half of bf16's 8-bit significand ulp
    assert np.all(np.abs(yb - y_ref) <= GEMM_TOL * rms + half_ulp), f"{what}: bf16 output outside tolerance"
