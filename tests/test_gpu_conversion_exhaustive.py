"""The quantizers' fp32 -> E4M3 conversion over every (x, amax) pair they can meet, byte for
byte against the oracle ([AIS] quantizer equation and worked rounding example; readings
c2-c5, c7, c21).

Why a few binades of amax suffice: a group's codes depend on x / s and on how the kernel
forms it. Multiplying every element of a group by 2^j (j an integer, all values staying
within bf16) multiplies amax by 2^j, and then
- fp32 scales s = fl32(amax / 448) become s * 2^j exactly, as long as s stays a normal fp32
  (a power-of-two factor commutes with a correctly rounded division away from underflow);
  the kernels' reciprocal pair (h = 1/s rounded toward zero, l = fl32((1 - h s) h)) becomes
  (h, l) * 2^-j as long as l stays normal, i.e. for amax below 1.75 * 2^110;
- power-of-two and MX scales 2^e become 2^(e + j), as long as e stays inside its clamp;
so every quotient, and every code, is unchanged. A bf16 x that would be subnormal in
another binade is, in this one, a normal bf16 with trailing zero bits, which the sweep
includes. So the sweep takes
- every amax of one binade, the 128 bf16 mantissas in [1, 2), each with every bf16 x of
  magnitude at most amax, both signs (the amax itself also with its sign flipped);
- separately, every amax whose scale leaves that regime: fp32 scales that are subnormal
  (amax < 448 * 2^-126) and power-of-two / MX exponents at the -127 clamp (amax <= 448 *
  2^-127 up to the first exponent above the clamp), each with every x of smaller magnitude;
- the binades where l is subnormal are not equivalent to one another; the sweep takes the
  first, [2^110, 2^111), and the last, [2^127, max bf16], each amax with every x of smaller
  magnitude (an exhaustive CPU check of the same arithmetic covers all of them).
Each group holds +-amax first and up to 127 (MX: 31) of the x values; the oracle quantizes the
same tensor. The 1x128 quantizer runs in its row kernel and, on the transposed tensor, in the
128x1 column kernel; the power-of-two and MXFP8 quantizers likewise."""

import numpy as np
import pytest
import torch

import fp8_block_scaled_quant_amd as F
from oracle import quantize as OQ
from gpu_util import dev

pytestmark = pytest.mark.gpu


def _bf16(bits):
    return (np.asarray(bits, np.uint32) << 16).view(np.float32)


def _groups(amax_bits, width):
    """Rows of `width` bf16 values: +-amax first, then every x with |x| <= amax (both signs)."""
    rows = []
    for i, ab in enumerate(amax_bits):
        mags = np.arange(0, int(ab) + 1, dtype=np.uint32)             # every magnitude <= amax
        xs = np.concatenate([mags, mags | 0x8000])
        n = width - 1
        pad = (-len(xs)) % n
        xs = np.concatenate([xs, np.zeros(pad, np.uint32)]).reshape(-1, n)
        lead = np.full((xs.shape[0], 1), ab | (0x8000 if i % 2 else 0), np.uint32)
        lead[1::2] ^= 0x8000                                         # both signs of amax
        rows.append(np.concatenate([lead, xs], axis=1))
    return _bf16(np.concatenate(rows))


def _pad_rows(x, mult):
    r = (-x.shape[0]) % mult
    return np.concatenate([x, np.zeros((r, x.shape[1]), np.float32)]) if r else x


def _to_dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).to(torch.bfloat16).to(dev())


def _eq(g, ref, what):
    torch.cuda.synchronize()
    g = g.cpu().numpy()
    ref = np.asarray(ref)
    if g.dtype == np.float32:
        g, ref = g.view(np.uint32), np.asarray(ref, np.float32).view(np.uint32)
    bad = np.argwhere(g != ref)
    assert len(bad) == 0, f"{what}: {len(bad)} mismatches, first at {bad[:3].tolist()}"


ONE_BINADE = np.arange(0x3F80, 0x4000, dtype=np.uint32)              # amax in [1, 2)
# fp32 scale fl32(amax / 448) subnormal: amax < 448 * 2^-126 = 1.75 * 2^-118 (bf16 0x04E0)
SUBNORMAL_SCALE = np.arange(0x0001, 0x04E0, dtype=np.uint32)
# power-of-two exponent at the -127 clamp: amax <= 448 * 2^-127 = 1.75 * 2^-119 (bf16 0x0460);
# include the binade above so the first unclamped exponents are covered too
CLAMPED_EXPONENT = np.arange(0x0001, 0x04E0, dtype=np.uint32)


# l = fl32((1 - h s) h) subnormal: amax >= 1.75 * 2^110; the first and the last such binade
LARGE_AMAX = np.concatenate([np.arange(0x7680, 0x7700, dtype=np.uint32), np.arange(0x7F00, 0x7F80, dtype=np.uint32)])


def _region(region, pow2):
    if region == "one_binade":
        return ONE_BINADE
    if region == "large_amax":
        return LARGE_AMAX
    return CLAMPED_EXPONENT if pow2 else SUBNORMAL_SCALE


@pytest.mark.parametrize("region", ["one_binade", "small_amax", "large_amax"])
@pytest.mark.parametrize("pow2", [False, True])
def test_1x128_conversion_exhaustive(region, pow2):
    amax = _region(region, pow2)
    x = _pad_rows(_groups(amax, 128), 128)                            # [G][128], G % 128 == 0
    quant_gpu = F.fp8_quant_act_1x128_pow2 if pow2 else F.fp8_quant_act_1x128
    rows_ref = OQ.quant_act_1x128_pow2 if pow2 else OQ.quant_act_1x128
    q, s = quant_gpu(_to_dev(x))[:2]
    rq, rs = rows_ref(x)
    _eq(q, rq, f"rows q ({region}, pow2={pow2}, {x.shape[0]} groups)")
    _eq(s, rs, f"rows s ({region}, pow2={pow2})")
    # the same groups as 128x1 columns: the transposed tensor [128][G], quantized column-wise
    xt = np.ascontiguousarray(x.T)
    _, _, qt, st = quant_gpu(_to_dev(xt), rowwise=False, colwise=True)
    _eq(qt, rq, f"cols qt ({region}, pow2={pow2})")
    _eq(st, rs, f"cols st ({region}, pow2={pow2})")


@pytest.mark.parametrize("region", ["one_binade", "small_amax", "large_amax"])
def test_mx_conversion_exhaustive(region):
    amax = _region(region, True)
    x = _groups(amax, 32)                                             # [G][32]
    x = _pad_rows(x, 4).reshape(-1, 128)                              # 4 groups per row of 128
    q, e = F.mxfp8_quant_1x32(_to_dev(x))
    rq, re = OQ.quant_mx_1x32(x)
    _eq(q, rq, f"MX q ({region})")
    _eq(e, re, f"MX e8m0 ({region})")
