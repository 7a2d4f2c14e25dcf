"""Pins for the oracle's number formats (E4M3, E8M0, bf16) against things other
than the oracle itself: torch's CPU dtype conversions (library routines), an
independent nearest-in-table encoder, closed-form special values, and the
worked rounding example printed on the AIS explainer page."""

import json
import os

import numpy as np
import pytest
import torch

from oracle import fp8_formats as F

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def torch_decode_e4m3(codes):
    return torch.from_numpy(np.asarray(codes, np.uint8)).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def torch_encode_e4m3(v32):
    """torch's fp32 -> float8_e4m3fn conversion (RNE, no saturation: valid for |v| <= 464)."""
    return torch.from_numpy(np.ascontiguousarray(v32, np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


ALL_CODES = np.arange(256, dtype=np.uint8)
FINITE_CODES = ALL_CODES[(ALL_CODES & 0x7F) != 0x7F]


def test_decode_all_256_codes_match_torch():
    ours = F.decode_e4m3(ALL_CODES)
    ref = torch_decode_e4m3(ALL_CODES)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert nan.sum() == 2 and set(ALL_CODES[nan]) == {0x7F, 0xFF}
    assert np.array_equal(ours[~nan], ref[~nan])
    assert np.array_equal(np.signbit(ours[~nan]), np.signbit(ref[~nan]))   # 0x80 is -0


def test_decode_special_values():
    d = F.decode_e4m3
    assert d(0x7E) == 448.0 and d(0xFE) == -448.0
    assert d(0x38) == 1.0
    assert d(0x08) == 2.0 ** -6          # smallest normal
    assert d(0x01) == 2.0 ** -9          # smallest subnormal
    assert d(0x07) == 7 * 2.0 ** -9      # largest subnormal
    assert d(0x00) == 0.0 and np.signbit(d(0x80))
    assert len(np.unique(d(FINITE_CODES))) == 253   # +0 and -0 compare equal


def test_encode_decode_roundtrip_all_finite_codes():
    vals = F.decode_e4m3(FINITE_CODES).astype(np.float32)
    assert np.array_equal(F.encode_e4m3(vals), FINITE_CODES)


def _near_grid_points():
    """fp32 values within +-4 ulp of every E4M3 value and of every midpoint between
    neighbours (the places where rounding decisions are made), both signs."""
    pos = np.unique(F.decode_e4m3(FINITE_CODES[FINITE_CODES < 0x80]))
    mids = (pos[:-1] + pos[1:]) / 2
    pts = np.concatenate([pos, mids, [464.0, 2.0 ** -10]]).astype(np.float32)
    bits = pts.view(np.uint32).astype(np.int64)
    off = np.arange(-4, 5)
    nb = (bits[:, None] + off[None, :]).reshape(-1)
    nb = nb[(nb >= 0)]
    v = nb.astype(np.uint32).view(np.float32)
    return np.concatenate([v, -v])


def test_encode_matches_torch_near_every_rounding_boundary():
    v = _near_grid_points()
    v = v[np.abs(v) <= 464]
    assert np.array_equal(F.encode_e4m3(v), torch_encode_e4m3(v))


def test_encode_matches_torch_on_all_bf16_values_in_range():
    bits = np.arange(1 << 16, dtype=np.uint32) << 16
    v = bits.view(np.float32)
    v = v[np.isfinite(v) & (np.abs(v) <= 464)]
    assert np.array_equal(F.encode_e4m3(v), torch_encode_e4m3(v))


def test_encode_matches_torch_on_strided_fp32_patterns():
    # every 1021st fp32 bit pattern with |v| <= 464 (about 2.2 M values), both signs
    top = np.float32(464).view(np.uint32)
    bits = np.arange(0, int(top) + 1, 1021, dtype=np.uint32)
    v = bits.view(np.float32)
    v = np.concatenate([v, -v])
    assert np.array_equal(F.encode_e4m3(v), torch_encode_e4m3(v))


def _table_encoder(v):
    """Independent encoder: nearest finite E4M3 value by exhaustive search over
    the 126 positive finite values (from torch's decode), ties to the even code,
    magnitudes above 448 clamp to 448, sign copied onto the code."""
    codes = np.arange(0, 0x7F, dtype=np.uint8)                # 0x00 .. 0x7E, positive
    table = torch_decode_e4m3(codes)
    out = np.empty(v.shape, np.uint8)
    for i, x in enumerate(v.astype(np.float64)):
        a = min(abs(x), 448.0)
        d = np.abs(table - a)
        best = np.flatnonzero(d == d.min())
        c = int(best[0]) if len(best) == 1 else int(best[best % 2 == 0][0])
        out[i] = c | (0x80 if np.signbit(x) else 0)
    return out


def test_encode_matches_table_search_including_saturation():
    rng = np.random.default_rng(0)
    v = np.concatenate([
        rng.standard_normal(3000).astype(np.float32) * 100,
        (rng.random(1000) * 2 ** -6).astype(np.float32),        # subnormal range
        np.array([464, 465, 480, 1000, 1e30, -466, -1e30, 0.0, -0.0, -1e-30, 2 ** -10, 3 * 2 ** -10],
                 np.float32),
        _near_grid_points()[::7],
    ])
    assert np.array_equal(F.encode_e4m3(v), _table_encoder(v))


def test_encode_saturation_and_signed_zero():
    e = F.encode_e4m3
    assert list(e(np.array([448, 463.9, 464, 465, 479, 480, 1e6, 3e38], np.float32))) == [0x7E] * 8
    assert list(e(np.array([-448, -464, -1e6], np.float32))) == [0xFE] * 3
    assert e(np.float32(0.0)) == 0x00 and e(np.float32(-0.0)) == 0x80
    assert e(np.float32(-1e-30)) == 0x80 and e(np.float32(1e-30)) == 0x00
    assert e(np.float32(2 ** -10)) == 0x00                       # exact tie with 0 -> even code 0
    assert e(np.float32(3 * 2 ** -10)) == 0x02                   # tie between 1 and 2 (x 2**-9) -> even 2
    assert e(np.float32(1.0625)) == 0x38 and e(np.float32(1.1875)) == 0x3A
    with pytest.raises(ValueError):
        e(np.float32(np.nan))


def test_ais_worked_rounding_example():
    """The AIS explainer's worked example: bf16 logits [1.06, 1.00, 0.94] round to
    [1.00, 1.00, 0.9375] in FP8 at unit scale; the printed softmax percentages of
    both vectors follow."""
    g = json.load(open(os.path.join(GOLDEN, "ais_logit_rounding.json")))
    bf = np.array(g["bf16_logits"], np.float32)
    got = F.decode_e4m3(F.encode_e4m3(bf))
    assert np.array_equal(got, np.array(g["fp8_logits"]))

    def softmax_pct(z):
        z = np.asarray(z, np.float64)
        p = np.exp(z - z.max())
        return 100 * p / p.sum()
    assert np.allclose(softmax_pct(g["bf16_logits"]), g["bf16_softmax_percent"], atol=0.006)
    assert np.allclose(softmax_pct(got), g["fp8_softmax_percent"], atol=0.006)


def test_e8m0_decode_matches_torch():
    b = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(b).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    ours = F.decode_e8m0(b)
    assert np.isnan(ours[255]) and np.isnan(ref[255])
    assert np.array_equal(ours[:255], ref[:255])
    assert ours[127] == 1.0 and ours[0] == 2.0 ** -127 and ours[254] == 2.0 ** 127


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(1)
    v = np.concatenate([
        rng.standard_normal(200000).astype(np.float32) * np.float32(10) ** rng.integers(-30, 30, 200000).astype(np.float32),
        # every pattern whose low 16 bits sit at or next to the tie 0x8000, across exponents
        ((np.arange(0, 0x7F7F, 3, dtype=np.uint32) << 16)[:, None] + np.array([0x7FFF, 0x8000, 0x8001], np.uint32)).reshape(-1).view(np.float32),
        np.array([0.0, -0.0, 1e-45, -1e-45, 3e38], np.float32),
    ])
    v = v[np.isfinite(v)]
    ref = torch.from_numpy(v).to(torch.bfloat16).to(torch.float32).numpy()
    ours = F.round_to_bf16(v)
    assert np.array_equal(ours.view(np.uint32), ref.view(np.uint32))
