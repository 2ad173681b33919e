"""Pins of the oracle's number formats (bf16, e4m3fn) against the pages and torch's CPU casts."""

import math
import os

import numpy as np
import pytest
import torch

from oracle import bf16_decode, bf16_encode_rne, e4m3_decode, e4m3_encode_rne_sat, E4M3_MAX

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_bf16_page_pin_0x4480():
    # Two-stage GEMM page, stage-1 commit: 0x4480 is 1024.0 as bf16 but 4.5 as f16.
    with open(os.path.join(GOLDEN, "bf16_f16_reinterpret.txt")) as f:
        rows = [l.split() for l in f if l.strip() and not l.startswith("#")]
    for bits_hex, bf_val, f16_val in rows:
        bits = np.array([int(bits_hex, 16)], dtype=np.uint16)
        assert bf16_decode(bits)[0] == float(bf_val)
        assert float(bits.view(np.float16)[0]) == float(f16_val)
        assert bf16_encode_rne(np.array([float(bf_val)]))[0] == bits[0]


def test_bf16_encode_matches_torch_on_fp32_inputs():
    g = torch.Generator().manual_seed(0)
    v = torch.cat([torch.randn(20000, generator=g) * s for s in (1e-30, 1e-3, 1.0, 1e5, 1e30)])
    # exact half-way cases: fp32 values whose low 16 bits are 0x8000
    bits = torch.randint(0, 2**15, (5000,), generator=g, dtype=torch.int32) << 16 | 0x8000
    v = torch.cat([v, bits.view(torch.float32)])
    v = v[torch.isfinite(v)]
    ref = v.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    ours = bf16_encode_rne(v.double().numpy())
    assert np.array_equal(ours, ref)
    assert np.array_equal(bf16_decode(ours), v.to(torch.bfloat16).double().numpy())


def test_bf16_subnormal_and_signed_zero():
    assert bf16_encode_rne(np.array([-0.0]))[0] == 0x8000
    tiny = 2.0 ** -133  # smallest bf16 subnormal
    assert bf16_encode_rne(np.array([tiny]))[0] == 1
    assert bf16_encode_rne(np.array([tiny / 2]))[0] == 0          # tie -> even (zero)
    assert bf16_encode_rne(np.array([1.5 * tiny]))[0] == 2        # tie -> even


def test_e4m3_decode_matches_torch_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    ours = e4m3_decode(codes)
    ref = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).double().numpy()
    both_nan = np.isnan(ours) & np.isnan(ref)
    assert np.array_equal(ours[~both_nan], ref[~both_nan])
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    assert np.nanmax(ours) == E4M3_MAX == 448.0
    assert list(np.nonzero(np.isnan(ours))[0]) == [0x7F, 0xFF]


def test_e4m3_encode_matches_torch_in_range():
    g = torch.Generator().manual_seed(1)
    v = torch.cat([torch.randn(50000, generator=g) * s for s in (1e-3, 0.1, 1.0, 30.0, 120.0)])
    # every code value and every midpoint between neighbouring codes (the rounding boundaries)
    pos = torch.arange(127, dtype=torch.uint8).view(torch.float8_e4m3fn).float()
    mids = (pos[1:] + pos[:-1]) / 2
    v = torch.cat([v, pos, -pos, mids, -mids, mids.nextafter(torch.tensor(0.0)),
                   mids.nextafter(torch.tensor(1e9))])
    v = v[v.abs() < 464.0]  # torch turns |v| >= 464 into NaN; saturation is checked below
    ref = v.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    ours = e4m3_encode_rne_sat(v.double().numpy())
    assert np.array_equal(ours, ref)


def test_e4m3_saturation_reading():
    # Values beyond the largest finite e4m3fn value clamp to +-448 (reading of the pages).
    v = np.array([448.0, 463.99, 464.0, 500.0, 1e9, -1e9])
    codes = e4m3_encode_rne_sat(v)
    assert list(e4m3_decode(codes)) == [448.0, 448.0, 448.0, 448.0, 448.0, -448.0]


@pytest.mark.parametrize("x,expected", [(1.0625, 1.0), (1.1875, 1.25), (2.0 ** -10, 0.0),
                                        (1.5 * 2.0 ** -9, 2.0 ** -8), (17.0, 16.0), (19.0, 20.0)])
def test_e4m3_ties_to_even(x, expected):
    assert e4m3_decode(e4m3_encode_rne_sat(np.array([x])))[0] == expected


def test_e4m3_roundtrip_all_finite_codes():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    back = e4m3_encode_rne_sat(e4m3_decode(codes))
    # +0 and -0 keep their sign bit; every finite code maps to itself
    assert np.array_equal(back, codes)
    assert not math.isnan(float(e4m3_decode(np.array([0x7E]))[0]))
