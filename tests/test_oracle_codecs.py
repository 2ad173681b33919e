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


# ---------------------------------------------------------------------------- mxfp4 (MX)
from oracle import (E2M1_TABLE, e2m1_decode, e2m1_encode_rne_sat, e8m0_decode, fp4_pack, fp4_unpack,  # noqa: E402
                    mx_dequantize, mx_quantize)


def test_e2m1_table_is_the_mx_fp4_value_set():
    # the eight FP4 E2M1 magnitudes of the MX format, then their negatives (code 8 = -0)
    assert list(E2M1_TABLE[:8]) == [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    assert list(E2M1_TABLE[8:]) == [-0.0, -0.5, -1.0, -1.5, -2.0, -3.0, -4.0, -6.0]
    assert math.copysign(1.0, E2M1_TABLE[8]) == -1.0


@pytest.mark.parametrize("y,expected", [(0.25, 0.0), (0.75, 1.0), (1.25, 1.0), (1.75, 2.0), (2.5, 2.0),
                                        (3.5, 4.0), (5.0, 4.0), (0.26, 0.5), (4.9, 4.0), (5.1, 6.0),
                                        (6.0, 6.0), (7.0, 6.0), (1e9, 6.0), (-5.0, -4.0), (-7.0, -6.0)])
def test_e2m1_ties_to_even_and_saturation(y, expected):
    assert e2m1_decode(e2m1_encode_rne_sat(np.array([y])))[0] == expected


def test_e2m1_encode_is_nearest_on_a_dense_grid():
    ys = np.linspace(-7.0, 7.0, 28001)
    got = e2m1_decode(e2m1_encode_rne_sat(ys))
    grid = np.array([-6, -4, -3, -2, -1.5, -1, -0.5, 0, 0.5, 1, 1.5, 2, 3, 4, 6], dtype=np.float64)
    best = np.abs(np.clip(ys, -6, 6)[:, None] - grid).min(axis=1)
    assert np.all(np.abs(np.clip(ys, -6, 6) - got) <= best + 1e-15)


def test_e2m1_roundtrip_all_codes():
    codes = np.arange(16, dtype=np.uint8)
    assert np.array_equal(e2m1_encode_rne_sat(e2m1_decode(codes)), codes)


def test_e8m0_points():
    got = e8m0_decode(np.array([0, 1, 120, 127, 130, 254, 255]))
    assert list(got[:6]) == [2.0 ** -127, 2.0 ** -126, 2.0 ** -7, 1.0, 8.0, 2.0 ** 127]
    assert math.isnan(got[6])


def test_fp4_nibble_packing():
    assert list(fp4_unpack(np.array([0x21, 0xF8], dtype=np.uint8))) == [1, 2, 8, 15]
    rng = np.random.default_rng(5)
    c = rng.integers(0, 16, size=(7, 64)).astype(np.uint8)
    assert np.array_equal(fp4_unpack(fp4_pack(c)), c)


def test_mx_block_rules():
    base = np.zeros(32)
    base[:3] = [6.0, 3.0, -1.5]
    codes, e = mx_quantize(base[None])
    assert e.tolist() == [[127]] and codes[0, :3].tolist() == [7, 5, 11] and not codes[0, 3:].any()
    # scaling by a power of two only moves the shared exponent
    codes2, e2 = mx_quantize(base[None] * 2.0 ** -10)
    assert e2.tolist() == [[117]] and np.array_equal(codes2, codes)
    # floor(log2(7.9)) = 2: scale 1, and 7.9 saturates to 6
    blk = base.copy()
    blk[0] = 7.9
    c3, e3 = mx_quantize(blk[None])
    assert e3.tolist() == [[127]] and c3[0, 0] == 7
    # floor(log2(0.1)) = -4: scale 2**-6, 0.1 / 2**-6 = 6.4 -> 6
    blk = np.zeros(32)
    blk[5] = 0.1
    c4, e4 = mx_quantize(blk[None])
    assert e4.tolist() == [[121]] and c4[0, 5] == 7
    assert mx_dequantize(c4, e4)[0, 5] == 6.0 * 2.0 ** -6
    # an all-zero block takes scale 1 and zero codes; blocks are independent
    c5, e5 = mx_quantize(np.concatenate([np.zeros(32), base])[None])
    assert e5.tolist() == [[127, 127]] and not c5[0, :32].any()


def test_mx_dequantize_error_bound():
    rng = np.random.default_rng(7)
    v = rng.standard_normal((200, 128)) * np.exp(rng.uniform(-8, 8, size=(200, 1)))
    codes, e = mx_quantize(v)
    deq = mx_dequantize(codes, e)
    scale = np.repeat(e8m0_decode(e), 32, axis=-1)
    y = np.abs(v) / scale
    # spacing of E2M1 is 0.5 below 2, 1 in [2, 4), 2 in [4, 6]: error <= half of it, and
    # magnitudes above 6 (possible since the block maximum lies in [4, 8)) clamp to 6
    half_step = np.where(y < 2, 0.25, np.where(y < 4, 0.5, 1.0))
    allowed = np.where(y <= 6, half_step, y - 6) * scale
    assert np.all(np.abs(deq - v) <= allowed * (1 + 1e-12))
    # the block maximum always lands in [4, 8) before rounding
    ymax = (np.abs(v).reshape(200, 4, 32) / e8m0_decode(e)[..., None]).max(axis=-1)
    assert np.all((ymax >= 4) & (ymax < 8))
