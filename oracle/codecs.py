"""Number formats used on the path: bfloat16 and fp8 e4m3 (OCP "fn" variant).

TEST INFRASTRUCTURE ONLY (see the package docstring).

bfloat16 is the activation/weight/intermediate type of the bf16 path.  The
two-stage GEMM page ("Port moe_gemm_2stage ... fp8", stage-1 commit and the
summary's "Notable fixes") pins the encoding by one example: the bit
pattern 0x4480 reads as 1024.0 in bf16 and as 4.5 in f16.

fp8: the same page names the builder's fp8 element type as e4m3 "FNUZ"
(the gfx942 encoding); the workload statement only says "e4m3".  Reading
taken: OCP e4m3fn (exponent bias 7, largest finite 448, no infinities,
0x7F/0xFF are NaN), the format gfx950's conversion and MFMA instructions
use.  The decode table below is written from that definition.  Rounding is
round-to-nearest-even; values beyond +-448 saturate to +-448 (reading: the
pages do not state the overflow rule).
"""

from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0
_E4M3_BIAS = 7
_E4M3_MIN_NORMAL_EXP = 1 - _E4M3_BIAS  # -6: smallest normal is 2**-6
_E4M3_MAN_BITS = 3


def _e4m3_table() -> np.ndarray:
    """Value of every one of the 256 e4m3fn codes, as float64 (NaN for 0x7F, 0xFF)."""
    vals = np.empty(256, dtype=np.float64)
    for code in range(256):
        sign = -1.0 if code & 0x80 else 1.0
        exp = (code >> 3) & 0xF
        man = code & 0x7
        if exp == 0xF and man == 0x7:
            vals[code] = np.nan
        elif exp == 0:  # subnormal: man/8 * 2**(1-bias)
            vals[code] = sign * (man / 8.0) * 2.0 ** _E4M3_MIN_NORMAL_EXP
        else:
            vals[code] = sign * (1.0 + man / 8.0) * 2.0 ** (exp - _E4M3_BIAS)
    return vals


E4M3_TABLE = _e4m3_table()
# positive finite codes 0..126 map monotonically onto increasing values
_E4M3_POS_VALUES = E4M3_TABLE[:127]


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    """uint8 e4m3fn codes -> float64 values (table lookup)."""
    return E4M3_TABLE[np.asarray(codes, dtype=np.uint8)]


def e4m3_encode_rne_sat(x: np.ndarray) -> np.ndarray:
    """Real values -> uint8 e4m3fn codes, round-to-nearest-even, saturating at +-448.

    Each value is split as m * 2**e with m in [0.5, 1).  A normal e4m3 number
    has 4 significant bits, so the spacing of representable values around x
    is 2**(e-4); below the smallest normal 2**-6 the spacing is the
    subnormal step 2**-9.  Dividing by the spacing and rounding half to even
    (np.rint) gives the nearest representable value; a result that lands on
    the next power of two is itself representable.
    """
    x = np.asarray(x, dtype=np.float64)
    if np.isnan(x).any():
        raise ValueError("NaN is outside the contract of the e4m3 encoder")
    mag = np.abs(x)
    _, e = np.frexp(mag)  # mag = m * 2**e, m in [0.5, 1)
    # exponent of the leading bit is e-1; clamp to the normal range's bottom
    lead = np.maximum(e - 1, _E4M3_MIN_NORMAL_EXP)
    spacing = np.ldexp(1.0, lead - _E4M3_MAN_BITS)
    rounded = np.rint(mag / spacing) * spacing
    rounded = np.minimum(rounded, E4M3_MAX)
    idx = np.searchsorted(_E4M3_POS_VALUES, rounded)
    if not np.array_equal(_E4M3_POS_VALUES[idx], rounded):
        raise AssertionError("rounded value is not an e4m3 code")
    sign = np.signbit(x).astype(np.uint8) << 7
    return (idx.astype(np.uint8) | sign).astype(np.uint8)


def bf16_decode(bits: np.ndarray) -> np.ndarray:
    """uint16 bfloat16 bit patterns -> float64 (the top half of an fp32)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def bf16_encode_rne(x: np.ndarray) -> np.ndarray:
    """Real values -> uint16 bfloat16 bit patterns, round-to-nearest-even, one rounding.

    bfloat16 keeps 8 significant bits and fp32's exponent range.  Around
    x = m * 2**e (m in [0.5, 1)) the spacing of bf16 values is 2**(e-8); in
    the subnormal range (below 2**-126) it is 2**-133.  Inputs must be finite
    and below the bf16 overflow threshold (all values on this path are).
    """
    x = np.asarray(x, dtype=np.float64)
    if not np.isfinite(x).all():
        raise ValueError("non-finite input is outside the contract of the bf16 encoder")
    mag = np.abs(x)
    _, e = np.frexp(mag)
    lead = np.maximum(e - 1, -126)
    spacing = np.ldexp(1.0, lead - 7)
    rounded = np.rint(mag / spacing) * spacing
    if (rounded >= 2.0**128).any():
        raise ValueError("bf16 overflow is outside the contract")
    val = np.where(np.signbit(x), -rounded, rounded)
    bits32 = val.astype(np.float32).view(np.uint32)  # exact: val has <= 8 significant bits
    if (bits32 & np.uint32(0xFFFF)).any():
        raise AssertionError("rounded value is not a bf16 number")
    return (bits32 >> np.uint32(16)).astype(np.uint16)


# ---------------------------------------------------------------------------- mxfp4
# "[RadeonFlow] flydsl mxfp4 a4w4 MoE" (ROCm/aiter #3828) runs both GEMMs with 4-bit
# activations and weights ("a4w4") in the mxfp4 format; the page does not define it.
# Reading taken: the OCP Microscaling (MX) format -- elements FP4 E2M1 (1 sign bit, 2
# exponent bits with bias 1, 1 mantissa bit: magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6; no
# infinities or NaN), one shared E8M0 scale 2**(e - 127) per block of 32 consecutive
# elements along K (e = 255 is NaN).  Block quantisation follows the MX definition:
# shared exponent = floor(log2(max |v|)) - 2 (2 = the largest E2M1 exponent), elements
# rounded to nearest even on the E2M1 grid after dividing by the scale, magnitudes
# beyond 6 saturating to 6; an all-zero block takes scale 1 (e = 127).  Storage: two
# elements per byte, element 2j in the low nibble.

MX_BLOCK = 32
E2M1_MAX = 6.0


def _e2m1_table() -> np.ndarray:
    """Value of every one of the 16 E2M1 codes, as float64 (code 8 is -0.0)."""
    vals = np.empty(16, dtype=np.float64)
    for code in range(16):
        sign = -1.0 if code & 0x8 else 1.0
        exp = (code >> 1) & 0x3
        man = code & 0x1
        if exp == 0:  # subnormal: man/2 * 2**(1 - bias), bias 1
            vals[code] = sign * (man / 2.0)
        else:
            vals[code] = sign * (1.0 + man / 2.0) * 2.0 ** (exp - 1)
    return vals


E2M1_TABLE = _e2m1_table()
_E2M1_POS = E2M1_TABLE[:8]  # codes 0..7, increasing


def e2m1_decode(codes: np.ndarray) -> np.ndarray:
    """E2M1 codes (0..15) -> float64 values (table lookup)."""
    return E2M1_TABLE[np.asarray(codes, dtype=np.uint8) & 0xF]


def e2m1_encode_rne_sat(y: np.ndarray) -> np.ndarray:
    """Real values -> E2M1 codes: the nearest of the 8 magnitudes, a tie going to the code
    with a zero mantissa bit (even), magnitudes above 6 saturating; the sign bit is the
    value's sign (so -0.0 and small negatives give code 8)."""
    y = np.asarray(y, dtype=np.float64)
    if np.isnan(y).any():
        raise ValueError("NaN is outside the contract of the E2M1 encoder")
    mag = np.minimum(np.abs(y), E2M1_MAX)
    dist = np.abs(mag[..., None] - _E2M1_POS)          # distance to every magnitude
    best = dist.min(axis=-1, keepdims=True)
    cand = dist == best                                  # one or two nearest codes
    even = cand & (np.arange(8) % 2 == 0)
    pick = np.where(even.any(axis=-1), even.argmax(axis=-1), cand.argmax(axis=-1))
    sign = np.signbit(y).astype(np.uint8) << 3
    return (pick.astype(np.uint8) | sign).astype(np.uint8)


def e8m0_decode(e: np.ndarray) -> np.ndarray:
    """E8M0 scale codes -> float64 2**(e - 127); 255 is NaN."""
    e = np.asarray(e, dtype=np.int64)
    return np.where(e == 255, np.nan, np.ldexp(1.0, e - 127))


def fp4_unpack(packed: np.ndarray) -> np.ndarray:
    """uint8 [..., n/2] -> codes uint8 [..., n]: element 2j from the low nibble, 2j+1 from the high."""
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (2 * p.shape[-1],), dtype=np.uint8)
    out[..., 0::2] = p & 0xF
    out[..., 1::2] = p >> 4
    return out


def fp4_pack(codes: np.ndarray) -> np.ndarray:
    """Codes uint8 [..., n] (n even) -> uint8 [..., n/2], element 2j in the low nibble."""
    c = np.asarray(codes, dtype=np.uint8)
    return ((c[..., 0::2] & 0xF) | ((c[..., 1::2] & 0xF) << 4)).astype(np.uint8)


def mx_quantize(v: np.ndarray):
    """MX block quantisation of the last axis (a multiple of 32): returns (codes uint8 [..., n],
    scale codes uint8 [..., n/32]).  The shared exponent comes from the block maximum's
    binary exponent (exact), and v / 2**shared is exact, so only the E2M1 rounding decides."""
    v = np.asarray(v, dtype=np.float64)
    blocks = v.reshape(v.shape[:-1] + (v.shape[-1] // MX_BLOCK, MX_BLOCK))
    amax = np.abs(blocks).max(axis=-1)
    _, ex = np.frexp(amax)                  # amax = m * 2**ex, m in [0.5, 1): floor(log2) = ex - 1
    shared = np.where(amax > 0, ex - 1 - 2, 0)
    e = np.clip(shared + 127, 0, 254)
    scale = np.ldexp(1.0, e - 127)
    codes = e2m1_encode_rne_sat(blocks / scale[..., None])
    return codes.reshape(v.shape), e.astype(np.uint8)


def mx_dequantize(codes: np.ndarray, scale_codes: np.ndarray) -> np.ndarray:
    """Codes [..., n] and scale codes [..., n/32] -> float64 values."""
    vals = e2m1_decode(codes)
    return vals * np.repeat(e8m0_decode(scale_codes), MX_BLOCK, axis=-1)
