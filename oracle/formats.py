"""Number formats, written out from their bit-level definitions.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The method's description ("EpiLoRA: Fusing Many LoRA Adapters into
Low-Precision GEMMs for Serving and RL", Introduction and Design section
"Multi-adapter kernels") names its formats only as "FP8", "NVFP4" and
"block-scaled 4-bit formats".  The definitions used here are the public ones:

* bf16: the upper 16 bits of an IEEE-754 binary32 value.
* FP8 E4M3FN (OCP 8-bit floating point specification): 1 sign bit, 4
  exponent bits with bias 7, 3 mantissa bits; exponent 0 is subnormal;
  S.1111.111 is NaN; there is no infinity; the largest finite value is 448.
* E2M1 (OCP Microscaling formats, the element type of NVFP4): 1 sign bit,
  2 exponent bits with bias 1, 1 mantissa bit; magnitudes
  0, 0.5, 1, 1.5, 2, 3, 4, 6.

Every table is built by evaluating these definitions code by code.
"""

import numpy as np

# ---------------------------------------------------------------------------
# bf16
# ---------------------------------------------------------------------------


def bf16_to_f32(bits):
    """bf16 bit patterns (uint16) -> float32, exactly (the bits become the
    upper half of a binary32 word)."""
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def f32_to_bf16(v):
    """float32 -> bf16 bit patterns, round to nearest, ties to even.

    Finite inputs only (the layer's outputs are finite for finite inputs)."""
    u = np.asarray(v, dtype=np.float32).view(np.uint32).astype(np.uint64)
    upper = u >> np.uint64(16)
    lower = u & np.uint64(0xFFFF)
    half = np.uint64(0x8000)
    up = (lower > half) | ((lower == half) & ((upper & np.uint64(1)) == 1))
    return (upper + up.astype(np.uint64)).astype(np.uint16)


# ---------------------------------------------------------------------------
# FP8 E4M3FN
# ---------------------------------------------------------------------------


def _e4m3_value(code):
    sign = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return sign * (m / 8.0) * 2.0 ** -6  # subnormal
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)


_E4M3 = np.array([_e4m3_value(c) for c in range(256)], dtype=np.float64)
# Magnitudes of codes 0x00..0x7E grow strictly with the code (0 .. 448).
_E4M3_POS = _E4M3[:0x7F].copy()
E4M3_MAX = float(_E4M3_POS[-1])  # 448


def e4m3_decode_table():
    """float64[256]: the value of every E4M3FN code (NaN for 0x7F, 0xFF)."""
    return _E4M3.copy()


def e4m3_decode(codes):
    """uint8 codes -> float64 values."""
    return _E4M3[np.asarray(codes, dtype=np.uint8)]


def e4m3_encode(v):
    """float32 -> E4M3FN code: the nearest finite E4M3 value, ties to the
    code whose mantissa LSB is 0, magnitudes at or above 448 saturated to
    448, the sign kept (so -0.0 -> 0x80).  NaN inputs are rejected.

    The choice between the two neighbouring codes is made by comparing the
    input with their midpoint; every E4M3 midpoint has at most 5
    significant bits, so the comparison is exact."""
    v = np.asarray(v, dtype=np.float32)
    if np.isnan(v).any():
        raise ValueError("e4m3_encode: NaN input")
    a = np.abs(v).astype(np.float64)
    lo = np.searchsorted(_E4M3_POS, a, side="right") - 1  # largest code <= a
    lo = np.clip(lo, 0, 0x7E)
    hi = np.minimum(lo + 1, 0x7E)
    mid = (_E4M3_POS[lo] + _E4M3_POS[hi]) * 0.5
    pick_hi = (a > mid) | ((a == mid) & (lo % 2 == 1))
    code = np.where(lo >= 0x7E, 0x7E, np.where(pick_hi, hi, lo))
    sign = np.signbit(v).astype(np.uint8) << np.uint8(7)
    return (code.astype(np.uint8) | sign).astype(np.uint8)


# ---------------------------------------------------------------------------
# E2M1 (4-bit)
# ---------------------------------------------------------------------------


def _e2m1_value(code):
    sign = -1.0 if code & 0x8 else 1.0
    e = (code >> 1) & 0x3
    m = code & 0x1
    if e == 0:
        return sign * m * 0.5  # subnormal: 0 or 0.5
    return sign * (1.0 + m / 2.0) * 2.0 ** (e - 1)


_E2M1 = np.array([_e2m1_value(c) for c in range(16)], dtype=np.float64)
_E2M1_POS = _E2M1[:8].copy()  # 0, .5, 1, 1.5, 2, 3, 4, 6


def e2m1_decode_table():
    """float64[16]: the value of every E2M1 code (bit 3 is the sign)."""
    return _E2M1.copy()


def e2m1_encode(v):
    """float32 -> E2M1 code (uint8 in 0..15): nearest value, ties to the
    even code, magnitudes at or above 6 saturated to 6, the sign kept."""
    v = np.asarray(v, dtype=np.float32)
    if np.isnan(v).any():
        raise ValueError("e2m1_encode: NaN input")
    a = np.abs(v).astype(np.float64)
    lo = np.searchsorted(_E2M1_POS, a, side="right") - 1
    lo = np.clip(lo, 0, 7)
    hi = np.minimum(lo + 1, 7)
    mid = (_E2M1_POS[lo] + _E2M1_POS[hi]) * 0.5
    pick_hi = (a > mid) | ((a == mid) & (lo % 2 == 1))
    code = np.where(lo >= 7, 7, np.where(pick_hi, hi, lo))
    sign = np.signbit(v).astype(np.uint8) << np.uint8(3)
    return (code.astype(np.uint8) | sign).astype(np.uint8)


# ---------------------------------------------------------------------------
# The fold of a 4-bit code and its block scale into one FP8 byte
# ---------------------------------------------------------------------------

FOLD_SHIFT = 3  # the fold pre-scales by 2**-3; the GEMM multiplies by 2**3


_FOLD = None


def fold_table():
    """uint8[16][256]: T[c][b] = E4M3( e2m1(c) * e4m3(b) * 2**-3 ).

    This is the reading of a 4-bit weight that the GEMM decodes to one FP8
    byte before its FP8 matrix-core product: the block scale is folded into
    the code and the product rounded once to E4M3.  The product and the 2**-3 are exact in
    fp32 (at most 6 significant bits, no overflow or underflow), so only
    the final encode rounds.  2**-3 is the smallest power-of-two pre-scale
    for which the largest product (6 * 448 = 2688) stays below 448.
    A NaN block scale (0x7F, 0xFF) gives the NaN code 0x7F."""
    global _FOLD
    if _FOLD is not None:
        return _FOLD.copy()
    t = np.zeros((16, 256), dtype=np.uint8)
    for c in range(16):
        for b in range(256):
            sb = _E4M3[b]
            if np.isnan(sb):
                t[c, b] = 0x7F
                continue
            p = np.float32(_E2M1[c]) * np.float32(sb) * np.float32(2.0 ** -FOLD_SHIFT)
            t[c, b] = e4m3_encode(np.float32(p))
    _FOLD = t
    return t.copy()
