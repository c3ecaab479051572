"""FP8 E4M3 / E5M2 codec of the oracle.

TEST INFRASTRUCTURE ONLY.  Nothing under ``oracle/`` is part of the product:
only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import it.  It shares no code with the HIP library.

Source: "GIFT 阅读笔记:量化用的坐标系,比量化器本身更重要" (zhongzhuzhou.org),
section 前置知识 / "FP8 到底是什么" -- an FP8 number is sign, exponent and
mantissa bits; E4M3 has 4 exponent and 3 mantissa bits (largest value about
±448), E5M2 has 5 and 2 (largest about ±57344); 256 codes in all.

What the page leaves open, and the reading taken here:

* Bit layout and bias: the OCP 8-bit formats (E4M3 "FN": bias 7, no
  infinities, 0x7F/0xFF are NaN; E5M2: bias 15, IEEE-like with Inf and NaN).
  These are the formats whose maxima are the page's 448 and 57344.
* Rounding: round to the nearest representable value, ties to the code whose
  least significant bit is 0 ("even code").
* Overflow: saturating.  Any |y| >= FMAX, including +-Inf, encodes as +-FMAX.
* NaN encodes as 0x7F with the sign bit of the input.
* Signed zero: the sign bit is copied, so -0 and negative values that round
  to zero encode as 0x80.

The encoder takes its input as float32 values (the quantiser scales in fp32
first, see ``oracle.gift.quantize``); every comparison below is exact in
float64 because float32 -> float64 is exact and midpoints between adjacent
FP8 values have at most 5 significant bits.
"""
from __future__ import annotations

import numpy as np

# Format parameters: exponent bits, mantissa bits, bias, largest finite code.
FORMATS = {
    "e4m3": dict(ebits=4, mbits=3, bias=7, max_code=0x7E),
    "e5m2": dict(ebits=5, mbits=2, bias=15, max_code=0x7B),
}
FMAX = {"e4m3": 448.0, "e5m2": 57344.0}
NAN_CODE = 0x7F


def code_value(code: int, fmt: str) -> float:
    """Value of one 8-bit code, from the bit-field definition of the format.

    Subnormal (exponent field 0): m / 2**mbits * 2**(1 - bias).
    Normal: (1 + m / 2**mbits) * 2**(e - bias).
    E4M3 has no infinities: only e=15, m=7 is NaN.  E5M2: e=31 is Inf (m=0)
    or NaN (m!=0).
    """
    p = FORMATS[fmt]
    eb, mb, bias = p["ebits"], p["mbits"], p["bias"]
    sign = -1.0 if (code >> 7) & 1 else 1.0
    e = (code >> mb) & ((1 << eb) - 1)
    m = code & ((1 << mb) - 1)
    emax_field = (1 << eb) - 1
    if fmt == "e4m3" and e == emax_field and m == (1 << mb) - 1:
        return float("nan")
    if fmt == "e5m2" and e == emax_field:
        return sign * float("inf") if m == 0 else float("nan")
    if e == 0:
        return sign * (m / (1 << mb)) * 2.0 ** (1 - bias)
    return sign * (1.0 + m / (1 << mb)) * 2.0 ** (e - bias)


def value_table(fmt: str) -> np.ndarray:
    """float64[256]: the value of every code."""
    return np.array([code_value(c, fmt) for c in range(256)], dtype=np.float64)


def decode(codes: np.ndarray, fmt: str) -> np.ndarray:
    """Codes (uint8, any shape) -> float64 values."""
    return value_table(fmt)[np.asarray(codes, dtype=np.uint8)]


def encode(y: np.ndarray, fmt: str) -> np.ndarray:
    """float32 values (any shape) -> uint8 codes, by bisection over the
    sorted table of non-negative finite values.

    For |y| between adjacent values v[i] < v[i+1] the code is the one on the
    nearer side of the midpoint (v[i] + v[i+1]) / 2; exactly at the midpoint
    it is whichever of i, i+1 is even.  |y| at or above the largest value
    saturates.
    """
    y = np.asarray(y, dtype=np.float32)
    p = FORMATS[fmt]
    max_code = p["max_code"]
    v = value_table(fmt)[: max_code + 1]          # increasing, v[0] = 0
    ax = np.abs(y.astype(np.float64))
    nan = np.isnan(ax)
    ax = np.where(nan, 0.0, ax)
    sat = ax >= v[max_code]
    i = np.searchsorted(v, ax, side="right") - 1   # v[i] <= ax < v[i+1]
    i = np.minimum(i, max_code - 1)
    lo, hi = v[i], v[i + 1]
    mid = (lo + hi) * 0.5
    code = np.where(ax < mid, i, i + 1)
    tie = ax == mid
    code = np.where(tie, np.where(i % 2 == 0, i, i + 1), code)
    code = np.where(sat, max_code, code)
    code = np.where(nan, NAN_CODE, code).astype(np.uint8)
    signbit = np.signbit(y)
    return (code | np.where(signbit, 0x80, 0).astype(np.uint8)).astype(np.uint8)
