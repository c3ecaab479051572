"""FP4 E2M1 codec of the oracle.

TEST INFRASTRUCTURE ONLY.  Nothing under ``oracle/`` is part of the product:
only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import it.  It shares no code with the HIP library.

Source: the pages name NVFP4 as a low-precision communication format next to
FP8 ("GIFT: Geometry-Informed Low-precision Gradient Communication for LLM
Pretraining", abstract) and call the coordinate-system idea forward
compatible with FP4 ("GIFT 阅读笔记", summary and limitations), without
defining the format.

Reading taken here (R12 in ``oracle.gift``): the element format is the OCP
4-bit float E2M1 -- sign, 2 exponent bits with bias 1, 1 mantissa bit; the
non-negative values are 0, 0.5 (subnormal), 1, 1.5, 2, 3, 4, 6; no
infinities and no NaN.

* Rounding: to the nearest value, ties to the even code.
* Overflow: saturating; |y| >= 6 and +-Inf encode as +-6.
* NaN encodes as +0 (E2M1 has no NaN: a NaN reaches the quantiser only with
  a NaN block scale, which carries it).
* Signed zero: the sign bit is copied (-0 and negative underflow give 0x8).

Codes are 4-bit values 0..15 held one per uint8 here; ``pack`` places two per
byte, the even column in the low nibble.
"""
from __future__ import annotations

import numpy as np

FMAX = 6.0
MAX_CODE = 0x7


def code_value(code: int) -> float:
    """Value of one 4-bit code from the bit fields: e = bits 2..1,
    m = bit 0; e = 0: m * 0.5 (subnormal, 2^(1 - bias) * m / 2);
    else (1 + m / 2) * 2^(e - 1)."""
    sign = -1.0 if (code >> 3) & 1 else 1.0
    e = (code >> 1) & 0x3
    m = code & 0x1
    if e == 0:
        return sign * m * 0.5
    return sign * (1.0 + m * 0.5) * 2.0 ** (e - 1)


def value_table() -> np.ndarray:
    """float64[16]: the value of every code."""
    return np.array([code_value(c) for c in range(16)], dtype=np.float64)


def decode(codes) -> np.ndarray:
    """Codes (uint8 values 0..15, any shape) -> float64 values."""
    return value_table()[np.asarray(codes, dtype=np.uint8) & 0xF]


def encode(y) -> np.ndarray:
    """float32 values (any shape) -> uint8 codes 0..15, by bisection over
    the non-negative values: the code on the nearer side of the midpoint
    between neighbours, the even one of the two exactly at the midpoint;
    |y| at or above 6 saturates."""
    y = np.asarray(y, dtype=np.float32)
    v = value_table()[: MAX_CODE + 1]             # 0, 0.5, 1, 1.5, 2, 3, 4, 6
    with np.errstate(invalid="ignore"):           # signalling NaN patterns
        ax = np.abs(y.astype(np.float64))
    nan = np.isnan(ax)
    ax = np.where(nan, 0.0, ax)
    sat = ax >= v[MAX_CODE]
    i = np.searchsorted(v, ax, side="right") - 1   # v[i] <= ax < v[i+1]
    i = np.minimum(i, MAX_CODE - 1)
    mid = (v[i] + v[i + 1]) * 0.5
    code = np.where(ax < mid, i, i + 1)
    code = np.where(ax == mid, np.where(i % 2 == 0, i, i + 1), code)
    code = np.where(sat, MAX_CODE, code)
    sign = np.where(np.signbit(y) & ~nan, 0x8, 0)
    return (code | sign).astype(np.uint8)


def pack(codes) -> np.ndarray:
    """[m][d] codes (d even) -> [m][d/2] bytes; column 2j in the low nibble,
    2j + 1 in the high nibble."""
    c = np.asarray(codes, dtype=np.uint8)
    return (c[:, 0::2] & 0xF) | ((c[:, 1::2] & 0xF) << 4)


def unpack(packed) -> np.ndarray:
    """Inverse of ``pack``."""
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty((p.shape[0], p.shape[1] * 2), dtype=np.uint8)
    out[:, 0::2] = p & 0xF
    out[:, 1::2] = p >> 4
    return out
