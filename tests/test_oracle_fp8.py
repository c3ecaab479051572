"""Pins of the oracle's FP8 codec against the format definitions.

GIFT 阅读笔记, §前置知识 "FP8 到底是什么": E4M3 = 4 exponent / 3 mantissa
bits, largest value 448; E5M2 = 5 / 2, largest 57344; 256 codes.  The
reference definitions here are built differently from the oracle (explicit
value sets, and rounding by arithmetic instead of bisection), so a wrong
bias, a shifted table or a wrong tie rule in the oracle fails one of them.
"""
import numpy as np
import pytest
import torch

from oracle import fp8

FMTS = ("e4m3", "e5m2")


def _value_set(fmt):
    """Finite non-negative values from the definition, as a sorted list of
    (value, code): subnormals m * 2^(1-bias-mbits), normals
    (2^mbits + m) * 2^(e-bias-mbits)."""
    eb, mb, bias = (4, 3, 7) if fmt == "e4m3" else (5, 2, 15)
    out = []
    for m in range(1 << mb):
        out.append((m * 2.0 ** (1 - bias - mb), m))
    emax = (1 << eb) - 1
    for e in range(1, emax + 1):
        for m in range(1 << mb):
            if fmt == "e4m3" and e == emax and m == (1 << mb) - 1:
                continue          # NaN
            if fmt == "e5m2" and e == emax:
                continue          # Inf / NaN
            out.append(((2 ** mb + m) * 2.0 ** (e - bias - mb), (e << mb) | m))
    return out


@pytest.mark.parametrize("fmt", FMTS)
def test_all_256_codes_decode(fmt):
    vs = _value_set(fmt)
    tab = fp8.value_table(fmt)
    assert len(tab) == 256
    for v, c in vs:
        assert tab[c] == v
        assert tab[c | 0x80] == -v or (v == 0 and tab[c | 0x80] == 0 and np.signbit(tab[c | 0x80]))
    finite = np.isfinite(tab)
    assert finite.sum() == 2 * len(vs)
    # format constants printed on the page
    assert tab[fp8.FORMATS[fmt]["max_code"]] == fp8.FMAX[fmt]
    assert fp8.FMAX[fmt] == (448.0 if fmt == "e4m3" else 57344.0)
    assert np.isnan(tab[0x7F]) and np.isnan(tab[0xFF])
    if fmt == "e5m2":
        assert tab[0x7C] == np.inf and tab[0xFC] == -np.inf
    else:
        assert np.isinf(tab).sum() == 0
    # increasing in the code over the finite non-negative range
    pos = tab[: fp8.FORMATS[fmt]["max_code"] + 1]
    assert np.all(np.diff(pos) > 0)


@pytest.mark.parametrize("fmt", FMTS)
def test_encode_decode_identity(fmt):
    tab = fp8.value_table(fmt)
    codes = np.array([c for c in range(256) if np.isfinite(tab[c])], dtype=np.uint8)
    y = tab[codes].astype(np.float32)
    assert np.array_equal(fp8.encode(y, fmt), codes)


@pytest.mark.parametrize("fmt", FMTS)
def test_midpoints_ties_and_neighbours(fmt):
    vs = [v for v, _ in _value_set(fmt)]
    ys, want = [], []
    for i in range(len(vs) - 1):
        lo, hi = vs[i], vs[i + 1]
        mid = np.float32((lo + hi) / 2)
        assert float(mid) == (lo + hi) / 2          # midpoints are exact in fp32
        even = i if i % 2 == 0 else i + 1           # code i equals position i here
        ys += [mid, np.nextafter(mid, np.float32(0)), np.nextafter(mid, np.float32(np.inf))]
        want += [even, i, i + 1]
    ys = np.array(ys, dtype=np.float32)
    got = fp8.encode(ys, fmt)
    codes = [c for _, c in _value_set(fmt)]
    assert np.array_equal(got, np.array([codes[w] for w in want], dtype=np.uint8))
    assert np.array_equal(fp8.encode(-ys, fmt), got | 0x80)


def test_named_cases_e4m3():
    e = lambda v: int(fp8.encode(np.array([v], np.float32), "e4m3")[0])
    assert e(7.5 * 2 ** -9) == 0x08          # subnormal/normal midpoint -> even code 8
    assert e(2 ** -10) == 0x00               # half the smallest subnormal -> 0 (even)
    assert e(np.nextafter(np.float32(2 ** -10), np.float32(1))) == 0x01
    assert e(-2 ** -12) == 0x80              # negative underflow keeps the sign
    assert e(-0.0) == 0x80 and e(0.0) == 0x00
    assert e(448.0) == 0x7E and e(464.0) == 0x7E and e(1e30) == 0x7E
    assert e(np.inf) == 0x7E and e(-np.inf) == 0xFE
    assert e(np.nan) == 0x7F
    assert e(1.0) == 0x38


def test_named_cases_e5m2():
    e = lambda v: int(fp8.encode(np.array([v], np.float32), "e5m2")[0])
    assert e(2 ** -17) == 0x00
    assert e(57344.0) == 0x7B and e(61440.0) == 0x7B and e(np.inf) == 0x7B
    assert e(1.0) == 0x3C
    assert e(-np.inf) == 0xFB


@pytest.mark.parametrize("fmt", FMTS)
def test_against_arithmetic_definition_sampled(fmt):
    rng = np.random.default_rng(1)
    bits = np.concatenate([
        np.arange(0, 1 << 32, 104729, dtype=np.uint64).astype(np.uint32),
        rng.integers(0, 1 << 32, 200000, dtype=np.uint64).astype(np.uint32),
    ])
    y = bits.view(np.float32)
    assert np.array_equal(fp8.encode(y, fmt), _arith_encode_fast(y, fmt))


@pytest.mark.parametrize("fmt,tdt", [("e4m3", torch.float8_e4m3fn), ("e5m2", torch.float8_e5m2)])
def test_against_torch_cast_in_range(fmt, tdt):
    """torch's CPU float8 casts round to nearest even but do not saturate,
    so only |y| < FMAX is compared."""
    rng = np.random.default_rng(2)
    y = (rng.standard_normal(300000) * rng.choice([1e-4, 1e-2, 1, 30, 300], 300000)).astype(np.float32)
    y = y[np.abs(y) < fp8.FMAX[fmt]]
    got = fp8.encode(y, fmt)
    ref = torch.from_numpy(y).to(tdt).view(torch.uint8).numpy()
    assert np.array_equal(got, ref)


def _sweep_chunk(args):
    fmt, start, n = args
    y = np.arange(start, start + n, dtype=np.uint64).astype(np.uint32).view(np.float32)
    return bool(np.array_equal(fp8.encode(y, fmt), _arith_encode_fast(y, fmt)))


def _arith_encode_fast(y, fmt):
    eb, mb, bias = (4, 3, 7) if fmt == "e4m3" else (5, 2, 15)
    fmax = fp8.FMAX[fmt]
    vs = _value_set(fmt)
    vals = np.array([v for v, _ in vs])
    cds = np.array([c for _, c in vs], dtype=np.uint8)
    ax = np.abs(y.astype(np.float64))
    mant, ex = np.frexp(ax)
    e = np.maximum(ex - 1, 1 - bias)
    q = np.ldexp(1.0, e - mb)
    val = np.minimum(np.rint(ax / q) * q, fmax)
    val = np.where(ax >= fmax, fmax, val)
    idx = np.searchsorted(vals, np.nan_to_num(val))
    c = cds[np.minimum(idx, len(vals) - 1)]
    c = np.where(np.isnan(ax), 0x7F, c).astype(np.uint8)
    return c | np.where(np.signbit(y), 0x80, 0).astype(np.uint8)


@pytest.mark.slow
@pytest.mark.parametrize("fmt", FMTS)
def test_exhaustive_all_fp32(fmt):
    """Every one of the 2^32 float32 bit patterns (long: run with -m slow)."""
    from multiprocessing import Pool
    n = 1 << 24
    with Pool(8) as p:
        ok = p.map(_sweep_chunk, [(fmt, s, n) for s in range(0, 1 << 32, n)])
    assert all(ok)
