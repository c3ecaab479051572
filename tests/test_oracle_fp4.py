"""Pins of the oracle's FP4 payload (E2M1 elements, 16-element block scales
in E4M3, one fp32 tensor scale) against the format definition and the
mathematics of the two-level scale.

The pages name NVFP4 as a communication format ("GIFT: Geometry-Informed
Low-precision Gradient Communication for LLM Pretraining", abstract) and
call the method forward compatible with FP4 ("GIFT 阅读笔记", summary);
the format itself is the reading R12 of ``oracle.gift``.  The references
here are built differently from the oracle (explicit value lists, rounding
by arithmetic, payloads constructed so that every step is exact), so a wrong
bias, tie rule, nibble order, block size or scale constant fails one of them.
"""
import numpy as np
import pytest

from oracle import fp4, fp8
from oracle import gift as G

# OCP E2M1: the eight non-negative values in code order
E2M1 = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def test_all_16_codes_decode():
    want = E2M1 + [-v for v in E2M1]
    got = fp4.decode(np.arange(16, dtype=np.uint8))
    assert np.array_equal(got, np.array(want))
    assert np.signbit(got[8]) and not np.signbit(got[0])


def test_encode_decode_identity():
    c = np.arange(16, dtype=np.uint8)
    assert np.array_equal(fp4.encode(fp4.decode(c).astype(np.float32)), c)


def test_midpoints_ties_and_neighbours():
    """Exactly between two values the even code wins; one float32 step off
    the midpoint goes to the nearer value.  Both signs."""
    for i in range(7):
        lo, hi = E2M1[i], E2M1[i + 1]
        mid = np.float32((lo + hi) / 2)
        even = i if i % 2 == 0 else i + 1
        for sgn, sb in ((1, 0), (-1, 8)):
            e = lambda v: int(fp4.encode(np.array([sgn * v], np.float32))[0])
            assert e(mid) == even | sb, (lo, hi)
            assert e(np.nextafter(mid, np.float32(np.inf))) == (i + 1) | sb
            assert e(np.nextafter(mid, np.float32(0))) == i | sb


def test_named_cases():
    e = lambda v: int(fp4.encode(np.array([v], np.float32))[0])
    assert e(6.0) == 0x7 and e(7.9) == 0x7 and e(1e30) == 0x7 and e(np.inf) == 0x7
    assert e(-np.inf) == 0xF and e(-6.5) == 0xF
    assert e(np.nan) == 0x0                    # no NaN code: +0
    assert e(-0.0) == 0x8 and e(-0.2) == 0x8   # sign kept on underflow
    assert e(0.25) == 0x0 and e(0.75) == 0x2 and e(1.25) == 0x2 and e(1.75) == 0x4
    assert e(2.5) == 0x4 and e(3.5) == 0x6 and e(5.0) == 0x6 and e(5.01) == 0x7


def _arith_encode(y):
    """Round |y| to a multiple of the spacing of its binade (0.5 below 2,
    then 2^(e-1) in [2^e, 2^(e+1))) with numpy's half-to-even rint, clamp at
    6, and find the code by value."""
    y = np.asarray(y, dtype=np.float32)
    with np.errstate(invalid="ignore"):
        a = np.abs(y.astype(np.float64))
    nan = np.isnan(a)
    a = np.where(nan, 0.0, a)
    _, ex = np.frexp(a)
    e = np.maximum(ex - 1, 0)                 # binade exponent, subnormals share binade 0
    q = np.ldexp(1.0, e - 1)
    val = np.minimum(np.rint(a / q) * q, 6.0)
    val = np.where(a >= 6.0, 6.0, val)
    code = np.searchsorted(np.array(E2M1), val)
    sign = np.where(np.signbit(y) & ~nan, 8, 0)
    return (code | sign).astype(np.uint8)


def test_against_arithmetic_definition_sampled():
    rng = np.random.default_rng(1)
    bits = np.concatenate([
        np.arange(0, 1 << 32, 104729, dtype=np.uint64).astype(np.uint32),
        rng.integers(0, 1 << 32, 200000, dtype=np.uint64).astype(np.uint32),
    ])
    y = bits.view(np.float32)
    dense = np.linspace(-7, 7, 200001).astype(np.float32)
    for v in (y, dense):
        assert np.array_equal(fp4.encode(v), _arith_encode(v))


def _sweep_chunk(args):
    start, n = args
    y = np.arange(start, start + n, dtype=np.uint64).astype(np.uint32).view(np.float32)
    return bool(np.array_equal(fp4.encode(y), _arith_encode(y)))


@pytest.mark.slow
def test_exhaustive_all_fp32():
    """Every one of the 2^32 float32 bit patterns (long: run with -m slow)."""
    from multiprocessing import Pool
    n = 1 << 24
    with Pool(8) as p:
        ok = p.map(_sweep_chunk, [(s, n) for s in range(0, 1 << 32, n)])
    assert all(ok)


def test_pack_nibble_order():
    c = np.array([[1, 2, 3, 4, 0xF, 0x8]], dtype=np.uint8)
    assert np.array_equal(fp4.pack(c), np.array([[0x21, 0x43, 0x8F]], dtype=np.uint8))
    rng = np.random.default_rng(3)
    c = rng.integers(0, 16, (5, 64)).astype(np.uint8)
    assert np.array_equal(fp4.unpack(fp4.pack(c)), c)


def _e4m3_code_of_pow2(j):
    """E4M3 code of 2^j from the bit layout: normal (j >= -6) exponent field
    j + 7, mantissa 0; subnormal 2^j = m 2^-9, m = 2^(j + 9)."""
    return (j + 7) << 3 if j >= -6 else 1 << (j + 9)


def test_round_trip_exact_two_level():
    """A payload built to be exact: the tensor amax is 6 * 448 (tensor scale
    g = 1), every 16-element block holds E2M1 values times 2^j_b with one
    entry at +-6 * 2^j_b (block scale exactly 2^j_b), one block at 448.
    Quantising must return those codes and block scales, and dequantising
    must return the tensor bit for bit."""
    rng = np.random.default_rng(4)
    m, d = 3, 96
    nbk = d // 16
    codes = rng.integers(0, 16, (m, d)).astype(np.uint8)
    js = rng.integers(-9, 9, (m, nbk))
    js[1, 2] = 99                               # the 448 block
    X = np.empty((m, d), np.float32)
    want_sc = np.empty((m, nbk), np.uint8)
    for i in range(m):
        for b in range(nbk):
            sl = slice(16 * b, 16 * b + 16)
            codes[i, 16 * b + (b % 16)] = 0x7 | (8 if (i + b) % 2 else 0)   # the block's +-6
            scale = 448.0 if js[i, b] == 99 else 2.0 ** js[i, b]
            want_sc[i, b] = 0x7E if js[i, b] == 99 else _e4m3_code_of_pow2(int(js[i, b]))
            X[i, sl] = np.array([E2M1[c & 7] * (-1 if c & 8 else 1) for c in codes[i, sl]]) * scale
    out = G.quantize_fp4(X)
    assert out["tscale"] == np.float32(1.0)
    # -0 codes come back as +0 only where the value is zero: compare values and nonzero codes
    nz = (codes & 7) != 0
    assert np.array_equal(out["codes"][nz], codes[nz])
    assert np.array_equal(out["bscales"], want_sc)
    back = G.dequantize_fp4(out["codes"], out["bscales"], out["tscale"])
    assert np.array_equal(back, X.astype(np.float64))


def test_power_of_two_invariance():
    """Scaling the tensor by 2^k scales only the tensor scale, by 2^k
    exactly: codes and block scales are relative to the tensor amax."""
    rng = np.random.default_rng(5)
    X = (rng.standard_t(3, (16, 128)) * np.arange(1, 129) ** -1.0).astype(np.float32)
    base = G.quantize_fp4(X)
    for k in (-20, -3, 4, 30):
        o = G.quantize_fp4((X * np.float32(2.0 ** k)).astype(np.float32))
        assert np.array_equal(o["codes"], base["codes"]) and np.array_equal(o["bscales"], base["bscales"])
        assert o["tscale"] == np.float32(base["tscale"] * 2.0 ** k)


def _half_spacing(y):
    a = np.abs(y)
    return np.where(a <= 2, 0.25, np.where(a <= 4, 0.5, 1.0))


def test_error_bound():
    """Every element is within half an E2M1 spacing (at y = x / S_b) of its
    dequantised value, times S_b, or saturated at 6 S_b; plus the float32
    roundings of y and 1 / S_b."""
    rng = np.random.default_rng(6)
    X = (rng.standard_t(3, (64, 512)) * np.arange(1, 513) ** -1.5).astype(np.float32)
    X[:, 7] *= 100.0                             # an outlier column
    o = G.quantize_fp4(X)
    S = np.repeat(G.fp4_block_scales(o["bscales"], o["tscale"]).astype(np.float64), 16, axis=1)
    x = X.astype(np.float64)
    deq = G.dequantize_fp4(o["codes"], o["bscales"], o["tscale"])
    y = x / np.where(S > 0, S, 1.0)
    room = np.where(np.abs(y) > 6.0, np.abs(y) - 6.0, _half_spacing(y))
    bound = S * room + 2.0 ** -22 * np.abs(x)
    assert np.all(np.abs(x - deq) <= bound)
    # the block amax lands in the top two codes when the block scale is normal in E4M3
    amax_code = np.take_along_axis(o["codes"].reshape(64, 32, 16) & 7,
                                   np.abs(X).reshape(64, 32, 16).argmax(axis=2)[:, :, None], axis=2)[:, :, 0]
    normal = (o["bscales"] & 0x78) != 0
    assert np.all(amax_code[normal] >= 6)


def test_block_independence_along_rows():
    """Blocks are 16 consecutive columns of one row: shrinking block 1 of
    row 0 leaves every other block's codes and scale unchanged (the tensor
    amax is elsewhere)."""
    rng = np.random.default_rng(7)
    X = rng.standard_normal((4, 64)).astype(np.float32)
    X[3, 40] = 50.0
    a = G.quantize_fp4(X)
    Y = X.copy()
    Y[0, 16:32] *= np.float32(0.01)
    b = G.quantize_fp4(Y)
    keep = np.ones((4, 64), bool)
    keep[0, 16:32] = False
    assert np.array_equal(a["codes"][keep], b["codes"][keep])
    ks = np.ones((4, 4), bool)
    ks[0, 1] = False
    assert np.array_equal(a["bscales"][ks], b["bscales"][ks]) and a["bscales"][0, 1] != b["bscales"][0, 1]


def test_zero_and_nonfinite():
    z = G.quantize_fp4(np.zeros((2, 32), np.float32))
    assert z["tscale"] == 0 and not z["codes"].any() and not z["bscales"].any()
    X = np.ones((2, 32), np.float32)
    for bad in (np.nan, np.inf):
        Y = X.copy()
        Y[1, 20] = bad
        o = G.quantize_fp4(Y)
        assert np.isnan(o["tscale"]) and np.all(o["bscales"] == 0x7F) and not o["codes"].any()
        assert np.all(np.isnan(G.dequantize_fp4(o["codes"], o["bscales"], o["tscale"])))
    # a finite shared amax with a local Inf: that block saturates, the rest are ordinary
    Y = X.copy()
    Y[1, 20] = np.inf
    o = G.quantize_fp4(Y, amax_in=np.float32(4.0))
    assert o["bscales"][1, 1] == 0x7E and o["codes"][1, 20] == 0x7
    p = G.quantize_fp4(X, amax_in=np.float32(4.0))
    assert np.array_equal(o["codes"][0], p["codes"][0])
    # -0 keeps its sign
    Y = X.copy()
    Y[0, 3] = -0.0
    assert G.quantize_fp4(Y)["codes"][0, 3] == 0x8


def test_payload_bytes():
    assert G.payload_bytes(4096, 16384, "block16") == 4096 * 16384 // 2 + 4096 * 1024 + 4


def _ef_steps_fp4(steps=4):
    rng = np.random.default_rng(8)
    m, d = 24, 96
    R = np.zeros((m, d), np.float32)
    outs = []
    for t in range(steps):
        W = (rng.standard_t(3, (m, d)) * np.arange(1, d + 1) ** -0.5).astype(np.float32)
        e = G.error_feedback_fp4(W, R)
        outs.append((W, e))
        R = e["residual"]
    return outs


def test_error_feedback_fp4_telescopes():
    """sum_t deq_t + R_T = sum_t W_t up to the float32 roundings of U~ and R
    (bounded elementwise), and far from it without the residual."""
    outs = _ef_steps_fp4()
    sum_deq = sum(G.dequantize_fp4(e["codes"], e["bscales"], e["tscale"]) for _, e in outs)
    sum_w = sum(W.astype(np.float64) for W, _ in outs)
    gap = np.abs(sum_deq + outs[-1][1]["residual"].astype(np.float64) - sum_w)
    bound = sum(2.0 ** -24 * (np.abs(e["u_tilde"]) + np.abs(e["residual"])) for _, e in outs)
    assert np.all(gap <= bound + 2.0 ** -50 * np.abs(sum_w))
    no_ef = sum(G.dequantize_fp4(*(lambda o: (o["codes"], o["bscales"], o["tscale"]))(G.quantize_fp4(W)))
                for W, _ in outs)
    assert np.linalg.norm(no_ef - sum_w) > 1e3 * np.linalg.norm(gap)


def test_error_feedback_fp4_first_step_is_plain():
    W = (np.random.default_rng(9).standard_normal((8, 32))).astype(np.float32)
    e = G.error_feedback_fp4(W, np.zeros_like(W))
    p = G.quantize_fp4(W)
    assert np.array_equal(e["codes"], p["codes"]) and np.array_equal(e["bscales"], p["bscales"])
    assert e["tscale"] == p["tscale"]
