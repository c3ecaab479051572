"""Pins of the oracle's flat-bucket Euclidean codec: one scale per tensor,
or per 512 consecutive elements of a tensor (the per-block Euclidean
baseline, block size 512, of "GIFT 阅读笔记", experiment setup; reading R13).

Payloads are built so that every step is exact (block maxima at FMAX times a
power of two), so a wrong block size, a block that does not restart at a
tensor boundary, or a scale taken from the wrong block fails.
"""
import numpy as np
import pytest

from oracle import gift as G


def _e4m3_finite_values():
    """Non-negative finite E4M3 values from the bit layout (bias 7, 3
    mantissa bits; exponent 15 with mantissa 7 is NaN)."""
    v = [m * 2.0 ** -9 for m in range(8)]
    v += [(8 + m) * 2.0 ** (e - 10) for e in range(1, 16) for m in range(8) if not (e == 15 and m == 7)]
    return np.array(v)


def _exact_tensor(n, js, rng):
    """n elements in blocks of 512: block b holds E4M3 values times 2^js[b],
    one of them +-448 * 2^js[b]; returns (x, expected scale per block)."""
    vals = _e4m3_finite_values()
    x = np.empty(n, np.float32)
    for b, j in enumerate(js):
        seg = slice(512 * b, min(n, 512 * b + 512))
        k = seg.stop - seg.start
        v = rng.choice(vals[vals <= 448], k) * rng.choice([-1.0, 1.0], k)
        v[k // 2] = 448.0 * (1 if b % 2 == 0 else -1)
        x[seg] = v * 2.0 ** j
    return x, np.array([2.0 ** j for j in js], np.float32)


def test_block512_exact():
    rng = np.random.default_rng(1)
    n = 3 * 700                                   # 4 full blocks and one of 52
    js = [-3, 5, 0, -12, 7]
    x, want_s = _exact_tensor(n, js, rng)
    c, s, am = G.quantize_flat(x.reshape(3, 700), "e4m3", 512)
    assert np.array_equal(s, want_s)
    assert np.array_equal(am, 448.0 * want_s.astype(np.float64))
    assert np.array_equal(G.dequantize_flat(c, s, "e4m3", 512), x.astype(np.float64))


def test_blocks_restart_at_each_tensor():
    """Tensor 2's first block is its own first 512 elements, not the flat
    bucket's elements 512..1023; it does not see tensor 1's amax."""
    rng = np.random.default_rng(2)
    t1 = rng.standard_normal(700).astype(np.float32)
    t1[650] = 1e4
    t2 = rng.standard_normal(300).astype(np.float32)
    c, s, _ = G.bucket_quantize([t1, t2], "e4m3", 512)
    assert c.size == 1000 and s.size == 3
    c2, s2, _ = G.quantize_flat(t2, "e4m3", 512)
    assert np.array_equal(c[700:], c2) and s[2] == s2[0]
    assert s[1] == np.float32(1e4 / 448.0)


def test_tensor_scaling_matches_the_2d_quantiser():
    rng = np.random.default_rng(3)
    ts = [rng.standard_normal((24, 40)).astype(np.float32) * 10 ** k for k in (-2, 0, 3)]
    c, s, _ = G.bucket_quantize(ts, "e5m2")
    off = 0
    for i, t in enumerate(ts):
        cq, sq, _ = G.quantize(t, "e5m2", "tensor")
        assert np.array_equal(c[off:off + t.size], cq.ravel()) and s[i] == sq[0, 0]
        off += t.size


def test_shared_amax_twice_the_local_one():
    """With a shared amax 2a instead of the local a (a power-of-two factor),
    every normal code moves down one binade (code - 8) and the scale
    doubles."""
    rng = np.random.default_rng(4)
    x = (rng.standard_normal(1024) * 3).astype(np.float32)
    c, s, am = G.quantize_flat(x, "e4m3", 512)
    c2, s2, _ = G.quantize_flat(x, "e4m3", 512, amax_in=2 * am)
    assert np.array_equal(s2, 2 * s)
    mag, mag2 = c & 0x7F, c2 & 0x7F
    normal = mag >= 16                             # still normal one binade down
    assert np.array_equal(mag2[normal], mag[normal] - 8)
    assert np.array_equal(c2 & 0x80, c & 0x80)


@pytest.mark.parametrize("R", [1, 2, 4])
def test_reduce_of_identical_payloads_is_exact(R):
    rng = np.random.default_rng(5)
    ts = [rng.standard_normal(n).astype(np.float32) for n in (512, 1000, 64)]
    c, s, _ = G.bucket_quantize(ts, "e4m3", 512)
    U = G.bucket_dequant_reduce([c] * R, [s] * R, [t.size for t in ts], "e4m3", 512)
    one = np.concatenate([G.dequantize_flat(*G.quantize_flat(t, "e4m3", 512)[:2], "e4m3", 512) for t in ts])
    assert np.array_equal(U, one)
