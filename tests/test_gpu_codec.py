"""GPU FP8 codec and quantiser against the oracle (bit-exact).

Pages: GIFT 阅读笔记, §前置知识 FP8 (formats, s = amax / FP8_MAX) and
Algorithm 1 (Scale, Q, Dequantize).  The quantiser is fed the oracle's own
fp32 tensor through the Euclidean path, so codes and scales must be
identical.
"""
import numpy as np
import pytest
import torch

from oracle import fp8
from oracle import gift as G

pytestmark = pytest.mark.gpu
DEV = "cuda"
FMTS = [("e4m3", 0), ("e5m2", 1)]


@pytest.fixture(scope="module")
def fw():
    import fac_whitening_amd as fw
    yield fw
    fw.set_fused(True)


def _euclid(fw, m, d):
    return fw.Layer(m, d, "euclid", device=DEV)


@pytest.mark.parametrize("fmt,f", FMTS)
@pytest.mark.parametrize("fused", [True, False])
def test_decode_all_256_codes(fw, fmt, f, fused):
    print(f"[decode all codes {fmt} fused={fused}]", flush=True)
    fw.set_fused(fused)
    L = _euclid(fw, 2, 128)
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8).reshape(2, 128).to(DEV)
    scales = torch.ones(1, 1, dtype=torch.float32, device=DEV)
    out = L.decode_reduce(codes.unsqueeze(0), scales, f, fw.SCALE_TENSOR).cpu().numpy().ravel()
    ref = fp8.value_table(fmt)
    assert np.array_equal(np.isnan(out), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(out[ok], ref[ok].astype(np.float32))
    assert np.array_equal(np.signbit(out[ok]), np.signbit(ref[ok]))


@pytest.mark.parametrize("fmt,f", FMTS)
def test_encode_bit_patterns_unit_scale(fw, fmt, f):
    """amax_in = FMAX makes r = 1 exactly, so the codes are the encoder
    applied to the raw values: 2^22 random fp32 bit patterns (NaN payloads
    excluded; Inf kept) plus every midpoint between adjacent values."""
    print(f"[encode bit patterns {fmt}]", flush=True)
    rng = np.random.default_rng(20)
    bits = rng.integers(0, 1 << 32, 1 << 22, dtype=np.uint64).astype(np.uint32)
    nan = ((bits >> 23) & 0xFF == 0xFF) & (bits & 0x7FFFFF != 0)
    bits[nan] = 0
    v = fp8.value_table(fmt)[: fp8.FORMATS[fmt]["max_code"] + 1]
    mids = ((v[:-1] + v[1:]) / 2).astype(np.float32)
    extra = np.concatenate([mids, -mids, np.nextafter(mids, np.float32(0)), np.nextafter(mids, np.float32(1e9)),
                            v.astype(np.float32), np.array([np.inf, -np.inf, 0.0, -0.0], np.float32)])
    y = np.concatenate([bits.view(np.float32), extra])
    n = -(-y.size // 1024) * 1024
    y = np.concatenate([y, np.zeros(n - y.size, np.float32)]).reshape(-1, 1024)
    L = _euclid(fw, y.shape[0], 1024)
    W = torch.from_numpy(y).to(DEV)
    amax_in = torch.full((1,), fp8.FMAX[fmt], dtype=torch.float32, device=DEV)
    codes, scales = L.encode(W, f, fw.SCALE_TENSOR, amax_in=amax_in)
    assert float(scales.item()) == 1.0
    assert np.array_equal(codes.cpu().numpy(), fp8.encode(y, fmt))


@pytest.mark.parametrize("fmt,f", FMTS)
@pytest.mark.parametrize("scaling,s", [("tensor", 0), ("block", 1)])
@pytest.mark.parametrize("shape", [(64, 256), (200, 328), (257, 1032)])
def test_quantizer_bit_exact_on_oracle_tensor(fw, fmt, f, scaling, s, shape):
    print(f"[quantizer {fmt} {scaling} {shape}]", flush=True)
    m, d = shape
    rng = np.random.default_rng(hash(shape) % 1000)
    X = (rng.standard_normal((m, d)) * np.exp(2.0 * rng.standard_normal((m, d)))
         * np.exp(3.0 * rng.standard_normal((1, d)))).astype(np.float32)
    X[3, :7] = 0.0
    X[5, 1] = -0.0
    codes_ref, scales_ref, am_ref = G.quantize(X, fmt, scaling)
    L = _euclid(fw, m, d)
    W = torch.from_numpy(X).to(DEV)
    nb = fw.nblocks(m, d, s)
    amax_out = torch.empty(nb, dtype=torch.float32, device=DEV)
    whit = torch.empty(m, d, dtype=torch.float32, device=DEV)
    codes, scales = L.encode(W, f, s, amax_out=amax_out, whitened=whit)
    assert np.array_equal(whit.cpu().numpy(), X)
    assert np.array_equal(scales.cpu().numpy(), scales_ref.ravel())
    assert np.array_equal(amax_out.cpu().numpy(), am_ref.ravel().astype(np.float32))
    assert np.array_equal(codes.cpu().numpy(), codes_ref)
    # amax-only mode writes the same local amax and no codes
    amax2 = torch.zeros(nb, dtype=torch.float32, device=DEV)
    L.encode(W, f, s, amax_out=amax2, want_codes=False)
    assert np.array_equal(amax2.cpu().numpy(), am_ref.ravel().astype(np.float32))


def test_quantizer_zero_and_nonfinite(fw):
    print("[quantizer zero / non-finite]", flush=True)
    L = _euclid(fw, 8, 64)
    Z = torch.zeros(8, 64, device=DEV)
    Z[1, 1] = -0.0
    codes, scales = L.encode(Z, 0, 0)
    c = codes.cpu().numpy()
    assert scales.item() == 0.0 and np.all((c & 0x7F) == 0) and c[1, 1] == 0x80
    assert L.flags() == 0
    X = torch.ones(8, 64, device=DEV)
    X[2, 3] = float("inf")
    codes, scales = L.encode(X, 0, 0)
    assert np.isnan(scales.item()) and np.all(codes.cpu().numpy() == 0x7F)
    assert L.flags() & fw.FLAG_NONFINITE
    out = L.decode_reduce(codes.unsqueeze(0), scales.reshape(1, 1), 0, 0)
    assert torch.isnan(out).all()


@pytest.mark.parametrize("R", [1, 3, 5, 8])
@pytest.mark.parametrize("scaling,s", [("tensor", 0), ("block", 1)])
@pytest.mark.parametrize("shape", [(150, 400), (37, 408)])
@pytest.mark.parametrize("fused", [True, False])
def test_dequant_reduce_matches_oracle(fw, R, scaling, s, shape, fused):
    """Both routes: the persistent kernel and the standalone dequant-sum
    (16 codes per lane, or 8 when d is not a multiple of 16)."""
    print(f"[dequant-reduce R={R} {scaling} {shape} fused={fused}]", flush=True)
    fw.set_fused(fused)
    rng = np.random.default_rng(30 + R)
    m, d = shape
    Xs = [(rng.standard_normal((m, d)) * np.exp(rng.standard_normal((1, d)))).astype(np.float32) for _ in range(R)]
    pl = [G.quantize(x, "e4m3", scaling)[:2] for x in Xs]
    ref = G.dequant_reduce([p[0] for p in pl], [p[1] for p in pl], "e4m3", scaling)
    L = _euclid(fw, m, d)
    stride = -(-m * d // 16) * 16     # replica rows 16-byte aligned
    codes = torch.empty(R, stride, dtype=torch.uint8, device=DEV)[:, :m * d].view(R, m, d)
    codes.copy_(torch.from_numpy(np.stack([p[0] for p in pl])))
    scales = torch.from_numpy(np.stack([p[1].ravel() for p in pl])).to(DEV)
    out = L.decode_reduce(codes, scales, 0, s).cpu().numpy()
    # fp32 sum of R exact products: error <= R ulps of the sum of magnitudes
    mag = sum(np.abs(G.dequantize(p[0], p[1], "e4m3", scaling)) for p in pl) / R
    assert np.all(np.abs(out - ref) <= (R + 1) * 2.0 ** -24 * mag)
