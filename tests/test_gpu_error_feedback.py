"""Error feedback (the residual carried in whitened coordinates) through
gift_encode_ef, on the persistent kernels and on the multi-kernel path, for
every transform, against the oracle.

Pages: GIFT 阅读笔记 Algorithm 1 (error-feedback lines: U~ = W~ + R, scale
and quantise U~, R <- U~ - dequantised U~), with the oracle's reading of
the rounding (U~ rounded to fp32 once, the new residual the fp32 rounding
of the exact difference).

Stage isolation: at every step the oracle takes the GPU's whitened tensor
and the GPU's residual from the step before, so codes, scales, amax and the
new residual must agree bit for bit.  Across the steps the outputs must
telescope: sum_t s_t dec(q_t) + R_T = sum_t W~_t up to the fp32 roundings of
U~ and R at each step.
"""
import numpy as np
import pytest
import torch

from oracle import gift as G

pytestmark = pytest.mark.gpu
DEV = "cuda"
STEPS = 4          # step 2 has a zero gradient; step 3 a shared amax 1.25 x the local one


@pytest.fixture(scope="module")
def fw():
    import fac_whitening_amd as fw
    yield fw
    fw.set_fused(True)


def _gradients(m, d, seed):
    rng = np.random.default_rng(seed)
    cs = (np.arange(1, d + 1) ** -0.5).astype(np.float32)
    rs = (np.arange(1, m + 1) ** -0.25).astype(np.float32)
    Ws = []
    for t in range(STEPS):
        if t == 2:
            Ws.append(np.zeros((m, d), np.float32))
        else:
            Ws.append((rng.standard_normal((m, d)).astype(np.float32) * cs) * rs[:, None])
    return Ws


def _layer(fw, kind, m, d, seed):
    """A layer of the given transform with its factor refreshed on the GPU
    from power-law activations (the EF stage takes the GPU's W~ as input,
    so the factor itself is not under test here)."""
    rng = np.random.default_rng(seed + 1)
    L = fw.Layer(m, d, kind, device=DEV)
    if kind == "euclid":
        return L
    a = (rng.standard_normal((512, d)) * np.arange(1, d + 1) ** -0.75).astype(np.float32)
    L.accumulate_stats(torch.from_numpy(a).to(DEV), fw.SIDE_A, commit=True)
    if kind == "twosided":
        dl = (rng.standard_normal((512, m)) * np.arange(1, m + 1) ** -0.5).astype(np.float32)
        L.accumulate_stats(torch.from_numpy(dl).to(DEV), fw.SIDE_G, commit=True)
    om = torch.from_numpy(rng.standard_normal((d, 48)).astype(np.float32)).to(DEV) if kind == "lowrank" else None
    L.refresh(om)
    return L


def _same(a, b):
    """Bit equality of float arrays (NaN payloads aside)."""
    a, b = np.asarray(a), np.asarray(b)
    return a.shape == b.shape and bool(np.all((a == b) | (np.isnan(a) & np.isnan(b))))


CASES = [
    ("lowrank", True, (200, 1544)),
    ("lowrank", False, (200, 1544)),
    ("lowrank", True, (1536, 6144)),
    ("euclid", True, (100, 1000)),
    ("euclid", False, (100, 1000)),
    ("euclid", True, (1536, 6144)),
    ("diag", False, (96, 264)),
    ("chol", False, (96, 264)),
    ("twosided", False, (96, 264)),
]


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
@pytest.mark.parametrize("scaling", ["tensor", "block"])
@pytest.mark.parametrize("kind,fused,shape", CASES)
def test_error_feedback_steps(fw, kind, fused, shape, scaling, fmt):
    m, d = shape
    print(f"[ef {kind} fused={fused} {shape} {scaling} {fmt}]", flush=True)
    fw.set_fused(fused)
    L = _layer(fw, kind, m, d, seed=m + d)
    f, s = fw.FORMATS[fmt], fw.SCALINGS[scaling]
    nb = fw.nblocks(m, d, s)
    resid = torch.zeros(m, d, device=DEV)
    Ws = _gradients(m, d, seed=m * 7 + d)
    deq_sum = np.zeros((m, d))
    wh_sum = np.zeros((m, d))
    bound = np.zeros((m, d))
    for t, w in enumerate(Ws):
        Wg = torch.from_numpy(w).to(DEV)
        R_prev = resid.cpu().numpy()
        # amax-only call: the amax of W~ + R, residual untouched
        am1 = torch.empty(nb, device=DEV)
        L.encode(Wg, f, s, amax_out=am1, want_codes=False, resid=resid)
        torch.cuda.synchronize()
        assert np.array_equal(resid.cpu().numpy(), R_prev), "an amax-only call changed the residual"
        amax_in = am1 * 1.25 if t == 3 else None
        codes = torch.empty(m, d, dtype=torch.uint8, device=DEV)
        scales = torch.empty(nb, device=DEV)
        wh = torch.empty(m, d, device=DEV)
        am2 = torch.empty(nb, device=DEV)
        L.encode(Wg, f, s, amax_in=amax_in, codes=codes, scales=scales, whitened=wh, amax_out=am2, resid=resid)
        # the inspection output is W~ itself, as without error feedback
        wh_plain = torch.empty(m, d, device=DEV)
        L.encode(Wg, f, s, whitened=wh_plain, amax_out=torch.empty(nb, device=DEV), want_codes=False)
        torch.cuda.synchronize()
        assert L.flags() == 0
        wh_np = wh.cpu().numpy()
        assert np.array_equal(wh_np, wh_plain.cpu().numpy())
        ref = G.error_feedback(wh_np, R_prev, fmt, scaling,
                               amax_in=None if amax_in is None else amax_in.cpu().numpy())
        assert np.array_equal(codes.cpu().numpy(), ref["codes"]), f"codes differ at step {t}"
        assert np.array_equal(scales.cpu().numpy(), ref["scales"].ravel()), f"scales differ at step {t}"
        am_ref = G.amax(ref["u_tilde"], scaling).ravel().astype(np.float32)
        assert np.array_equal(am1.cpu().numpy(), am_ref) and np.array_equal(am2.cpu().numpy(), am_ref)
        Rn = resid.cpu().numpy()
        assert _same(Rn, ref["residual"]), f"residual differs at step {t}"
        deq_sum += G.dequantize(ref["codes"], ref["scales"], fmt, scaling)
        wh_sum += wh_np
        bound += 2.0 ** -24 * (np.abs(ref["u_tilde"]) + np.abs(Rn))
    # telescoping: what was sent plus what is still owed is what was produced
    gap = np.abs(deq_sum + resid.cpu().numpy() - wh_sum)
    bound += 2.0 ** -50 * (np.abs(deq_sum) + np.abs(wh_sum))   # the float64 sums of this check
    assert np.all(gap <= bound), float(np.max(gap - bound))
    L.close()


@pytest.mark.parametrize("fused", [True, False])
@pytest.mark.parametrize("kind", ["euclid", "lowrank"])
def test_error_feedback_nonfinite_block(fw, kind, fused):
    """An Inf in the gradient: its block gets scale NaN and codes 0x7F and a
    NaN residual, the other blocks are encoded as usual, the flag is set."""
    m, d = 200, 1544
    print(f"[ef nonfinite {kind} fused={fused}]", flush=True)
    fw.set_fused(fused)
    L = _layer(fw, kind, m, d, seed=3)
    nb = fw.nblocks(m, d, fw.SCALE_BLOCK128)
    w = _gradients(m, d, seed=5)[0]
    R0 = (np.random.default_rng(9).standard_normal((m, d)) * 1e-3).astype(np.float32)
    resid = torch.from_numpy(R0).to(DEV)
    w[130, 700] = np.inf
    codes = torch.empty(m, d, dtype=torch.uint8, device=DEV)
    scales = torch.empty(nb, device=DEV)
    wh = torch.empty(m, d, device=DEV)
    L.encode(torch.from_numpy(w).to(DEV), fw.E4M3, fw.SCALE_BLOCK128, codes=codes, scales=scales, whitened=wh,
             resid=resid)
    torch.cuda.synchronize()
    assert L.flags() & fw.FLAG_NONFINITE
    ref = G.error_feedback(wh.cpu().numpy(), R0, "e4m3", "block")
    assert np.array_equal(codes.cpu().numpy(), ref["codes"])
    assert _same(scales.cpu().numpy(), ref["scales"].ravel())
    assert _same(resid.cpu().numpy(), ref["residual"])
    assert np.isnan(ref["scales"]).any() and not np.isnan(ref["scales"]).all()
    L.close()


def test_error_feedback_rejects_missing_residual(fw):
    """gift_encode_ef requires the residual buffer."""
    import ctypes
    L = fw.Layer(64, 256, "euclid", device=DEV)
    W = torch.zeros(64, 256, device=DEV)
    am = torch.empty(1, device=DEV)
    st = fw._lib.gift_encode_ef(L.handle, W.data_ptr(), 256, 0, 0, None, am.data_ptr(), None, None, None, None,
                                L.work.data_ptr(), ctypes.c_size_t(L.work_bytes), None)
    assert st == 1
    L.close()
