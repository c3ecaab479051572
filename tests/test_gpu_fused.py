"""The persistent rank-k kernels (one launch per direction) against the oracle
and against the multi-kernel path, on ragged multi-tile shapes.

Pages: GIFT 阅读笔记 §简化二 Eq. (17) (rank-32 factor), Eq. (16) (input-side
whitening), Algorithm 1 (scale, quantise, reduce, map back).  The factor is
the oracle's, written into the layer state (stage isolation), so every
difference comes from the whitening / quantisation / reduction kernels.
"""
import numpy as np
import pytest
import torch

from oracle import gift as G
from tests.helpers import assert_codes, layer_with_factor, rel_fro

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module")
def fw():
    import fac_whitening_amd as fw
    yield fw
    fw.set_fused(True)


def _case(m, d, R, seed):
    """Power-law activations (rotated), W_r = delta_r^T a_r / T, oracle factor."""
    rng = np.random.default_rng(seed)
    big = d > 2000                 # keep the host-side draw cheap: no rotation, T = 2048
    T = 2048 if big else max(2 * d, 512)
    Q = np.eye(d) if big else np.linalg.qr(rng.standard_normal((d, d)))[0]
    sd = np.arange(1, d + 1) ** -0.75
    a0 = ((rng.standard_normal((T, d)) * sd) @ Q.T).astype(np.float32)
    A = G.second_moment(a0)
    om = rng.standard_normal((d, 48)).astype(np.float32)
    fac = G.lowrank_factor(A, om, 32, 4, G.damping(A))
    Ws = []
    for r in range(R):
        a = a0 if r == 0 else ((rng.standard_normal((T, d)) * sd) @ Q.T).astype(np.float32)
        dl = (rng.standard_normal((T, m)) * np.arange(1, m + 1) ** -0.5).astype(np.float32)
        Ws.append((dl.T.astype(np.float64) @ a.astype(np.float64) / T).astype(np.float32))
    return Ws, fac


def _layer_with_factor(fw, m, d, fac):
    return layer_with_factor(fw, m, d, fac, DEV)


SHAPES = [(100, 1000), (200, 1544), (48, 768), (1536, 6144)]


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("scaling", ["tensor", "block"])
@pytest.mark.parametrize("fused", [True, False])
def test_lowrank_paths_against_oracle(fw, shape, scaling, fused):
    m, d = shape
    R = 3
    print(f"[lowrank {shape} {scaling} fused={fused}]", flush=True)
    fw.set_fused(fused)
    Ws, fac = _case(m, d, R, seed=m + d)
    T, Tinv = G.transform_lowrank(fac)
    L = _layer_with_factor(fw, m, d, fac)
    s = fw.SCALINGS[scaling]
    nb = fw.nblocks(m, d, s)
    codes, scales = [], []
    for r, w in enumerate(Ws):
        whit = torch.empty(m, d, device=DEV) if r == 0 else None
        am = torch.empty(nb, device=DEV) if r == 0 else None
        c, sc = L.encode(torch.from_numpy(w).to(DEV), 0, s, whitened=whit, amax_out=am)
        codes.append(c)
        scales.append(sc)
        if r == 0:
            e = G.encode(w, T, "e4m3", scaling)
            err = rel_fro(whit.cpu().numpy(), e["whitened"])
            assert err <= 1e-5, f"whitened rel err {err:.3e}"
            assert_codes(c.cpu().numpy(), e["codes"])
            # scales and amax are those of the GPU's own whitened tensor
            cq, sq, amq = G.quantize(whit.cpu().numpy(), "e4m3", scaling)
            assert np.array_equal(sc.cpu().numpy(), sq.ravel())
            assert np.array_equal(am.cpu().numpy(), amq.ravel().astype(np.float32))
            assert np.array_equal(c.cpu().numpy(), cq)
    out = L.decode_reduce(torch.stack(codes), torch.stack(scales), 0, s)
    ref = G.decode_reduce([c.cpu().numpy() for c in codes], [x.cpu().numpy().reshape(G.nblocks(m, d, scaling))
                                                             for x in scales], Tinv, "e4m3", scaling)
    err = rel_fro(out.cpu().numpy(), ref)
    assert err <= 1e-5, f"decode (same payloads) rel err {err:.3e}"
    assert L.flags() == 0


def test_fused_equals_multikernel_and_is_repeatable(fw):
    m, d = 1536, 6144
    print("[fused vs multi-kernel, repeated calls]", flush=True)
    Ws, fac = _case(m, d, 2, seed=7)
    W = torch.from_numpy(Ws[0]).to(DEV)
    outs = {}
    payload = None
    for fused in (False, True):
        fw.set_fused(fused)
        L = _layer_with_factor(fw, m, d, fac)
        whit = torch.empty(m, d, device=DEV)
        c, s = L.encode(W, 0, 0, whitened=whit)
        if payload is None:
            payload = (c.clone(), s.clone())   # both paths decode the same payload
        o = L.decode_reduce(payload[0].unsqueeze(0), payload[1].reshape(1, 1), 0, 0)
        outs[fused] = (whit.clone(), c.clone(), s.clone(), o.clone())
        c, s = payload
        if fused:
            c1, s1 = outs[True][1], outs[True][2]
            for it in range(25):   # barrier epochs advance; results stay identical
                c2, s2 = L.encode(W, 0, 0)
                o2 = L.decode_reduce(c, s.reshape(1, 1), 0, 0)
                assert torch.equal(c2, c1) and torch.equal(s2, s1) and torch.equal(o2, o), it
            assert L.counters()[5] == 26 and L.counters()[6] == 26
        assert L.flags() == 0
    assert rel_fro(outs[True][0].cpu().numpy(), outs[False][0].cpu().numpy()) <= 2e-6
    assert_codes(outs[True][1].cpu().numpy(), outs[False][1].cpu().numpy())
    assert rel_fro(outs[True][3].cpu().numpy(), outs[False][3].cpu().numpy()) <= 1e-5


@pytest.mark.parametrize("scaling", ["tensor", "block"])
def test_fused_shared_amax(fw, scaling):
    """amax_in (the AllReduceMax result) drives the scale; amax_out still
    reports the local amax."""
    m, d = 200, 1544
    print(f"[fused shared amax {scaling}]", flush=True)
    fw.set_fused(True)
    Ws, fac = _case(m, d, 1, seed=11)
    L = _layer_with_factor(fw, m, d, fac)
    s = fw.SCALINGS[scaling]
    nb = fw.nblocks(m, d, s)
    W = torch.from_numpy(Ws[0]).to(DEV)
    whit = torch.empty(m, d, device=DEV)
    local = torch.empty(nb, device=DEV)
    L.encode(W, 0, s, whitened=whit, amax_out=local)
    shared = local * 1.75
    c, sc = L.encode(W, 0, s, amax_in=shared)
    cq, sq, _ = G.quantize(whit.cpu().numpy(), "e4m3", scaling,
                           amax_in=shared.cpu().numpy().astype(np.float64).reshape(G.nblocks(m, d, scaling)))
    assert np.array_equal(c.cpu().numpy(), cq) and np.array_equal(sc.cpu().numpy(), sq.ravel())
    local2 = torch.empty(nb, device=DEV)
    L.encode(W, 0, s, amax_in=shared, amax_out=local2)
    assert torch.equal(local2, local)


@pytest.mark.parametrize("scaling", ["tensor", "block"])
def test_fused_nonfinite_rows_under_shared_amax(fw, scaling):
    """A finite shared amax (Algorithm 1's AllReduceMax) with Inf and NaN in
    a few rows of this worker's gradient: the whitening spreads them along
    their rows, so the waves holding those rows quantise element by element
    (exact integer encoder: Inf saturates, NaN -> 0x7F with its sign) while
    every other wave of the launch takes the uniform finite path.  Codes
    and scales bit-exact against the oracle's quantiser on the GPU's own
    whitened tensor (reading R4)."""
    m, d = 200, 1544
    print(f"[fused non-finite rows, shared amax, {scaling}]", flush=True)
    fw.set_fused(True)
    Ws, fac = _case(m, d, 1, seed=13)
    L = _layer_with_factor(fw, m, d, fac)
    s = fw.SCALINGS[scaling]
    nb = fw.nblocks(m, d, s)
    W = torch.from_numpy(Ws[0]).to(DEV)
    local = torch.empty(nb, device=DEV)
    L.encode(W, 0, s, amax_out=local)
    shared = local * 1.25
    W[37, 100] = float("inf")
    W[150, 901] = float("-inf")
    W[151, 5] = float("nan")
    whit = torch.empty(m, d, device=DEV)
    c, sc = L.encode(W, 0, s, amax_in=shared, whitened=whit)
    wh = whit.cpu().numpy()
    bad_rows = ~np.isfinite(wh).all(axis=1)
    assert bad_rows[[37, 150, 151]].all() and bad_rows.sum() < m // 4
    cq, sq, _ = G.quantize(wh, "e4m3", scaling,
                           amax_in=shared.cpu().numpy().astype(np.float64).reshape(G.nblocks(m, d, scaling)))
    assert np.array_equal(c.cpu().numpy(), cq)
    assert np.array_equal(sc.cpu().numpy(), sq.ravel())


@pytest.mark.parametrize("R", [1, 16, 64, 65])
@pytest.mark.parametrize("scaling", ["tensor", "block"])
def test_fused_decode_replica_count_extremes(fw, R, scaling):
    """One replica (the run-time count), 16 (compiled, whole-tile order), 64
    (the most whose scales the persistent decode stages) and 65 (past it:
    the multi-kernel route) on a ragged multi-tile shape, against the
    oracle's decode-reduce of the same payloads (Algorithm 1: dequantise,
    average over the R workers, map back)."""
    m, d = 100, 1000
    print(f"[fused decode R={R} {scaling}]", flush=True)
    fw.set_fused(True)
    _, fac = _case(m, d, 1, seed=17)
    _, Tinv = G.transform_lowrank(fac)
    L = _layer_with_factor(fw, m, d, fac)
    s = fw.SCALINGS[scaling]
    nb = fw.nblocks(m, d, s)
    rng = np.random.default_rng(100 + R)
    cs = (np.arange(1, d + 1) ** -0.5).astype(np.float32)
    codes = torch.empty(R, m, d, dtype=torch.uint8, device=DEV)
    scales = torch.empty(R, nb, dtype=torch.float32, device=DEV)
    for r in range(R):
        w = (rng.standard_normal((m, d)).astype(np.float32) * cs * (1.0 + 0.05 * r)).astype(np.float32)
        L.encode(torch.from_numpy(w).to(DEV), 0, s, codes=codes[r], scales=scales[r])
    out = L.decode_reduce(codes, scales, 0, s)
    bm, bd = G.nblocks(m, d, scaling)
    ref = G.decode_reduce([codes[r].cpu().numpy() for r in range(R)],
                          [scales[r].cpu().numpy().reshape(bm, bd) for r in range(R)], Tinv, "e4m3", scaling)
    err = rel_fro(out.cpu().numpy(), ref)
    assert err <= 1e-5, f"decode rel err {err:.3e}"
    assert L.flags() == 0


@pytest.mark.parametrize("R", [4, 8])
@pytest.mark.parametrize("scaling", ["tensor", "block"])
@pytest.mark.parametrize("shape", [(200, 1544), (1536, 6144)])
def test_fused_decode_compiled_replica_counts(fw, R, scaling, shape):
    """The decode compiled for a fixed replica count (4, 8: the replicas
    stream block by block and each 16-row block is projected as it lands)
    against the oracle's decode-reduce of the same payloads, on a ragged
    multi-tile shape (d % 16 == 8) and the full layer."""
    m, d = shape
    print(f"[fused decode R={R} {scaling} {shape}]", flush=True)
    fw.set_fused(True)
    Ws, fac = _case(m, d, R, seed=3 * R + m)
    _, Tinv = G.transform_lowrank(fac)
    L = _layer_with_factor(fw, m, d, fac)
    s = fw.SCALINGS[scaling]
    nb = fw.nblocks(m, d, s)
    codes = torch.empty(R, m, d, dtype=torch.uint8, device=DEV)
    scales = torch.empty(R, nb, dtype=torch.float32, device=DEV)
    for r, w in enumerate(Ws):
        L.encode(torch.from_numpy(w).to(DEV), 0, s, codes=codes[r], scales=scales[r])
    out = L.decode_reduce(codes, scales, 0, s)
    bm, bd = G.nblocks(m, d, scaling)
    ref = G.decode_reduce([codes[r].cpu().numpy() for r in range(R)],
                          [scales[r].cpu().numpy().reshape(bm, bd) for r in range(R)], Tinv, "e4m3", scaling)
    err = rel_fro(out.cpu().numpy(), ref)
    assert err <= 1e-5, f"decode rel err {err:.3e}"
    assert L.flags() == 0


@pytest.mark.parametrize("k", [-80, -40, 40, 90])
def test_fused_scale_invariance_by_powers_of_two(fw, k):
    """Every scale inside the fused kernels is a power of two (the row scales
    of the two-piece f16 products, 2^14 on U_k, the FP8 scale pair), so
    W 2^k must give the same codes with every scale times 2^k, and the
    decode of those payloads exactly 2^k times the decode at k = 0, down to
    gradients near 1e-30 and up to 1e24."""
    m, d, R = 200, 1544, 3
    print(f"[fused scale invariance 2^{k}]", flush=True)
    Ws, fac = _case(m, d, R, 11)
    L = _layer_with_factor(fw, m, d, fac)
    fw.set_fused(True)
    for scaling in (fw.SCALE_TENSOR, fw.SCALE_BLOCK128):
        base_c, base_s, sc_c, sc_s = [], [], [], []
        for W in Ws:
            Wt = torch.from_numpy(W).to(DEV)
            c0, s0 = L.encode(Wt, fw.E4M3, scaling)
            c1, s1 = L.encode(Wt * 2.0 ** k, fw.E4M3, scaling)
            assert torch.equal(c0, c1)
            assert torch.equal(s1, s0 * 2.0 ** k)
            base_c.append(c0); base_s.append(s0); sc_c.append(c1); sc_s.append(s1)
        o0 = L.decode_reduce(torch.stack(base_c), torch.stack(base_s), fw.E4M3, scaling)
        o1 = L.decode_reduce(torch.stack(sc_c), torch.stack(sc_s), fw.E4M3, scaling)
        assert torch.equal(o1, o0 * 2.0 ** k)
    assert L.flags() == 0
