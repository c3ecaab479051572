"""Pins of the oracle's GIFT path against the pages and the mathematics.

Sources: GIFT 阅读笔记 (zhongzhuzhou.org) -- Eq. (1)-(17), Algorithm 1, the
toy example Eq. (A1)-(A3).  Each test pins one oracle function to something
other than itself: a value the page prints, a closed form, a brute-force
loop, or an independent library route.
"""
import numpy as np
import pytest
import scipy.linalg as sla

from oracle import fp8
from oracle import gift as G
from tests.golden.load import load

WX = load("worked_example_2x2.txt")


def _close(a, key):
    v, tol = WX[key]
    np.testing.assert_allclose(np.ravel(a), v, rtol=0, atol=tol)


# ---------------------------------------------------------------------------
# Worked example (Eq. A1-A3 and the toy quantiser)
# ---------------------------------------------------------------------------

def test_worked_example_cholesky_and_direction():
    A = WX["A"][0].reshape(2, 2)
    _close(np.linalg.eigvalsh(A)[::-1], "eigenvalues")
    L = G.cholesky_lower(A)
    _close(L, "L_A")
    T, Tinv = G.transform_cholesky(A, 0.0)
    _close(T.T, "L_A_inv")                 # T_A = L_A^-T
    g = WX["g"][0]
    # a gradient row g is sent to L_A^-1 g (Eq. A3): row-vector form g T_A
    _close(g @ T, "g_tilde")
    np.testing.assert_allclose(g @ T @ Tinv, g, atol=1e-14)
    # the oracle's whiten() on the 1x2 gradient gives the same row
    _close(G.whiten(g[None, :].astype(np.float32), T), "g_tilde")


def test_worked_example_toy_quantiser():
    g = WX["g"][0]
    A = WX["A"][0].reshape(2, 2)
    T, Tinv = G.transform_cholesky(A, 0.0)
    gh = G.toy_quantize(g)
    _close(gh, "toy_g_hat")
    _close(np.linalg.norm(gh - g), "toy_err_raw")
    gt = g @ T
    gth = G.toy_quantize(gt)
    _close(gth, "toy_g_tilde_hat")
    _close(np.linalg.norm(gth - gt), "toy_err_white")
    # mapped back, the whitened-coordinate error is smaller than the raw one
    # (the page says "smaller"; the value 0.1438 is derived here)
    back = np.linalg.norm((gth - gt) @ Tinv)
    assert back == pytest.approx(0.14384, abs=2e-4)
    assert back < np.linalg.norm(gh - g)


def test_worked_example_rank1():
    """k = d - 1 = 1 of the 2x2 example: the rank-k form equals A^-1/2 (the
    trailing eigenvalue is exactly rho).  Independent route: sqrtm."""
    A = WX["A"][0].reshape(2, 2)
    om = np.array([[1.0, -0.2], [0.3, 0.9]])   # l = min(k + p, d) = 2 columns
    f = G.lowrank_factor(A, om, k=1, q=4, lam=0.0)
    assert f["rho"] == pytest.approx(1.0, abs=1e-12)
    T, _ = G.transform_lowrank(f)
    ref = np.linalg.inv(sla.sqrtm(A).real)
    np.testing.assert_allclose(T, ref, atol=1e-12)
    np.testing.assert_allclose(T, [[0.68898, -0.31102], [-0.31102, 0.68898]], atol=1e-5)
    np.testing.assert_allclose(WX["g"][0] @ T, [3.13389, -0.86611], atol=1e-5)


# ---------------------------------------------------------------------------
# Statistics (Eq. 4) and EMA
# ---------------------------------------------------------------------------

def test_second_moment_bruteforce():
    rng = np.random.default_rng(3)
    a = rng.standard_normal((5, 3)).astype(np.float32)
    A = G.second_moment(a)
    B = np.zeros((3, 3))
    for t in range(5):
        for i in range(3):
            for j in range(3):
                B[i, j] += float(a[t, i]) * float(a[t, j])
    np.testing.assert_allclose(A, B / 5, rtol=1e-15)
    # closed form: tr(A) = mean squared norm of the rows
    assert np.trace(A) == pytest.approx(np.mean(np.sum(a.astype(np.float64) ** 2, 1)), rel=1e-14)
    assert np.all(np.linalg.eigvalsh(A) >= -1e-15)


def test_ema_closed_form():
    rng = np.random.default_rng(4)
    batches = [rng.standard_normal((4, 4)) for _ in range(4)]
    beta = 0.95
    A = None
    for b in batches:
        A = G.ema_commit(A, b, beta)
    S = len(batches)
    ref = beta ** (S - 1) * batches[0] + sum(beta ** (S - t) * (1 - beta) * batches[t - 1] for t in range(2, S + 1))
    np.testing.assert_allclose(A, ref, rtol=1e-14)
    # identical batches -> the EMA is the batch
    B = None
    for _ in range(3):
        B = G.ema_commit(B, batches[0], beta)
    np.testing.assert_allclose(B, batches[0], rtol=1e-14)


# ---------------------------------------------------------------------------
# Identities of the derivation (Eq. 5-6, 9, 11-12, 14)
# ---------------------------------------------------------------------------

def _spd(n, rng, cond=10.0):
    Q, _ = np.linalg.qr(rng.standard_normal((n, n)))
    return (Q * np.linspace(1, cond, n)) @ Q.T


def _vec(X):
    return X.reshape(-1, order="F")       # column stacking, as on the page


def test_two_sided_kronecker_form_bruteforce():
    """Eq. (12): vec(W~) = (L_A^-1 kron L_G^-1) vec(W), m = 3, d = 4."""
    rng = np.random.default_rng(5)
    A, Gm = _spd(4, rng), _spd(3, rng)
    W = rng.standard_normal((3, 4)).astype(np.float32)
    T, Tinv = G.transform_cholesky(A, 0.0)
    LG = G.output_factor(Gm, 0.0)
    LA = G.cholesky_lower(A)
    Wt = np.linalg.solve(LG, W.astype(np.float64)) @ T
    K = np.kron(np.linalg.inv(LA), np.linalg.inv(LG))
    np.testing.assert_allclose(_vec(Wt), K @ _vec(W.astype(np.float64)), atol=1e-12)
    np.testing.assert_allclose(G.whiten(W, T, LG), Wt.astype(np.float32), rtol=0, atol=0)
    # Eq. (14) undoes Eq. (11)
    np.testing.assert_allclose(LG @ Wt @ Tinv, W, atol=1e-12)


def test_metric_identities_and_isometry():
    """Eq. (5)-(6) and Eq. (9) with the oracle's factors."""
    rng = np.random.default_rng(6)
    A, Gm = _spd(4, rng), _spd(3, rng)
    dW = rng.standard_normal((3, 4))
    kron = _vec(dW) @ np.kron(A, Gm) @ _vec(dW)
    tr = np.trace(A @ dW.T @ Gm @ dW)
    assert kron == pytest.approx(tr, rel=1e-12)
    LA, LG = G.cholesky_lower(A), G.output_factor(Gm, 0.0)
    assert np.linalg.norm(LG.T @ dW @ LA) ** 2 == pytest.approx(tr, rel=1e-12)


def test_a_metric_report_matches_kronecker():
    """The A-metric error of metrics() is Eq. (5) with G = I."""
    rng = np.random.default_rng(7)
    A = _spd(4, rng)
    W = rng.standard_normal((3, 4))
    Wh = W + 0.01 * rng.standard_normal((3, 4))
    E = Wh - W
    K = np.kron(A, np.eye(3))
    ref = np.sqrt((_vec(E) @ K @ _vec(E)) / (_vec(W) @ K @ _vec(W)))
    m = G.metrics(Wh, W, A)
    assert m["ARel"] == pytest.approx(ref, rel=1e-12)
    assert m["RelL2"] == pytest.approx(np.linalg.norm(E) / np.linalg.norm(W), rel=1e-14)
    assert m["MSE"] == pytest.approx(np.sum(E ** 2) / 12, rel=1e-14)
    assert m["MaxErr"] == pytest.approx(np.abs(E).max(), rel=1e-15)
    assert m["Cos"] == pytest.approx(np.sum(Wh * W) / np.linalg.norm(Wh) / np.linalg.norm(W), rel=1e-14)


# ---------------------------------------------------------------------------
# Rank-k factor (Eq. 17 with reading R1)
# ---------------------------------------------------------------------------

def _spiked(d, k, rng, c=0.01):
    Q, _ = np.linalg.qr(rng.standard_normal((d, d)))
    sig = np.concatenate([np.geomspace(100.0, 10.0, k), np.full(d - k, c)])
    return (Q * sig) @ Q.T, Q, sig


def test_lowrank_spiked_closed_form():
    """A = U diag(sigma) U^T + c (I - U U^T): T_A equals A^-1/2 (lam = 0)."""
    rng = np.random.default_rng(8)
    d, k = 96, 8
    A, Q, sig = _spiked(d, k, rng)
    om = rng.standard_normal((d, k + 8))
    f = G.lowrank_factor(A, om, k, q=4, lam=0.0)
    assert f["rho"] == pytest.approx(0.01, rel=1e-10)
    np.testing.assert_allclose(f["theta"], sig[:k], rtol=1e-10)
    T, Tinv = G.transform_lowrank(f)
    ref = (Q * sig ** -0.5) @ Q.T
    np.testing.assert_allclose(T, ref, atol=1e-10 * np.abs(ref).max())
    np.testing.assert_allclose(Tinv, (Q * sig ** 0.5) @ Q.T, atol=1e-9)
    # whitened covariance is the identity on a spiked A
    np.testing.assert_allclose(T @ A @ T, np.eye(d), atol=1e-9)


@pytest.mark.parametrize("kk", [0, 1])
def test_lowrank_full_rank_is_symmetric_whitening(kk):
    """Invariant: rank = d (and d - 1) reproduces (A + lam I)^-1/2,
    computed independently with scipy's eigh."""
    rng = np.random.default_rng(9)
    d = 40
    A = _spd(d, rng, cond=1e3)
    lam = G.damping(A)
    k = d - kk
    om = rng.standard_normal((d, min(k + 16, d)))
    f = G.lowrank_factor(A, om, k, q=4, lam=lam)
    T, Tinv = G.transform_lowrank(f)
    w, V = sla.eigh(A + lam * np.eye(d))
    ref = (V * w ** -0.5) @ V.T
    assert np.linalg.norm(T - ref) / np.linalg.norm(ref) < 1e-10
    np.testing.assert_allclose(T.T @ (A + lam * np.eye(d)) @ T, np.eye(d), atol=1e-10)


def _mgs(Y):
    Q = np.array(Y, dtype=np.float64)
    for j in range(Q.shape[1]):
        for i in range(j):
            Q[:, j] -= (Q[:, i] @ Q[:, j]) * Q[:, i]
        for i in range(j):
            Q[:, j] -= (Q[:, i] @ Q[:, j]) * Q[:, i]
        Q[:, j] /= np.linalg.norm(Q[:, j])
    return Q


def _cholqr2(Y):
    Q = Y
    for _ in range(2):
        R = np.linalg.cholesky(Q.T @ Q).T
        Q = sla.solve_triangular(R, Q.T, trans="T").T
    return Q


def test_lowrank_basis_independent():
    """span(A^(q+1) Omega) and the Ritz pairs do not depend on the
    orthonormalisation: Householder, Gram-Schmidt and CholeskyQR2 agree."""
    rng = np.random.default_rng(10)
    d = 128
    i = np.arange(1, d + 1)
    Q, _ = np.linalg.qr(rng.standard_normal((d, d)))
    A = (Q * i ** -1.5) @ Q.T
    om = rng.standard_normal((d, 48))
    lam = G.damping(A)
    T0, _ = G.transform_lowrank(G.lowrank_factor(A, om, 32, 4, lam))
    for fn in (_mgs, _cholqr2):
        T1, _ = G.transform_lowrank(G.lowrank_factor(A, om, 32, 4, lam, orth_fn=fn))
        assert np.linalg.norm(T1 - T0) / np.linalg.norm(T0) < 1e-9


def test_lowrank_large_gap_matches_eigh():
    rng = np.random.default_rng(11)
    d, k = 200, 32
    A, Q, sig = _spiked(d, k, rng, c=1e-3)
    A = A + 1e-5 * _spd(d, rng)          # break the exact spike, keep the gap
    f = G.lowrank_factor(A, rng.standard_normal((d, k + 16)), k, 4, 0.0)
    w, V = sla.eigh(A)
    Vk = V[:, ::-1][:, :k]
    np.testing.assert_allclose(f["U"] @ f["U"].T, Vk @ Vk.T, atol=1e-9)
    np.testing.assert_allclose(f["theta"], w[::-1][:k], rtol=1e-10)


# ---------------------------------------------------------------------------
# Invariants on the tiny configuration
# ---------------------------------------------------------------------------

@pytest.fixture(scope="module")
def tiny():
    import synth
    case = synth.make_layer(1, device="cpu")
    a = case.a_steps[0].numpy()
    A = G.second_moment(a)
    return dict(case=case, a=a, A=A, lam=G.damping(A), W=[w.numpy() for w in case.W],
                omega=case.omega.numpy(), delta=case.delta_steps[0].numpy())


@pytest.mark.parametrize("kind", ["diag", "lowrank", "chol", "twosided"])
def test_invariant_round_trip(tiny, kind):
    """Transform round trip without quantisation recovers W to 1e-12."""
    Gm = G.second_moment(tiny["delta"])
    T, Tinv, LG = G.build_transform(kind, A=tiny["A"], lam=tiny["lam"], omega=tiny["omega"],
                                    G=Gm, lam_G=G.damping(Gm))
    W = tiny["W"][0].astype(np.float64)
    X = W @ T
    if LG is not None:
        X = np.linalg.solve(LG, X)
        back = LG @ (X @ Tinv)
    else:
        back = X @ Tinv
    assert np.linalg.norm(back - W) / np.linalg.norm(W) <= 1e-12


def test_invariant_identity_covariance(tiny):
    """Full-rank whitened activations have identity covariance (lam = 0,
    T = 1024 >= d = 256): Cholesky and rank = d."""
    a, A = tiny["a"].astype(np.float64), tiny["A"]
    d = A.shape[0]
    T_chol, _ = G.transform_cholesky(A, 0.0)
    f = G.lowrank_factor(A, np.random.default_rng(12).standard_normal((d, d)), d, 4, 0.0)
    T_lr, _ = G.transform_lowrank(f)
    for T in (T_chol, T_lr):
        at = a @ T
        C = at.T @ at / a.shape[0]
        assert np.linalg.norm(C - np.eye(d)) / np.sqrt(d) <= 1e-10


@pytest.mark.parametrize("kind", ["diag", "chol", "lowrank"])
@pytest.mark.parametrize("mexp", [-3, 0, 2])
@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_invariant_power_of_four_identity(tiny, kind, mexp, fmt):
    """A = 4^m I with lam = 0 gives codes bit-identical to the Euclidean
    baseline and scales s_euclid * 2^-m."""
    d = tiny["A"].shape[0]
    c = 4.0 ** mexp
    A = c * np.eye(d)
    T, Tinv, _ = G.build_transform(kind, A=A, lam=0.0, omega=tiny["omega"])
    W = tiny["W"][0]
    for scaling in ("tensor", "block"):
        e = G.encode(W, np.eye(d), fmt, scaling)
        g = G.encode(W, T, fmt, scaling)
        assert np.array_equal(g["whitened"], (W.astype(np.float64) * 2.0 ** -mexp).astype(np.float32))
        assert np.array_equal(g["codes"], e["codes"])
        assert np.array_equal(g["scales"], (e["scales"].astype(np.float64) * 2.0 ** -mexp).astype(np.float32))


def test_invariant_payload_is_quarter_of_fp32():
    for (m, d, sc) in [(1536, 6144, "tensor"), (1536, 6144, "block"), (64, 256, "tensor"), (100, 300, "block")]:
        pb = G.payload_bytes(m, d, sc)
        bm, bd = G.nblocks(m, d, sc)
        assert pb == m * d + 4 * bm * bd
        assert pb - 4 * bm * bd == (4 * m * d) // 4
    rng = np.random.default_rng(13)
    X = rng.standard_normal((100, 300)).astype(np.float32)
    codes, scales, _ = G.quantize(X, "e4m3", "block")
    assert codes.nbytes + scales.nbytes == G.payload_bytes(100, 300, "block")


# ---------------------------------------------------------------------------
# Damping (reading R2: lam = 1e-3 tr(A) / n of the undamped statistics)
# ---------------------------------------------------------------------------

def test_damping_hand_values():
    """lam = rel * tr(A) / n, from the diagonal only, written out by hand."""
    assert G.damping(np.diag([1.0, 2.0, 3.0, 4.0])) == pytest.approx(2.5e-3, rel=1e-15)
    assert G.damping(np.diag([1.0, 2.0, 3.0, 4.0]), rel=0.5) == pytest.approx(1.25, rel=1e-15)
    # off-diagonal entries do not enter; n is the matrix order
    assert G.damping(np.array([[2.0, 1.0], [1.0, 4.0]])) == pytest.approx(3e-3, rel=1e-15)
    assert G.damping(np.full((3, 3), 7.0)) == pytest.approx(7e-3, rel=1e-15)


def test_damping_enters_the_transforms_on_the_undamped_trace():
    """The diagonal and Cholesky transforms of A = c I (d = 8) with the
    damping written out by hand: lam = 1e-3 * (8 c) / 8 = 1e-3 c, so
    T_A = (c + 1e-3 c)^-1/2 I.  A lam taken from the damped trace, or over
    a wrong count, moves T_A by more than the tolerance."""
    d, c = 8, 4.0
    A = c * np.eye(d)
    lam = G.damping(A)
    assert lam == pytest.approx(4e-3, rel=1e-15)
    want = (c * 1.001) ** -0.5
    for kind in ("diag", "chol"):
        T, Tinv, _ = G.build_transform(kind, A=A, lam=lam)
        np.testing.assert_allclose(T, want * np.eye(d), rtol=1e-14, atol=0)
        np.testing.assert_allclose(Tinv, np.eye(d) / want, rtol=1e-14, atol=0)


def test_damping_on_a_spiked_lowrank_factor():
    """A = Q diag(sigma) Q^T with k spikes and a flat tail c: the rank-k
    factor with lam = 1e-3 tr(A) / d (tr(A) = sum sigma, computed from the
    spectrum, not from A) gives rho = c + lam, Lt = sigma_k + lam and
    T_A = (A + lam I)^-1/2 exactly."""
    rng = np.random.default_rng(21)
    d, k = 64, 6
    A, Q, sig = _spiked(d, k, rng, c=0.02)
    lam_hand = 1e-3 * float(sig.sum()) / d
    assert G.damping(A) == pytest.approx(lam_hand, rel=1e-12)
    f = G.lowrank_factor(A, rng.standard_normal((d, k + 8)), k, 4, G.damping(A))
    assert f["rho"] == pytest.approx(0.02 + lam_hand, rel=1e-10)
    np.testing.assert_allclose(f["lam_t"], sig[:k] + lam_hand, rtol=1e-10)
    T, _ = G.transform_lowrank(f)
    ref = (Q * (sig + lam_hand) ** -0.5) @ Q.T
    np.testing.assert_allclose(T, ref, atol=1e-10 * np.abs(ref).max())


# ---------------------------------------------------------------------------
# Quantiser and reduction
# ---------------------------------------------------------------------------

def test_quantize_blocks_bruteforce():
    """Per-tile amax and scale on a ragged 200 x 300 tensor, element by element."""
    rng = np.random.default_rng(14)
    X = (rng.standard_normal((200, 300)) * np.exp(rng.standard_normal((200, 300)) * 2)).astype(np.float32)
    codes, scales, am = G.quantize(X, "e4m3", "block")
    assert scales.shape == (2, 3)
    for (i, j) in [(0, 0), (150, 299), (199, 130), (127, 128), (128, 127)]:
        bi, bj = i // 128, j // 128
        tile = X[bi * 128:(bi + 1) * 128, bj * 128:(bj + 1) * 128]
        a = float(np.abs(tile).max())
        r = np.float32(448.0 / a)
        assert scales[bi, bj] == np.float32(a / 448.0)
        y = np.float32(np.float64(X[i, j]) * np.float64(r))
        assert codes[i, j] == fp8.encode(np.array([y]), "e4m3")[0]
    # the largest element of each tile encodes to the largest code
    for bi in range(2):
        for bj in range(3):
            tile = np.abs(X[bi * 128:(bi + 1) * 128, bj * 128:(bj + 1) * 128])
            ii, jj = np.unravel_index(np.argmax(tile), tile.shape)
            assert codes[bi * 128 + ii, bj * 128 + jj] & 0x7F == 0x7E


def _e4m3_finite_values():
    """Non-negative finite E4M3 values from the bit layout (bias 7, 3
    mantissa bits; exponent 15 with mantissa 7 is NaN)."""
    v = [m * 2.0 ** -9 for m in range(8)]
    v += [(8 + m) * 2.0 ** (e - 10) for e in range(1, 16) for m in range(8) if not (e == 15 and m == 7)]
    return np.array(v)


def test_block_dequantize_exact_on_ragged_tiles():
    """Per-128x128 round trip on a ragged 200 x 300 tensor (tiles of
    128/72 rows and 128/128/44 columns): tile (i, j) holds E4M3 values
    times 2^e_ij with one element at +-448 * 2^e_ij, every e_ij different.
    Then r = 2^-e_ij and s = 2^e_ij exactly, every code is exact, and
    dequantize() must give the tensor back bit for bit; a transposed or
    shifted tile-to-scale map, or an edge tile read with the wrong extent,
    scales some element by the wrong power of two."""
    rng = np.random.default_rng(22)
    m, d = 200, 300
    vals = _e4m3_finite_values()
    vals = vals[vals <= 448]
    ex = np.array([[-7, 3, 11], [5, -2, 0]])
    X = np.empty((m, d), np.float32)
    for i in range(2):
        for j in range(3):
            rs, cs = slice(128 * i, min(m, 128 * i + 128)), slice(128 * j, min(d, 128 * j + 128))
            h, w = rs.stop - rs.start, cs.stop - cs.start
            v = rng.choice(vals, (h, w)) * rng.choice([-1.0, 1.0], (h, w))
            v[h // 2, w // 3] = 448.0 * (-1) ** (i + j)
            X[rs, cs] = v * 2.0 ** ex[i, j]
    codes, scales, am = G.quantize(X, "e4m3", "block")
    np.testing.assert_array_equal(scales, (2.0 ** ex).astype(np.float32))
    np.testing.assert_array_equal(am, 448.0 * 2.0 ** ex)
    back = G.dequantize(codes, scales, "e4m3", "block")
    np.testing.assert_array_equal(back, X.astype(np.float64))
    # the reduction of R copies of the same payload is that payload
    U = G.dequant_reduce([codes] * 4, [scales] * 4, "e4m3", "block")
    np.testing.assert_array_equal(U, X.astype(np.float64))
    # and a transposed scale grid (2 x 3 -> 3 x 2 read back row-major) fails
    bad = np.ascontiguousarray(scales.T).reshape(2, 3)
    assert not np.array_equal(G.dequantize(codes, bad, "e4m3", "block"), back)


def test_quantize_zero_and_nonfinite():
    Z = np.zeros((4, 5), np.float32)
    Z[1, 1] = -0.0
    c, s, _ = G.quantize(Z, "e4m3", "tensor")
    assert s[0, 0] == 0 and np.all((c & 0x7F) == 0) and c[1, 1] == 0x80
    X = np.ones((4, 5), np.float32)
    X[2, 3] = np.inf
    c, s, _ = G.quantize(X, "e4m3", "tensor")
    assert np.isnan(s[0, 0]) and np.all(c == 0x7F)
    assert np.all(np.isnan(G.dequantize(c, s, "e4m3", "tensor")))


def test_dequant_reduce_linearity():
    rng = np.random.default_rng(15)
    Ws = [rng.standard_normal((50, 70)).astype(np.float32) for _ in range(3)]
    payloads = [G.quantize(w, "e4m3", "block")[:2] for w in Ws]
    U = G.dequant_reduce([p[0] for p in payloads], [p[1] for p in payloads], "e4m3", "block")
    ref = sum(fp8.decode(p[0], "e4m3") * np.repeat(np.repeat(p[1].astype(np.float64), 128, 0), 128, 1)[:50, :70]
              for p in payloads) / 3
    np.testing.assert_allclose(U, ref, rtol=1e-15)
    # R identical replicas -> one decode
    U1 = G.dequant_reduce([payloads[0][0]] * 4, [payloads[0][1]] * 4, "e4m3", "block")
    np.testing.assert_array_equal(U1, G.dequantize(payloads[0][0], payloads[0][1], "e4m3", "block"))


def test_lossless_equivalence(tiny):
    """With the quantiser removed, decode(encode(W_r)) averaged is the mean
    gradient (the page: lossless communication makes GIFT the baseline)."""
    T, Tinv, _ = G.build_transform("lowrank", A=tiny["A"], lam=tiny["lam"], omega=tiny["omega"])
    Ws = [w.astype(np.float64) for w in tiny["W"]]
    Ubar = sum(w @ T for w in Ws) / len(Ws)
    Wbar = sum(Ws) / len(Ws)
    assert np.linalg.norm(Ubar @ Tinv - Wbar) / np.linalg.norm(Wbar) <= 1e-12


def test_fidelity_report_runs(tiny):
    """The Table I/II analogue on the tiny layer (values are reported, not
    pinned: the pages' numbers come from real gradients)."""
    Ws = tiny["W"]
    Wbar = sum(w.astype(np.float64) for w in Ws) / len(Ws)
    out = {}
    for kind in ("euclid", "diag", "lowrank", "chol"):
        T, Tinv, _ = G.build_transform(kind, A=tiny["A"], lam=tiny["lam"], omega=tiny["omega"])
        enc = [G.encode(w, T, "e4m3", "tensor") for w in Ws]
        Wh = G.decode_reduce([e["codes"] for e in enc], [e["scales"] for e in enc], Tinv, "e4m3", "tensor")
        out[kind] = G.metrics(Wh, Wbar, tiny["A"])
    for kind, mtr in out.items():
        assert 0 < mtr["RelL2"] < 0.2 and mtr["Cos"] > 0.98


# ---------------------------------------------------------------------------
# Boundary-hit profiler (Note §简化三, Fig. 3)
# ---------------------------------------------------------------------------

def test_boundary_hits_bruteforce():
    rng = np.random.default_rng(16)
    X = (rng.standard_normal((30, 40)) * np.exp(3 * rng.standard_normal((30, 40)))).astype(np.float32)
    X[0, :5] = 0
    up, lo = G.boundary_hits(X, "e4m3")
    a = float(np.abs(X).max())
    r = np.float32(448.0 / a)
    bu = bl = 0
    for x in X.ravel():
        y = np.float32(np.float64(x) * np.float64(r))
        c = int(fp8.encode(np.array([y]), "e4m3")[0]) & 0x7F
        bu += c == 0x7E
        bl += (c == 0) and x != 0
    assert (up, lo) == (bu, bl)
    assert up >= 1 and lo > 0


def test_knee_selects_thirteen():
    rng = np.random.default_rng(17)
    n = 48
    s = np.concatenate([rng.uniform(0.08, 0.1, 13), rng.uniform(0.004, 0.006, n - 13)])
    perm = rng.permutation(n)
    order, sel = G.select_layers(s[perm], max_select=24)
    assert sorted(sel) == sorted(np.argsort(perm)[:13].tolist())
    assert len(sel) == 13
    # a cap below the knee
    _, sel5 = G.select_layers(s[perm], max_select=5)
    assert len(sel5) == 5
    # zero tail: cut where the scores drop to zero
    _, selz = G.select_layers(np.array([3.0, 2.0, 0.0, 0.0]), max_select=4)
    assert selz == [0, 1]
    # ties rank the lower index first
    order, _ = G.select_layers(np.array([1.0, 2.0, 2.0, 1.0]), max_select=2)
    assert order == [1, 2, 0, 3]


def test_layer_scores_mean_over_steps():
    counts = np.array([[10, 30], [0, 4]])
    sc = G.layer_scores(counts, [100, 50], n_steps=2)
    np.testing.assert_allclose(sc, [40 / 200, 4 / 100])


# ---------------------------------------------------------------------------
# Error feedback ([Note] 算法 1, its error-feedback steps; reading R11)
# ---------------------------------------------------------------------------

def _spacing(y, fmt):
    """Distance between consecutive finite FP8 values in the binade of |y|,
    from the format's layout (E4M3: bias 7, 3 mantissa bits, normals from
    2^-6; E5M2: bias 15, 2 mantissa bits, normals from 2^-14)."""
    mant, emin = (3, -6) if fmt == "e4m3" else (2, -14)
    a = np.abs(np.asarray(y, dtype=np.float64))
    e = np.floor(np.log2(np.maximum(a, 2.0 ** emin)))
    return 2.0 ** (e - mant)


def _ef_steps(tiny, kind, fmt, scaling, steps=4):
    T = G.build_transform(kind, A=tiny["A"], lam=tiny["lam"], omega=tiny["omega"])[0]
    rng = np.random.default_rng(11)
    m, d = tiny["W"][0].shape
    R = np.zeros((m, d), np.float32)
    outs = []
    for t in range(steps):
        W = (tiny["W"][t % len(tiny["W"])] * (1.0 + 0.3 * rng.standard_normal((m, d)))).astype(np.float32)
        e = G.encode_ef(W, T, R, fmt, scaling)
        outs.append((e, R))
        R = e["residual"]
    return outs


@pytest.mark.parametrize("kind", ["lowrank", "diag"])
@pytest.mark.parametrize("fmt,scaling", [("e4m3", "tensor"), ("e5m2", "block")])
def test_error_feedback_telescopes(tiny, kind, fmt, scaling):
    """R_t = U~_t - deq_t and U~_t = W~_t + R_{t-1} give, with R_0 = 0,
    sum_t deq_t + R_T = sum_t W~_t (up to the float32 roundings of U~ and R):
    nothing the quantiser rounds away is lost, it is carried."""
    outs = _ef_steps(tiny, kind, fmt, scaling)
    sum_deq = sum(G.dequantize(e["codes"], e["scales"], fmt, scaling) for e, _ in outs)
    sum_w = sum(e["whitened"].astype(np.float64) for e, _ in outs)
    lhs = sum_deq + outs[-1][0]["residual"].astype(np.float64)
    err = np.linalg.norm(lhs - sum_w) / np.linalg.norm(sum_w)
    assert err < 1e-6, err
    # dropping the residual breaks it at the quantiser's error level
    no_ef = sum(G.dequantize(*G.quantize(e["whitened"], fmt, scaling)[:2], fmt, scaling) for e, _ in outs)
    assert np.linalg.norm(no_ef - sum_w) / np.linalg.norm(sum_w) > 100 * err


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_error_feedback_residual_is_half_a_step(tiny, fmt):
    """Each new residual is the rounding error of U~'s code: at most half the
    FP8 spacing at U~ r, times the scale (plus the float32 rounding of y)."""
    for e, _ in _ef_steps(tiny, "lowrank", fmt, "tensor"):
        s = float(e["scales"][0, 0])
        y = e["u_tilde"].astype(np.float64) / s
        bound = 0.5 * s * _spacing(y, fmt) + 4e-7 * np.abs(e["u_tilde"]) + 1e-30
        assert np.all(np.abs(e["residual"].astype(np.float64)) <= bound)


def test_error_feedback_first_step_is_plain_encode(tiny):
    """With a zero residual the codes and scales are those of Algorithm 1
    without error feedback, and the residual is U~ - s dec(q)."""
    T = G.build_transform("lowrank", A=tiny["A"], lam=tiny["lam"], omega=tiny["omega"])[0]
    W = tiny["W"][0]
    e = G.encode_ef(W, T, np.zeros_like(W), "e4m3", "block")
    p = G.encode(W, T, "e4m3", "block")
    assert np.array_equal(e["codes"], p["codes"]) and np.array_equal(e["scales"], p["scales"])
    deq = G.dequantize(p["codes"], p["scales"], "e4m3", "block")
    assert np.array_equal(e["residual"], (p["whitened"].astype(np.float64) - deq).astype(np.float32))
