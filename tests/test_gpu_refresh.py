"""Rank-32 refresh at the 1536 x 6144 layer against the oracle.

Pages: GIFT 阅读笔记 §简化二 Eq. (17) (rank-32 factor of A) and Eq. (16)
(input-side whitening).  Stage isolation: the oracle factors the GPU's own
fp32 A with the same Omega, so the comparison covers the subspace iteration,
orthonormalisation, Rayleigh-Ritz eigensolver and coefficients at the full
size (d = 6144: the product kernels split A's rows over many workgroups).
"""
import numpy as np
import pytest
import torch

import synth
from oracle import gift as G
from tests.helpers import rel_fro

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module")
def fw():
    import fac_whitening_amd as fw
    return fw


def test_refresh_metric_layer(fw):
    m, d = 1536, 6144
    print("[refresh 1536x6144]", flush=True)
    case = synth.make_layer(4, device=DEV, R=1, T=4096)
    L = fw.Layer(m, d, "lowrank", device=DEV)
    L.accumulate_stats(case.a_steps[0], commit=True)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    L.refresh(case.omega)
    e1.record()
    torch.cuda.synchronize()
    print(f"  refresh {e0.elapsed_time(e1):.3f} ms", flush=True)
    assert L.flags() == 0
    A = L.buffers()["A"].double().cpu().numpy()
    fac = G.lowrank_factor(A, case.omega.cpu().numpy(), 32, 4, G.damping(A))
    coef = L.buffers()["coef"].cpu().numpy().astype(np.float64)
    assert abs(coef[67] / fac["rho"] - 1) <= 1e-6, (coef[67], fac["rho"])
    assert abs(coef[66] / G.damping(A) - 1) <= 1e-6
    assert np.max(np.abs(coef[:32] - fac["c_enc"]) / np.abs(fac["c_enc"])) <= 1e-5
    assert np.max(np.abs(coef[32:64] - fac["c_dec"]) / np.abs(fac["c_dec"])) <= 1e-5
    # whitened tensor (fused encode of the GPU factor) on the first 192 rows
    T, _ = G.transform_lowrank(fac)
    whit = torch.empty(m, d, device=DEV)
    L.encode(case.W[0], 0, 0, whitened=whit)
    rows = 192
    ref = G.whiten(case.W[0][:rows].cpu().numpy(), T)
    err = rel_fro(whit[:rows].cpu().numpy(), ref)
    print(f"  whitened rel err {err:.3e}", flush=True)
    assert err <= 1e-5


def _factor_from_activations(fw, x, d, seed):
    L = fw.Layer(64, d, "lowrank", device=DEV)
    L.accumulate_stats(x, commit=True)
    om = torch.from_numpy(np.random.default_rng(seed).standard_normal((d, 48)).astype(np.float32)).to(DEV)
    L.refresh(om)
    torch.cuda.synchronize()
    assert L.flags() == 0
    b = L.buffers()
    return L, b["A"].double().cpu().numpy(), om.cpu().numpy(), b["U"].double().cpu().numpy(), \
        b["coef"].cpu().numpy().astype(np.float64)


def test_refresh_repeated_eigenvalues(fw):
    """Spectra with repeated Ritz values, where the eigenvectors of the
    Rayleigh-Ritz step are not unique (the tridiagonal solver hands such
    spectra to the Jacobi solver).  A = 4 I (activations 32 I over 256
    tokens): every coefficient against the oracle, c_enc = c_dec = 0 up to
    rounding, U orthonormal.  A with eigenvalues 4 and 1 on 128-dimensional
    subspaces: U orthonormal, its residual in the eigenspace of 4 no larger
    than the oracle's, the coefficients against the oracle."""
    d = 256
    print("[refresh, repeated eigenvalues]", flush=True)
    x = 32.0 * torch.eye(d, device=DEV)
    L, A, om, U, coef = _factor_from_activations(fw, x, d, 1)
    assert np.array_equal(A, 4.0 * np.eye(d))
    fac = G.lowrank_factor(A, om, 32, 4, G.damping(A))
    assert abs(coef[67] / fac["rho"] - 1) <= 1e-6 and abs(coef[64] * np.sqrt(fac["rho"]) - 1) <= 1e-6
    assert np.max(np.abs(coef[:32])) <= 1e-6 * coef[64] and np.max(np.abs(coef[32:64])) <= 1e-6 * coef[65]
    assert np.max(np.abs(U.T @ U - np.eye(32))) <= 1e-5
    L.close()
    rng = np.random.default_rng(2)
    Q = np.linalg.qr(rng.standard_normal((d, d)))[0]
    lam = np.concatenate([np.full(d // 2, 4.0), np.ones(d // 2)])
    xs = np.ascontiguousarray((np.sqrt(d) * np.sqrt(lam)[:, None] * Q.T).astype(np.float32))   # x^T x / d = Q diag(lam) Q^T
    L, A, om, U, coef = _factor_from_activations(fw, torch.from_numpy(xs).to(DEV), d, 3)
    fac = G.lowrank_factor(A, om, 32, 4, G.damping(A))
    assert np.max(np.abs(U.T @ U - np.eye(32))) <= 1e-5
    # four iterations leave (1/4)^5 of the other eigenspace in the basis:
    # the residual is the oracle's own, not zero
    resid = np.linalg.norm(A @ U - U * fac["theta"]) / np.linalg.norm(A @ U)
    Uo = fac["U"]
    resid_o = np.linalg.norm(A @ Uo - Uo * fac["theta"]) / np.linalg.norm(A @ Uo)
    print(f"  eigenspace residual {resid:.3e} (oracle {resid_o:.3e})", flush=True)
    assert resid <= 1.05 * resid_o + 1e-6
    assert abs(coef[67] / fac["rho"] - 1) <= 1e-6
    assert np.max(np.abs(coef[:32] - fac["c_enc"]) / np.abs(fac["c_enc"])) <= 1e-5
    L.close()


def test_refresh_graded_spectrum_with_close_pairs(fw):
    """A spectrum graded over three decades (the k largest eigenvalues
    10^(-3 i / 31)) with two neighbouring pairs 3e-7 and 2.5e-7 of the largest
    apart, 1e-4 and 2e-4 of their own size: close for a test on |T| alone,
    well separated for the tridiagonal solver's eigenvectors.  The rest of
    the spectrum lies below 1e-5.  U orthonormal, its residual no larger than
    the oracle's (to the fp32 storage of U), rho and the coefficients
    against the oracle at the tolerance of the other refresh tests."""
    d = 256
    print("[refresh, graded spectrum with close pairs]", flush=True)
    rng = np.random.default_rng(4)
    lam = np.concatenate([10.0 ** (-3.0 * np.arange(32) / 31), 1e-5 * rng.uniform(0.5, 1.0, d - 32)])
    lam[27] = lam[26] * (1 - 1e-4)
    lam[31] = lam[30] * (1 - 2e-4)
    Q = np.linalg.qr(rng.standard_normal((d, d)))[0]
    xs = np.ascontiguousarray((np.sqrt(d) * np.sqrt(lam)[:, None] * Q.T).astype(np.float32))
    L, A, om, U, coef = _factor_from_activations(fw, torch.from_numpy(xs).to(DEV), d, 5)
    fac = G.lowrank_factor(A, om, 32, 4, G.damping(A))
    orth = np.max(np.abs(U.T @ U - np.eye(32)))
    resid = np.linalg.norm(A @ U - U * fac["theta"]) / np.linalg.norm(A @ U)
    Uo = fac["U"]
    resid_o = np.linalg.norm(A @ Uo - Uo * fac["theta"]) / np.linalg.norm(A @ Uo)
    e_enc = np.max(np.abs(coef[:32] - fac["c_enc"]) / np.abs(fac["c_enc"]))
    e_dec = np.max(np.abs(coef[32:64] - fac["c_dec"]) / np.abs(fac["c_dec"]))
    print(f"  orthogonality {orth:.2e}, residual {resid:.3e} (oracle {resid_o:.3e}), "
          f"c_enc {e_enc:.2e}, c_dec {e_dec:.2e}", flush=True)
    assert orth <= 1e-5
    assert resid <= 1.05 * resid_o + 1e-6
    assert abs(coef[67] / fac["rho"] - 1) <= 1e-6
    assert e_enc <= 1e-5 and e_dec <= 1e-5
    L.close()
