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
