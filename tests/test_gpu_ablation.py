"""The two-sided K-FAC ablation at its real size: one 1536 x 6144 fc2 layer,
A (6144^2) and G (1536^2) from T = 16384 bf16 tokens, E4M3 per 128 x 128
block, R = 8, compared with the input-only Cholesky, rank-32, diagonal and
Euclidean variants on the same payload recipe.

Pages: GIFT 阅读笔记, §核心想法 Eq. (7) (A = L_A L_A^T, G = L_G L_G^T),
Eq. (11) (W~ = L_G^-1 W L_A^-T), Eq. (14) (map back L_G U L_A^T), §简化一
Eq. (16) and Table I (full K-FAC against input-side only), §简化二 Table II
(diagonal, rank 32, full A).

Gates: A and G within 1e-5; the whitened tensor within 1e-5 of the oracle
fed the GPU's fp32 A and G (the full factor amplifies the fp32 rounding of
the stored statistics by about the condition number of A + lam I, so the
stage-isolated form is the binding one); >= 99.9 % of codes identical and
the rest one code step away; the decoded mean within 1e-3.  The fully
independent whitened error (oracle from the bf16 activations in fp64) is
asserted at the bound it meets on this workload.
"""
import numpy as np
import pytest
import torch

import synth
from oracle import gift as G
from tests.helpers import assert_codes, rel_fro

pytestmark = pytest.mark.gpu
DEV = "cuda"
KINDS = ("twosided", "chol", "lowrank", "diag", "euclid")


def _np(t):
    return t.detach().float().cpu().numpy() if t.dtype == torch.bfloat16 else t.detach().cpu().numpy()


@pytest.fixture(scope="module")
def ab():
    import fac_whitening_amd as fw
    print("[ablation] GPU side: statistics, refresh, encode, decode of 5 variants", flush=True)
    case = synth.make_layer(4, device=DEV)          # 1536 x 6144, T = 16384 bf16, R = 8
    m, d, R = case.cfg["m"], case.cfg["d"], len(case.W)
    a, dl = case.a_steps[0], case.delta_steps[0]
    out = dict(case=case, m=m, d=d, R=R, gpu={})
    for kind in KINDS:
        L = fw.Layer(m, d, kind, rank=32, oversample=16, power_iters=4, device=DEV)
        if kind != "euclid":
            L.accumulate_stats(a, fw.SIDE_A, commit=True)
        if kind == "twosided":
            L.accumulate_stats(dl, fw.SIDE_G, commit=True)
        L.refresh(case.omega)
        codes, scales = [], []
        whit = torch.empty(m, d, device=DEV)
        for r, W in enumerate(case.W):
            c, s = L.encode(W, fw.E4M3, fw.SCALE_BLOCK128, whitened=whit if r == 0 else None)
            codes.append(c)
            scales.append(s)
        dec = L.decode_reduce(torch.stack(codes), torch.stack(scales), fw.E4M3, fw.SCALE_BLOCK128)
        torch.cuda.synchronize()
        assert L.flags() == 0, kind
        b = L.buffers()
        out["gpu"][kind] = dict(
            codes=[c.cpu().numpy() for c in codes], scales=[s.cpu().numpy().reshape(12, 48) for s in scales],
            whitened=whit.cpu().numpy(), decoded=dec.cpu().numpy(),
            A=b["A"].cpu().numpy() if "A" in b else None, G=b["G"].cpu().numpy() if "G" in b else None)
        del L
    out["W"] = [_np(w) for w in case.W]
    out["a"] = _np(a)
    out["dl"] = _np(dl)
    return out


def test_ablation_statistics(ab):
    """A and G of the 16384 bf16 tokens within 1e-5 of the fp64 definition."""
    print("[ablation] statistics", flush=True)
    A = G.second_moment(ab["a"])
    Gm = G.second_moment(ab["dl"])
    for kind in ("twosided", "chol", "lowrank", "diag"):
        assert rel_fro(ab["gpu"][kind]["A"], A) <= 1e-5, kind
    assert rel_fro(ab["gpu"]["twosided"]["G"], Gm) <= 1e-5
    ab["A_ind"], ab["G_ind"] = A, Gm


@pytest.mark.parametrize("kind", ["chol", "twosided"])
def test_ablation_full_variants_stage_isolated(ab, kind):
    """The oracle fed the GPU's fp32 A (and G): whitened tensor, codes and
    decoded mean of all 8 replicas."""
    print(f"[ablation] {kind}: oracle on the GPU's statistics", flush=True)
    g = ab["gpu"][kind]
    A = g["A"].astype(np.float64)
    Gm = g["G"].astype(np.float64) if kind == "twosided" else None
    T, Tinv, LG = G.build_transform(kind, A=A, lam=G.damping(A), G=Gm,
                                    lam_G=G.damping(Gm) if Gm is not None else None)
    refs = [G.encode(w, T, "e4m3", "block", L_G=LG) for w in ab["W"]]
    err = rel_fro(g["whitened"], refs[0]["whitened"])
    print(f"  whitened rel err (stage-isolated) {err:.3e}", flush=True)
    assert err <= 1e-5
    assert_codes(g["codes"][0], refs[0]["codes"])
    for r in range(ab["R"]):
        assert_codes(g["codes"][r], refs[r]["codes"])
    ref = G.decode_reduce([e["codes"] for e in refs], [e["scales"] for e in refs], Tinv, "e4m3", "block", L_G=LG)
    derr = rel_fro(g["decoded"], ref)
    print(f"  decoded rel err {derr:.3e}", flush=True)
    assert derr <= 1e-3


@pytest.mark.parametrize("kind", ["chol", "twosided"])
def test_ablation_full_variants_independent(ab, kind):
    """Fully independent: the oracle's own A and G from the bf16 tokens.
    The full factor carries the fp32 rounding of the stored A (relative
    2^-24 per entry, and the fp32 sums over 16384 tokens) times about the
    condition number of A + lam I (near 1e6 here) into the whitened tensor,
    so 1e-5 is out of reach of any fp32 A; measured 1.4e-3 (input side).
    The assertion is a regression bound a few times above that."""
    print(f"[ablation] {kind}: independent oracle", flush=True)
    A = ab.get("A_ind")
    if A is None:
        A = G.second_moment(ab["a"])
    Gm = None
    if kind == "twosided":
        Gm = ab.get("G_ind")
        if Gm is None:
            Gm = G.second_moment(ab["dl"])
    T, _, LG = G.build_transform(kind, A=A, lam=G.damping(A), G=Gm, lam_G=G.damping(Gm) if Gm is not None else None)
    ref = G.whiten(ab["W"][0], T, LG)
    err = rel_fro(ab["gpu"][kind]["whitened"], ref)
    w, _ = np.linalg.eigh(A + G.damping(A) * np.eye(A.shape[0]))
    print(f"  whitened rel err (independent) {err:.3e}; cond(A + lam I) = {w[-1] / w[0]:.3e}", flush=True)
    assert err <= 5e-3


def test_ablation_variants_against_the_mean(ab):
    """Table I / II analogue on this layer: every variant's decoded mean
    against the fp32 mean gradient (RelL2, Cos, MaxErr, MSE and the A-metric
    error, Eq. (15) and Eq. (6) with G = I).  Reported; the only assertions
    are that every variant decodes to a close copy of the mean and that the
    payload recipe is the same (per-block E4M3)."""
    print("[ablation] variants against the fp32 mean", flush=True)
    Wbar = sum(w.astype(np.float64) for w in ab["W"]) / ab["R"]
    A = ab.get("A_ind")
    if A is None:
        A = G.second_moment(ab["a"])
    for kind in KINDS:
        mt = G.metrics(ab["gpu"][kind]["decoded"], Wbar, A)
        print(f"  {kind:9s} RelL2 {mt['RelL2']:.4e} Cos {mt['Cos']:.6f} MaxErr {mt['MaxErr']:.3e} "
              f"MSE {mt['MSE']:.3e} ARel {mt['ARel']:.4e}", flush=True)
        assert mt["RelL2"] < 0.1 and mt["Cos"] > 0.99
