"""The stress layer at full size: W 4096 x 16384 fp32, heavy-tailed
gradients (Student-t, nu = 3, column scales i^-1.5, 0.1 % of the columns x
100), bf16 activations of the same law (T = 8192), rank-32 factor refreshed
from this step's statistics (q = 4, p = 16), per-128x128-block E5M2 and E4M3
payloads of R = 16 independent replicas.

Pages: GIFT 阅读笔记 §前置知识 Eq. (4) (statistics), §简化二 Eq. (17)
(rank-32 factor) and Eq. (16) (input-side whitening), Algorithm 1 (scale,
quantise, reduce, map back).

At this size the oracle works on samples, stage by stage, from the GPU's own
inputs to each stage (stage isolation): entries of A against exact float64
dot products; the factor of the GPU's A; whole 128-row block rows of the
whitened tensor, codes, scales and the decoded mean.  The dense transform
(d = 16384, 2 GiB in float64) is the oracle's definition, as at every size.
"""
import numpy as np
import pytest
import torch

import synth
from oracle import gift as G
from tests.helpers import assert_codes, rel_fro

pytestmark = pytest.mark.gpu
DEV = "cuda"
M, D, T, R = 4096, 16384, 8192, 16
BLOCK_ROWS = (0, 17)        # 128-row block rows checked (rows 0..127 and 2176..2303)


@pytest.fixture(scope="module")
def fw():
    import fac_whitening_amd as fw
    return fw


@pytest.fixture(scope="module")
def stress(fw):
    print("[stress 4096x16384 R=16: drawing]", flush=True)
    a = synth.stress_activations(T, D, 0, DEV)
    Ws = [synth.stress_gradient(M, D, 0, r, DEV) for r in range(R)]
    om = synth.omega(D, 48, synth.seed_for(5, synth.ROLE_OMEGA), DEV)
    L = fw.Layer(M, D, "lowrank", device=DEV)
    L.accumulate_stats(a, commit=True)
    L.refresh(om)
    torch.cuda.synchronize()
    assert L.flags() == 0
    A = L.buffers()["A"].double().cpu().numpy()
    print("[stress: oracle factor of the GPU's A]", flush=True)
    fac = G.lowrank_factor(A, om.cpu().numpy(), 32, 4, G.damping(A))
    Tm, Tinv = G.transform_lowrank(fac)
    yield dict(L=L, a=a, Ws=Ws, A=A, fac=fac, T=Tm, Tinv=Tinv)
    L.close()


def _rows():
    return np.concatenate([np.arange(128 * b, 128 * b + 128) for b in BLOCK_ROWS])


def test_stress_statistics_sampled(stress):
    """Entries of A = a^T a / T (bf16 inputs upcast exactly) against float64
    dot products, normalised by sqrt(A_ii A_jj) (off-diagonal entries of a
    heavy-tailed sample can cancel to near zero)."""
    A, a = stress["A"], stress["a"]
    rng = np.random.default_rng(5)
    i = rng.integers(0, D, 192)
    j = rng.integers(0, D, 192)
    i = np.concatenate([i, [0, 1, D - 1]])
    j = np.concatenate([j, [0, D - 1, D - 1]])
    cols = torch.from_numpy(np.unique(np.concatenate([i, j]))).to(DEV)
    sub = a[:, cols].double().cpu().numpy()
    pos = {int(c): k for k, c in enumerate(cols.cpu().numpy())}
    for ii, jj in zip(i, j):
        ref = float(sub[:, pos[int(ii)]] @ sub[:, pos[int(jj)]]) / T
        scale = np.sqrt(A[ii, ii] * A[jj, jj])
        assert abs(A[ii, jj] - ref) <= 1e-5 * scale, (ii, jj, A[ii, jj], ref)
    assert np.array_equal(A, A.T)


def test_stress_factor(stress):
    """The rank-32 coefficients of the GPU refresh against the oracle's
    factor of the same A with the same Omega."""
    L, fac = stress["L"], stress["fac"]
    coef = L.buffers()["coef"].cpu().numpy().astype(np.float64)
    assert abs(coef[67] / fac["rho"] - 1) <= 1e-6, (coef[67], fac["rho"])
    assert np.max(np.abs(coef[:32] - fac["c_enc"]) / np.abs(fac["c_enc"])) <= 1e-5
    assert np.max(np.abs(coef[32:64] - fac["c_dec"]) / np.abs(fac["c_dec"])) <= 1e-5


@pytest.mark.parametrize("fmt", ["e5m2", "e4m3"])
def test_stress_encode_decode_block_rows(fw, stress, fmt):
    L, Ws, Tm, Tinv = stress["L"], stress["Ws"], stress["T"], stress["Tinv"]
    print(f"[stress encode/decode {fmt} per block, R={R}]", flush=True)
    f = fw.E5M2 if fmt == "e5m2" else fw.E4M3
    s = fw.SCALE_BLOCK128
    nb = fw.nblocks(M, D, s)
    codes = torch.empty(R, M, D, dtype=torch.uint8, device=DEV)
    scales = torch.empty(R, nb, dtype=torch.float32, device=DEV)
    whit = torch.empty(M, D, device=DEV)
    am = torch.empty(nb, device=DEV)
    for r in range(R):
        L.encode(Ws[r], f, s, codes=codes[r], scales=scales[r], whitened=whit if r == 0 else None,
                 amax_out=am if r == 0 else None)
    out = L.decode_reduce(codes, scales, f, s)
    torch.cuda.synchronize()
    assert L.flags() == 0
    rows = _rows()
    nbd = -(-D // 128)
    w0 = Ws[0][torch.from_numpy(rows).to(DEV)].cpu().numpy()
    g_whit = whit[torch.from_numpy(rows).to(DEV)].cpu().numpy()
    # whitening of whole block rows
    ref_whit = G.whiten(w0, Tm)
    err = rel_fro(g_whit, ref_whit)
    print(f"  whitened rel err {err:.3e}", flush=True)
    assert err <= 1e-5
    sc_all = scales.cpu().numpy()
    am_all = am.cpu().numpy().reshape(-1, nbd)
    c_all = codes[:, torch.from_numpy(rows).to(DEV)].cpu().numpy()
    for k, b in enumerate(BLOCK_ROWS):
        sl = slice(128 * k, 128 * k + 128)
        # the quantiser, bit-exact on the GPU's own whitened block row
        cq, sq, amq = G.quantize(g_whit[sl], fmt, "block")
        assert np.array_equal(c_all[0, sl], cq)
        assert np.array_equal(sc_all[0].reshape(-1, nbd)[b], sq.ravel())
        assert np.array_equal(am_all[b], amq.ravel().astype(np.float32))
        # against the oracle's own whitened rows: one code step at most
        ce, _, _ = G.quantize(ref_whit[sl], fmt, "block")
        assert_codes(c_all[0, sl], ce)
    # decode-reduce of the same 16 payloads, whole block rows
    for k, b in enumerate(BLOCK_ROWS):
        sl = slice(128 * k, 128 * k + 128)
        cl = [c_all[r, sl] for r in range(R)]
        sl_scales = [sc_all[r].reshape(-1, nbd)[b:b + 1] for r in range(R)]
        ubar = G.dequant_reduce(cl, sl_scales, fmt, "block")
        ref = G.unwhiten(ubar, Tinv)
        got = out[torch.from_numpy(rows[sl]).to(DEV)].cpu().numpy()
        err = rel_fro(got, ref)
        print(f"  decoded block row {b}: rel err {err:.3e}", flush=True)
        assert err <= 1e-5


def test_stress_fp4_rows(fw, stress):
    """The FP4 payload (E2M1, 16-element row blocks with E4M3 scales, fp32
    tensor scale) of the 16 stress replicas: the tensor amax against the
    whole GPU whitened tensor; codes, block scales and tensor scale of whole
    rows bit for bit against the oracle on the GPU's whitened rows with the
    GPU's tensor amax; the decoded mean of those rows mapped back with the
    oracle's transform."""
    from oracle import fp4
    L, Ws, Tinv = stress["L"], stress["Ws"], stress["Tinv"]
    print(f"[stress fp4, R={R}]", flush=True)
    codes = torch.empty(R, M, D // 2, dtype=torch.uint8, device=DEV)
    bsc = torch.empty(R, M, D // 16, dtype=torch.uint8, device=DEV)
    tsc = torch.empty(R, device=DEV)
    whit = torch.empty(M, D, device=DEV)
    am = torch.empty(1, device=DEV)
    for r in range(R):
        L.encode_fp4(Ws[r], codes=codes[r], bscales=bsc[r], tscale=tsc[r:r + 1],
                     whitened=whit if r == 0 else None, amax_out=am if r == 0 else None)
    out = L.decode_reduce_fp4(codes, bsc, tsc)
    torch.cuda.synchronize()
    assert L.flags() == 0
    assert am.item() == whit.abs().max().item()
    rows = torch.from_numpy(_rows()).to(DEV)
    g_whit = whit[rows].cpu().numpy()
    ref = G.quantize_fp4(g_whit, amax_in=am.cpu().numpy())
    assert np.array_equal(codes[0][rows].cpu().numpy(), fp4.pack(ref["codes"]))
    assert np.array_equal(bsc[0][rows].cpu().numpy(), ref["bscales"])
    assert tsc[0].item() == ref["tscale"]
    cl = [fp4.unpack(codes[r][rows].cpu().numpy()) for r in range(R)]
    U = G.dequant_reduce_fp4(cl, [bsc[r][rows].cpu().numpy() for r in range(R)], tsc.cpu().numpy())
    err = rel_fro(out[rows].cpu().numpy(), G.unwhiten(U, Tinv))
    print(f"  decoded rows rel err {err:.3e}", flush=True)
    assert err <= 1e-5
