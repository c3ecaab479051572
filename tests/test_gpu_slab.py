"""One GPU's share of the row-slab exchange (the multi-GPU design for the
rank-k path at R GPUs), at a small shape, against the oracle: the slab
dequant-sum in whitened coordinates, its requantisation, and the
unwhitening of a slab by a layer of the slab's rows with the same factor.

Pages: GIFT 阅读笔记 Algorithm 1 (quantise in the whitened coordinates,
AllReduceSum, Dequantize / N, map back with the input-side factor); the
input-side transform acts on the rows of W (§简化一 Eq. (16)), so each row,
and each slab of rows, maps back independently.
"""
import numpy as np
import pytest
import torch

from oracle import gift as G
from tests.helpers import layer_with_factor, rel_fro

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module")
def fw():
    import fac_whitening_amd as fw
    return fw


def test_slab_share_against_oracle(fw):
    m, d, R = 96, 512, 8
    rows = m // R
    print(f"[slab share {m}x{d} R={R}]", flush=True)
    rng = np.random.default_rng(12)
    a0 = (rng.standard_normal((2048, d)) * np.arange(1, d + 1) ** -0.75).astype(np.float32)
    A = G.second_moment(a0)
    fac = G.lowrank_factor(A, rng.standard_normal((d, 48)).astype(np.float32), 32, 4, G.damping(A))
    _, Tinv = G.transform_lowrank(fac)
    L = layer_with_factor(fw, m, d, fac, DEV)
    codes = torch.empty(R, m, d, dtype=torch.uint8, device=DEV)
    scales = torch.empty(R, 1, device=DEV)
    for r in range(R):
        w = (rng.standard_normal((m, d)) * np.arange(1, d + 1) ** -0.5).astype(np.float32)
        L.encode(torch.from_numpy(w).to(DEV), fw.E4M3, fw.SCALE_TENSOR, codes=codes[r], scales=scales[r])
    Le = fw.Layer(rows, d, "euclid", device=DEV)
    Lr = layer_with_factor(fw, rows, d, fac, DEV)
    sc = scales.cpu().numpy()
    for g in (0, 5, R - 1):
        slab = codes[:, g * rows:(g + 1) * rows, :]
        mean = Le.decode_reduce(slab, scales, fw.E4M3, fw.SCALE_TENSOR)
        c2, s2 = Le.encode(mean, fw.E4M3, fw.SCALE_TENSOR)
        back = Lr.decode_reduce(c2.unsqueeze(0), s2.reshape(1, 1), fw.E4M3, fw.SCALE_TENSOR)
        torch.cuda.synchronize()
        assert L.flags() == 0 and Le.flags() == 0 and Lr.flags() == 0
        sl = slab.cpu().numpy()
        ref_mean = G.dequant_reduce([sl[r] for r in range(R)], [sc[r].reshape(1, 1) for r in range(R)], "e4m3",
                                    "tensor")
        assert rel_fro(mean.cpu().numpy(), ref_mean) <= 1e-6, g
        cq, sq, _ = G.quantize(mean.cpu().numpy(), "e4m3", "tensor")
        assert np.array_equal(c2.cpu().numpy(), cq) and np.array_equal(s2.cpu().numpy(), sq.ravel()), g
        ref_back = G.unwhiten(G.dequantize(cq, sq, "e4m3", "tensor"), Tinv)
        err = rel_fro(back.cpu().numpy(), ref_back)
        print(f"  slab {g}: unwhitened rel err {err:.3e}", flush=True)
        assert err <= 1e-5, (g, err)


def test_slab_shared_scale_gather_and_unwhiten(fw):
    """All slabs requantised with one shared scale (AllReduceMax of the slab
    amax), gathered into one tensor and unwhitened with one R = 1 decode of
    the full layer: codes bit-exact, the result within the whitened
    tensor's tolerance of the oracle."""
    m, d, R = 96, 512, 8
    rows = m // R
    print(f"[slab shared scale {m}x{d} R={R}]", flush=True)
    rng = np.random.default_rng(13)
    a0 = (rng.standard_normal((2048, d)) * np.arange(1, d + 1) ** -0.75).astype(np.float32)
    A = G.second_moment(a0)
    fac = G.lowrank_factor(A, rng.standard_normal((d, 48)).astype(np.float32), 32, 4, G.damping(A))
    _, Tinv = G.transform_lowrank(fac)
    L = layer_with_factor(fw, m, d, fac, DEV)
    codes = torch.empty(R, m, d, dtype=torch.uint8, device=DEV)
    scales = torch.empty(R, 1, device=DEV)
    for r in range(R):
        w = (rng.standard_t(3, (m, d)) * np.arange(1, d + 1) ** -0.5).astype(np.float32)
        L.encode(torch.from_numpy(w).to(DEV), fw.E4M3, fw.SCALE_TENSOR, codes=codes[r], scales=scales[r])
    Le = fw.Layer(rows, d, "euclid", device=DEV)
    means, ams = [], []
    for g in range(R):
        mean = Le.decode_reduce(codes[:, g * rows:(g + 1) * rows, :], scales, fw.E4M3, fw.SCALE_TENSOR)
        a = torch.empty(1, device=DEV)
        Le.encode(mean, fw.E4M3, fw.SCALE_TENSOR, amax_out=a, want_codes=False)
        means.append(mean)
        ams.append(a)
    shared = torch.stack(ams).max(dim=0).values
    gathered = torch.empty(1, m, d, dtype=torch.uint8, device=DEV)
    gscale = torch.empty(1, 1, device=DEV)
    for g in range(R):
        Le.encode(means[g], fw.E4M3, fw.SCALE_TENSOR, amax_in=shared, codes=gathered[0, g * rows:(g + 1) * rows],
                  scales=gscale[0])
    out = L.decode_reduce(gathered, gscale, fw.E4M3, fw.SCALE_TENSOR)
    torch.cuda.synchronize()
    assert L.flags() == 0 and Le.flags() == 0
    sh = shared.cpu().numpy()
    for g in range(R):
        mg = means[g].cpu().numpy()
        assert np.float32(np.abs(mg).max()) == ams[g].item()
        cq, sq, _ = G.quantize(mg, "e4m3", "tensor", amax_in=sh)
        assert np.array_equal(gathered[0, g * rows:(g + 1) * rows].cpu().numpy(), cq), g
        assert gscale.item() == sq.ravel()[0]
    ref = G.unwhiten(G.dequantize(gathered[0].cpu().numpy(), gscale.cpu().numpy(), "e4m3", "tensor"), Tinv)
    err = rel_fro(out.cpu().numpy(), ref)
    print(f"  unwhitened rel err {err:.3e}", flush=True)
    assert err <= 1e-5, err
