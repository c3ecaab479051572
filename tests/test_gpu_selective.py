"""The 600M-class selective deployment: one Euclidean tensor of every shape
(q/k/v/o 1536 x 1536, fc1/fc3 6144 x 1536, fc2 1536 x 6144) and one rank-32
fc2 layer, each encoded for R = 8 replicas (E4M3, per-tensor scale) and
decoded, against the oracle on the full tensors.

Pages: GIFT 阅读笔记 Algorithm 1 (Euclidean branch: local amax,
AllReduceMax, one scale shared by the replicas, quantise, AllReduceSum,
dequantise, divide by N; geometry branch with the rank-32 factor of
§简化二 Eq. (17)), §实验设置 (Llama-600M, fc2 selected by the profiler).
The Euclidean gradients are the direct Gaussian draw of the selective
workload; the rank-32 layer's activations are bf16 with a rotated power-law
covariance (exponent alpha of that layer), T = 8192.
"""
import numpy as np
import pytest
import torch

import synth
from oracle import gift as G
from tests.helpers import assert_codes, rel_fro

pytestmark = pytest.mark.gpu
DEV = "cuda"
R = 8


@pytest.fixture(scope="module")
def fw():
    import fac_whitening_amd as fw
    return fw


@pytest.mark.parametrize("name", ["q", "fc1", "fc2"])
def test_selective_euclid_shapes(fw, name):
    """Shared amax over the replicas (AllReduceMax), every replica quantised
    with it, the mean decoded: codes and scales bit-exact, the mean within
    the fp32 rounding of a sum of R terms."""
    mo, di = synth.SELECTIVE_SHAPES[name]
    layer = 1   # a Euclidean layer for every tensor name (fc2 of layer 1 is rank-32: use layer 20)
    if name == "fc2":
        layer = 20
    alpha = float(synth.selective_alphas()[layer])
    print(f"[selective euclid {name} {mo}x{di}]", flush=True)
    Ws = [synth.direct_gradient(mo, di, alpha, 8192, synth.seed_for(3, synth.ROLE_A, layer, r), DEV)
          for r in range(R)]
    L = fw.Layer(mo, di, "euclid", device=DEV)
    ams = []
    for W in Ws:
        a = torch.empty(1, device=DEV)
        L.encode(W, fw.E4M3, fw.SCALE_TENSOR, amax_out=a, want_codes=False)
        ams.append(a)
    shared = torch.stack(ams).max(dim=0).values
    ws = [W.cpu().numpy() for W in Ws]
    am_ref = max(float(np.abs(w).max()) for w in ws)
    assert float(shared.item()) == np.float32(am_ref)
    codes = torch.empty(R, mo, di, dtype=torch.uint8, device=DEV)
    scales = torch.empty(R, 1, dtype=torch.float32, device=DEV)
    cl, sl = [], []
    for r, (W, w) in enumerate(zip(Ws, ws)):
        L.encode(W, fw.E4M3, fw.SCALE_TENSOR, amax_in=shared, codes=codes[r], scales=scales[r])
        cr, sr, _ = G.quantize(w, "e4m3", "tensor", amax_in=am_ref)
        assert np.array_equal(codes[r].cpu().numpy(), cr) and scales[r].item() == sr[0, 0]
        cl.append(cr)
        sl.append(sr)
    out = L.decode_reduce(codes, scales, fw.E4M3, fw.SCALE_TENSOR)
    ref = G.dequant_reduce(cl, sl, "e4m3", "tensor")
    err = rel_fro(out.cpu().numpy(), ref)
    assert err <= 1e-6, err
    assert L.flags() == 0


def test_selective_gift_fc2(fw):
    """A rank-32 fc2 layer of the deployment: statistics of its bf16
    activations, refresh, encode of R replicas and the decoded mean, against
    the oracle (the oracle factors the GPU's A with the same Omega)."""
    layer = 3
    alpha = float(synth.selective_alphas()[layer])
    m, d, T = 1536, 6144, 8192
    print(f"[selective rank-32 fc2, alpha {alpha:.3f}]", flush=True)
    QA = synth.haar(d, synth.seed_for(3, synth.ROLE_QA, layer))
    acts = [synth.gaussian_rows(T, d, alpha, QA, synth.seed_for(3, synth.ROLE_A, layer, r), DEV, torch.bfloat16)
            for r in range(R)]
    dels = [synth.gaussian_rows(T, m, 1.0, None, synth.seed_for(3, synth.ROLE_DELTA, layer, r), DEV,
                                torch.bfloat16) for r in range(R)]
    Ws = [synth.layer_gradient(dl, a).contiguous() for dl, a in zip(dels, acts)]
    om = synth.omega(d, 48, synth.seed_for(3, synth.ROLE_OMEGA, layer), DEV)
    L = fw.Layer(m, d, "lowrank", device=DEV)
    L.accumulate_stats(acts[0], commit=True)
    L.refresh(om)
    A = L.buffers()["A"].double().cpu().numpy()
    A_ref = G.second_moment(acts[0].float().cpu().numpy())
    assert rel_fro(A, A_ref) <= 1e-5
    fac = G.lowrank_factor(A, om.cpu().numpy(), 32, 4, G.damping(A))
    Tm, Tinv = G.transform_lowrank(fac)
    codes = torch.empty(R, m, d, dtype=torch.uint8, device=DEV)
    scales = torch.empty(R, 1, dtype=torch.float32, device=DEV)
    whit = torch.empty(m, d, device=DEV)
    for r in range(R):
        L.encode(Ws[r], fw.E4M3, fw.SCALE_TENSOR, codes=codes[r], scales=scales[r],
                 whitened=whit if r == 0 else None)
    out = L.decode_reduce(codes, scales, fw.E4M3, fw.SCALE_TENSOR)
    torch.cuda.synchronize()
    assert L.flags() == 0
    e = G.encode(Ws[0].cpu().numpy(), Tm, "e4m3", "tensor")
    assert rel_fro(whit.cpu().numpy(), e["whitened"]) <= 1e-5
    assert_codes(codes[0].cpu().numpy(), e["codes"])
    cl = [codes[r].cpu().numpy() for r in range(R)]
    sl = [scales[r].cpu().numpy().reshape(1, 1) for r in range(R)]
    ref = G.decode_reduce(cl, sl, Tinv, "e4m3", "tensor")
    err = rel_fro(out.cpu().numpy(), ref)
    print(f"  decoded rel err {err:.3e}", flush=True)
    assert err <= 1e-5
