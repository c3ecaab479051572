"""The fidelity figures bench.py reports (RelL2, Cos, MaxErr, MSE of
"GIFT 阅读笔记" §简化一 Eq. (15), and the A-metric error of §核心想法 Eq. (6)
with G = I), computed on the device, against the oracle's metrics() on the
same arrays."""
import numpy as np
import pytest
import torch

from oracle import gift as G

pytestmark = pytest.mark.gpu


def test_bench_fidelity_matches_oracle_metrics():
    import bench
    rng = np.random.default_rng(31)
    m, d = 96, 200
    W = rng.standard_normal((m, d)).astype(np.float32)
    Wh = (W + 1e-2 * rng.standard_normal((m, d))).astype(np.float32)
    X = rng.standard_normal((400, d))
    A = X.T @ X / 400
    dev = torch.device("cuda:0")
    got = bench.fidelity(torch, torch.from_numpy(Wh).to(dev), torch.from_numpy(W).double().to(dev),
                         torch.from_numpy(A).to(dev))
    want = G.metrics(Wh, W, A)
    for k in ("RelL2", "Cos", "MaxErr", "MSE", "ARel"):
        assert got[k] == pytest.approx(want[k], rel=1e-4), k
