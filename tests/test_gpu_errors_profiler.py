"""Host-forced failure paths and the boundary-hit profiler on the GPU.

Every failure here is raised by the host checks before anything is enqueued,
or is a documented sticky flag set by a kernel that still exits normally.
Profiler: GIFT 阅读笔记 §简化三, Fig. 3 (boundary-hit rate, knee selection).
"""
import ctypes

import numpy as np
import pytest
import torch

from oracle import gift as G

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module")
def fw():
    import fac_whitening_amd as fw
    return fw


def _status(excinfo):
    return excinfo.value.status


def test_not_ready_paths(fw):
    print("[not ready]", flush=True)
    L = fw.Layer(16, 64, "lowrank", device=DEV)
    W = torch.randn(16, 64, device=DEV)
    with pytest.raises(fw.GiftError) as e:
        L.encode(W)
    assert _status(e) == 3
    with pytest.raises(fw.GiftError) as e:
        L.refresh(torch.randn(64, 48, device=DEV))
    assert _status(e) == 3
    with pytest.raises(fw.GiftError) as e:
        L.commit_stats()
    assert _status(e) == 3
    with pytest.raises(fw.GiftError) as e:
        L.decode_reduce(torch.zeros(1, 16, 64, dtype=torch.uint8, device=DEV), torch.ones(1, 1, device=DEV))
    assert _status(e) == 3


def test_invalid_args_and_workspace(fw):
    print("[invalid args]", flush=True)
    L = fw.Layer(16, 64, "euclid", device=DEV)
    W = torch.randn(16, 64, device=DEV)
    lib = fw._lib
    codes = torch.empty(16, 64, dtype=torch.uint8, device=DEV)
    sc = torch.empty(1, device=DEV)
    s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    p = lambda t: ctypes.c_void_p(t.data_ptr())
    # ldw < d_in
    assert lib.gift_encode(L.handle, p(W), 32, 0, 0, None, None, p(codes), p(sc), None, p(L.work), L.work_bytes, s) == 1
    # bad format / scaling
    assert lib.gift_encode(L.handle, p(W), 64, 7, 0, None, None, p(codes), p(sc), None, p(L.work), L.work_bytes, s) == 1
    assert lib.gift_encode(L.handle, p(W), 64, 0, 5, None, None, p(codes), p(sc), None, p(L.work), L.work_bytes, s) == 1
    # misaligned W
    Wb = torch.randn(16 * 64 + 1, device=DEV)
    assert lib.gift_encode(L.handle, ctypes.c_void_p(Wb.data_ptr() + 4), 64, 0, 0, None, None, p(codes), p(sc), None,
                           p(L.work), L.work_bytes, s) == 1
    # workspace too small
    assert lib.gift_encode(L.handle, p(W), 64, 0, 0, None, None, p(codes), p(sc), None, p(L.work), 16, s) == 2
    # decode: R < 1, code stride too small
    assert lib.gift_decode_reduce(L.handle, p(codes), 0, p(sc), 1, 0, 0, 0, p(W), 64, p(L.work), L.work_bytes, s) == 1
    assert lib.gift_decode_reduce(L.handle, p(codes), 100, p(sc), 1, 2, 0, 0, p(W), 64, p(L.work), L.work_bytes, s) == 1
    # statistics side G on an input-side layer
    La = fw.Layer(16, 64, "diag", device=DEV)
    with pytest.raises(fw.GiftError) as e:
        La.accumulate_stats(torch.randn(10, 16, device=DEV), side=fw.SIDE_G)
    assert _status(e) == 1
    # state buffer too small
    h = ctypes.c_void_p()
    assert lib.gift_layer_create(ctypes.byref(La.desc), p(La.state), 256, s, ctypes.byref(h)) == 2


def test_nonfinite_statistics_flag(fw):
    print("[non-finite statistics]", flush=True)
    L = fw.Layer(16, 64, "lowrank", device=DEV)
    a = torch.randn(128, 64, device=DEV)
    a[5, 7] = float("nan")
    L.accumulate_stats(a, commit=True)
    L.refresh(torch.randn(64, 48, device=DEV))
    torch.cuda.synchronize()
    assert L.flags() & fw.FLAG_NONFINITE


def test_zero_statistics_without_damping_flag(fw):
    """A = 0 and lam = 0: rho = 0, the factor is NaN and the flag is set."""
    print("[zero statistics]", flush=True)
    for kind in ("lowrank", "diag", "chol"):
        L = fw.Layer(16, 64, kind, damping_rel=0.0, device=DEV)
        L.accumulate_stats(torch.zeros(32, 64, device=DEV), commit=True)
        L.refresh(torch.randn(64, 48, device=DEV) if kind == "lowrank" else None)
        assert L.flags() & fw.FLAG_NONFINITE, kind


def test_profiler_counts_and_selection(fw):
    print("[profiler]", flush=True)
    rng = np.random.default_rng(50)
    shapes = [(64, 256), (256, 64), (96, 96), (128, 512), (40, 200), (64, 64)]
    spread = [4.0, 0.5, 3.0, 1.0, 0.2, 2.5]
    P = fw.Profiler(len(shapes), fw.E4M3)
    want = np.zeros((len(shapes), 2), np.int64)
    steps = 3
    for st in range(steps):
        grads = []
        for (m, d), sp in zip(shapes, spread):
            g = (rng.standard_normal((m, d)) * np.exp(sp * rng.standard_normal((m, d)))).astype(np.float32)
            g[0, :3] = 0
            grads.append(g)
        P.step([torch.from_numpy(g).to(DEV) for g in grads])
        for i, g in enumerate(grads):
            u, lo = G.boundary_hits(g, "e4m3")
            want[i] += (u, lo)
    assert np.array_equal(P.counts.cpu().numpy(), want)
    scores, order, sel = P.select(max_select=4)
    ref_scores = G.layer_scores(want, [m * d for m, d in shapes], steps)
    np.testing.assert_allclose(scores, ref_scores, rtol=1e-15)
    ro, rs = G.select_layers(ref_scores, 4)
    assert order == ro and sel == rs
