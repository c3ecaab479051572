"""Statistics windows held in the workspace (GIFT_LAYER_TRANSIENT_STATS).

A layer created with the flag keeps no window sum S in its state: each
window is accumulated into the caller's workspace and committed in the same
call.  Its committed A (and G) must be bit-identical to those of a layer that
keeps S, for both statistics kernels (bf16 on the matrix cores, fp32 on the
vector units), over several EMA windows, and at the 6144-wide fc2 shape
whose tail tiles are split over workgroups.  The windows of the ordinary
layer also check that a window's first call replaces the sums left by the
previous window (S is not cleared at commit)."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


@pytest.fixture(scope="module")
def fw():
    import fac_whitening_amd as fw
    return fw


def _pair(fw, m, d, transform="diag", beta=0.0, shared_work=None):
    kw = dict(ema_decay=beta, device=DEV)
    if transform == "lowrank":
        kw.update(rank=32)
    ref = fw.Layer(m, d, transform, **kw)
    tra = fw.Layer(m, d, transform, transient_stats=True, workspace=shared_work, **kw)
    return ref, tra


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_transient_equals_kept_sum(fw, dtype):
    print(f"[transient stats] dtype {dtype}", flush=True)
    g = torch.Generator(device=DEV).manual_seed(7)
    m, d, beta = 16, 520, 0.9
    ref, tra = _pair(fw, m, d, beta=beta)
    for step in range(3):
        x = (torch.randn(1000 + 24 * step, d, generator=g, device=DEV) *
             torch.linspace(0.2, 3.0, d, device=DEV)).to(dtype)
        ref.accumulate_stats(x, commit=True)
        tra.accumulate_stats(x, commit=True)
        assert torch.equal(ref.buffers()["A"], tra.buffers()["A"]), f"window {step}"
    assert tra.counters()[:3] == [0, 0, 3]
    assert ref.flags() == 0 and tra.flags() == 0


def test_transient_two_sided_both_sides(fw):
    print("[transient stats] two-sided", flush=True)
    g = torch.Generator(device=DEV).manual_seed(8)
    m, d = 136, 264
    ref, tra = _pair(fw, m, d, transform="twosided", beta=0.5)
    for step in range(2):
        a = torch.randn(512, d, generator=g, device=DEV).to(torch.bfloat16)
        dl = torch.randn(512, m, generator=g, device=DEV).to(torch.bfloat16)
        for L in (ref, tra):
            L.accumulate_stats(a, fw.SIDE_A, commit=True)
            L.accumulate_stats(dl, fw.SIDE_G, commit=True)
        assert torch.equal(ref.buffers()["A"], tra.buffers()["A"])
        assert torch.equal(ref.buffers()["G"], tra.buffers()["G"])


def test_transient_rejects_open_windows(fw):
    print("[transient stats] argument checks", flush=True)
    _, tra = _pair(fw, 8, 64)
    x = torch.randn(32, 64, device=DEV)
    with pytest.raises(fw.GiftError):
        tra.accumulate_stats(x, commit=False)          # a window may not stay open
    with pytest.raises(fw.GiftError):
        tra.commit_stats()                             # it commits inside accumulate
    with pytest.raises(fw.GiftError):
        tra.accumulate_stats(x[:0], commit=True)       # nothing to commit
    tra.accumulate_stats(x, commit=True)               # the checks enqueued nothing
    assert tra.counters()[:3] == [0, 0, 1]


def test_transient_full_size_shared_workspace(fw):
    """fc2 1536 x 6144, 16384 bf16 tokens: 300 output tiles of 256 x 256 over
    the resident workgroups, so the tail tiles are split and handed over
    between workgroups; two transient layers share one workspace."""
    print("[transient stats] 1536 x 6144, shared workspace", flush=True)
    import synth
    case = synth.make_layer(4, device=DEV, R=1)
    x = case.a_steps[0]
    m, d = 1536, 6144
    ref = fw.Layer(m, d, "lowrank", rank=32, device=DEV)
    tra = fw.Layer(m, d, "lowrank", rank=32, device=DEV, transient_stats=True)
    tra2 = fw.Layer(m, d, "lowrank", rank=32, device=DEV, transient_stats=True, workspace=tra.work)
    ref.accumulate_stats(x, commit=True)
    tra.accumulate_stats(x, commit=True)
    tra2.accumulate_stats(x[: x.shape[0] // 2], commit=True)
    tra2.accumulate_stats(x, commit=True)              # second window through the shared workspace
    torch.cuda.synchronize()
    A_ref = ref.buffers()["A"]
    assert torch.equal(A_ref, tra.buffers()["A"])
    assert torch.equal(A_ref, tra2.buffers()["A"])     # beta = 0: the last window alone
    assert ref.state.numel() - tra.state.numel() >= d * d * 4
    assert ref.flags() == 0 and tra.flags() == 0 and tra2.flags() == 0
    # the refresh of the transient layer reads the same A
    ref.refresh(case.omega)
    tra.refresh(case.omega)
    assert torch.equal(ref.buffers()["U"], tra.buffers()["U"])
    assert np.array_equal(ref.buffers()["coef"].cpu().numpy(), tra.buffers()["coef"].cpu().numpy())
