"""Route choice of the persistent kernels (their workgroups wait on one
another, so they run only when the whole grid can be resident at once) and
the span guard of their 32-bit buffer offsets.  The fallback is forced from
the host with a cap on the co-resident workgroups: no kernel ever waits on a
workgroup that cannot run."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu


@pytest.fixture
def fw():
    import fac_whitening_amd as fw
    yield fw
    fw.set_max_resident(0)


def _layer(fw, m, d, seed=0):
    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev).manual_seed(seed)
    L = fw.Layer(m, d, "lowrank", rank=32, device=dev)
    a = torch.randn(4096, d, generator=g, device=dev).to(torch.bfloat16)
    L.accumulate_stats(a, fw.SIDE_A, commit=True)
    L.refresh(torch.randn(d, 48, generator=g, device=dev))
    Ws = [torch.randn(m, d, generator=g, device=dev) * 1e-3 for _ in range(4)]
    return L, Ws


def _unit(fw, L, Ws):
    out = []
    for W in Ws:
        out.append(L.encode(W, fw.E4M3, fw.SCALE_TENSOR))
    codes = torch.stack([c for c, _ in out])
    scales = torch.stack([s for _, s in out])
    return codes, scales, L.decode_reduce(codes, scales, fw.E4M3, fw.SCALE_TENSOR)


def test_cap_forces_the_multi_kernel_route(fw):
    m, d = 192, 3072                       # 4 x 4 tiles of 48 x 768
    L, Ws = _layer(fw, m, d)
    assert L.route("encode") == "fused" and L.route("decode", R=4) == "fused"
    c0, s0, o0 = _unit(fw, L, Ws)
    fw.set_max_resident(15)                # one tile short
    assert L.route("encode") == "multi" and L.route("decode", R=4) == "multi"
    c1, s1, _ = _unit(fw, L, Ws)
    o1 = L.decode_reduce(c0, s0, fw.E4M3, fw.SCALE_TENSOR)   # the same payloads on the other route
    fw.set_max_resident(16)                # exactly enough
    assert L.route("encode") == "fused"
    torch.cuda.synchronize()
    assert L.flags() == 0
    # the two routes agree to the parity bar: >= 99.9 % of the codes equal,
    # the rest one code step away; the decoded means of the same payloads
    # within 1e-5
    same = (c0 == c1).float().mean().item()
    assert same >= 0.999
    diff = (c0.int() - c1.int()).abs()
    assert int(diff[c0 != c1].max().item() if (c0 != c1).any() else 0) <= 1
    torch.testing.assert_close(s1, s0, rtol=1e-6, atol=0)
    rel = ((o1.double() - o0.double()).norm() / o0.double().norm()).item()
    assert rel < 1e-5


def test_span_guard_of_the_buffer_offsets(fw):
    m, d = 1536, 6144
    L, _ = _layer(fw, m, d)
    assert L.route("encode", ld=d) == "fused"
    # (m - 1) ld 4 + 4 d >= 2^31: the 32-bit offsets of the fused kernels
    # cannot address the rows, so the multi-kernel route is taken
    big = (2 ** 31 // 4 - d) // (m - 1) + 4
    big -= big % 4
    assert ((m - 1) * big + d) * 4 >= 2 ** 31
    assert L.route("encode", ld=big) == "multi"
    assert L.route("decode", ld=big, R=8) == "multi"
    small = big - 8
    assert ((m - 1) * small + d) * 4 < 2 ** 31
    assert L.route("encode", ld=small) == "fused"


def test_statistics_grid_under_a_cap_is_bit_exact(fw):
    """Integer-valued bf16 activations make every partial sum exact: the
    statistics kernel on a grid shrunk to 3 workgroups (each tile then split
    over several of them, handing over through the layer state) gives the
    same A bit for bit."""
    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev).manual_seed(3)
    n, T = 1024, 2048
    a = torch.randint(-8, 9, (T, n), generator=g, device=dev).to(torch.bfloat16)
    outs = []
    for cap in (0, 3):
        fw.set_max_resident(cap)
        L = fw.Layer(16, n, "diag", device=dev)
        L.accumulate_stats(a, fw.SIDE_A, commit=True)
        torch.cuda.synchronize()
        assert L.flags() == 0
        outs.append(L.buffers()["A"].clone())
    ref = (a.double().cpu().T @ a.double().cpu()) / T
    assert torch.equal(outs[0].cpu(), ref.float())
    assert torch.equal(outs[1], outs[0])


def test_two_streams_give_the_single_stream_results(fw):
    """Two layers driven from two streams, their persistent calls
    interleaved (the library orders persistent launches device-wide when the
    stream changes): codes and decoded means equal those of one stream."""
    m, d = 192, 3072
    La, Wa = _layer(fw, m, d, seed=5)
    Lb, Wb = _layer(fw, m, d, seed=6)
    ref = [_unit(fw, La, Wa), _unit(fw, Lb, Wb)]
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    got = [[], []]
    for W_a, W_b in zip(Wa, Wb):
        with torch.cuda.stream(s1):
            got[0].append(La.encode(W_a, fw.E4M3, fw.SCALE_TENSOR))
        with torch.cuda.stream(s2):
            got[1].append(Lb.encode(W_b, fw.E4M3, fw.SCALE_TENSOR))
    outs = []
    for L, g_, s in ((La, got[0], s1), (Lb, got[1], s2)):
        with torch.cuda.stream(s):
            c = torch.stack([x for x, _ in g_])
            sc = torch.stack([y for _, y in g_])
            outs.append((c, sc, L.decode_reduce(c, sc, fw.E4M3, fw.SCALE_TENSOR)))
    torch.cuda.synchronize()
    assert La.flags() == 0 and Lb.flags() == 0
    for (c0, s0, o0), (c1, s1_, o1) in zip(ref, outs):
        assert torch.equal(c0, c1) and torch.equal(s0, s1_) and torch.equal(o0, o1)
