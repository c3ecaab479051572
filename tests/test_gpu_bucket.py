"""Flat gradient buckets (gift_bucket_*): the Euclidean FP8 codec over a
whole buffer of tensors in one launch per phase, per tensor or per 512
elements, against the oracle.

Pages: GIFT 阅读笔记 Algorithm 1, the Euclidean branch (local amax, AllReduceMax, one
shared scale, quantise, AllReduceSum, dequantise, divide by N) for every
layer outside the selected set; the per-block Euclidean baseline with block
size 512 (experiment setup; reading R13 of the oracle).

Codes, scales and amax are bit-exact against the oracle on the same inputs;
the decoded mean is within the fp32 rounding of a sum of R terms.  At the
size of the 600M-class buffer the oracle checks sampled tensors (the codec
of one tensor does not depend on the others).
"""
import numpy as np
import pytest
import torch

import synth
from oracle import gift as G
from tests.helpers import rel_fro

pytestmark = pytest.mark.gpu
DEV = "cuda"
SIZES = [1536 * 1536, 4, 2800, 512, 2048 * 3 + 4, 6144 * 64, 516, 2048]


@pytest.fixture(scope="module")
def fw():
    import fac_whitening_amd as fw
    return fw


def _tensors(sizes, seed):
    rng = np.random.default_rng(seed)
    return [(rng.standard_t(4, n) * 10.0 ** rng.uniform(-4, 2)).astype(np.float32) for n in sizes]


def _flat(ts):
    return torch.from_numpy(np.concatenate(ts)).to(DEV)


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
@pytest.mark.parametrize("scaling", ["tensor", "block512"])
def test_bucket_against_oracle(fw, scaling, fmt):
    R = 4
    print(f"[bucket {scaling} {fmt}]", flush=True)
    blk = 512 if scaling == "block512" else None
    B = fw.Bucket(SIZES, fw.SCALE_BLOCK512 if blk else fw.SCALE_TENSOR, device=DEV)
    assert B.numel == sum(SIZES)
    reps = [_tensors(SIZES, 10 + r) for r in range(R)]
    grads = [_flat(ts) for ts in reps]
    f = fw.FORMATS[fmt]
    # local scale: amax per block, codes and scales bit for bit
    am = B.amax(grads[0])
    c, sc = B.encode(grads[0], f, amax_out=(am_out := torch.empty(B.nscales, device=DEV)))
    cr, sr, ar = G.bucket_quantize(reps[0], fmt, blk)
    torch.cuda.synchronize()
    assert np.array_equal(am.cpu().numpy(), ar.astype(np.float32))
    assert np.array_equal(am_out.cpu().numpy(), ar.astype(np.float32))
    assert np.array_equal(c.cpu().numpy(), cr) and np.array_equal(sc.cpu().numpy(), sr)
    # shared scale (AllReduceMax over the replicas), then the decoded mean
    shared = torch.stack([B.amax(g) for g in grads]).max(dim=0).values
    stride = -(-B.numel // 16) * 16     # replica rows 16-byte aligned
    codes = torch.empty(R, stride, dtype=torch.uint8, device=DEV)[:, :B.numel]
    scales = torch.empty(R, B.nscales, device=DEV)
    cl, sl = [], []
    for r in range(R):
        B.encode(grads[r], f, amax_in=shared, codes=codes[r], scales=scales[r])
        cq, sq, _ = G.bucket_quantize(reps[r], fmt, blk, amax_in=shared.cpu().numpy())
        assert np.array_equal(codes[r].cpu().numpy(), cq) and np.array_equal(scales[r].cpu().numpy(), sq)
        cl.append(cq)
        sl.append(sq)
    out = B.decode_reduce(codes, scales, f)
    ref = G.bucket_dequant_reduce(cl, sl, SIZES, fmt, blk)
    torch.cuda.synchronize()
    assert rel_fro(out.cpu().numpy(), ref) <= 1e-6
    assert B.flags() == 0
    B.close()


def test_bucket_nonfinite(fw):
    """An Inf in one tensor: that tensor's scale NaN, its codes 0x7F, the
    flag set; the other tensors encoded as usual."""
    sizes = [1024, 4096, 2048]
    ts = _tensors(sizes, 3)
    ts[1][100] = np.inf
    B = fw.Bucket(sizes, fw.SCALE_TENSOR, device=DEV)
    c, sc = B.encode(_flat(ts), fw.E4M3)
    cr, sr, _ = G.bucket_quantize(ts, "e4m3")
    torch.cuda.synchronize()
    assert B.flags() & fw.FLAG_NONFINITE
    assert np.array_equal(c.cpu().numpy(), cr)
    s = sc.cpu().numpy()
    assert np.isnan(s[1]) and s[0] == sr[0] and s[2] == sr[2]
    B.close()


@pytest.mark.parametrize("scaling", ["tensor", "block512"])
def test_bucket_selective_buffer_sampled(fw, scaling):
    """The 155 Euclidean gradients of the 600M-class selective deployment in
    one bucket (3.5 GB fp32): shared amax over R = 2 replicas, encode and
    decode-reduce of the whole buffer; sampled tensors (first, middle, last,
    one of each shape) against the oracle."""
    R = 2
    blk = 512 if scaling == "block512" else None
    eu = [(l, name, mo, di, alpha) for (l, name, mo, di, alpha, gift) in synth.selective_tensors() if not gift]
    assert len(eu) == 155
    sizes = [mo * di for (_, _, mo, di, _) in eu]
    print(f"[bucket selective {scaling}: {len(eu)} tensors, {sum(sizes)} values]", flush=True)
    B = fw.Bucket(sizes, fw.SCALE_BLOCK512 if blk else fw.SCALE_TENSOR, device=DEV)
    grads = []
    for r in range(R):
        g = torch.empty(B.numel, device=DEV)
        off = 0
        for k, (l, name, mo, di, alpha) in enumerate(eu):
            g[off:off + mo * di] = synth.direct_gradient(mo, di, alpha, 8192, synth.seed_for(6, k, r), DEV).reshape(-1)
            off += mo * di
        grads.append(g)
    shared = torch.maximum(B.amax(grads[0]), B.amax(grads[1]))
    codes = torch.empty(R, -(-B.numel // 16) * 16, dtype=torch.uint8, device=DEV)[:, :B.numel]
    scales = torch.empty(R, B.nscales, device=DEV)
    for r in range(R):
        B.encode(grads[r], fw.E4M3, amax_in=shared, codes=codes[r], scales=scales[r])
    out = B.decode_reduce(codes, scales, fw.E4M3)
    torch.cuda.synchronize()
    assert B.flags() == 0
    eoff = np.concatenate([[0], np.cumsum(sizes)])
    nsc = [1 if blk is None else -(-n // 512) for n in sizes]
    soff = np.concatenate([[0], np.cumsum(nsc)])
    picks = {0, len(eu) // 2, len(eu) - 1}
    for shape in {(mo, di) for (_, _, mo, di, _) in eu}:
        picks.add(next(k for k, t in enumerate(eu) if (t[2], t[3]) == shape))
    sh = shared.cpu().numpy()
    for k in sorted(picks):
        e0, e1, s0, s1 = eoff[k], eoff[k + 1], soff[k], soff[k + 1]
        cl, sl = [], []
        for r in range(R):
            x = grads[r][e0:e1].cpu().numpy()
            cq, sq, _ = G.quantize_flat(x, "e4m3", blk, amax_in=sh[s0:s1])
            assert np.array_equal(codes[r, e0:e1].cpu().numpy(), cq), (k, r)
            assert np.array_equal(scales[r, s0:s1].cpu().numpy(), sq), (k, r)
            cl.append(cq)
            sl.append(sq)
        ref = G.bucket_dequant_reduce(cl, sl, [e1 - e0], "e4m3", blk)
        assert rel_fro(out[e0:e1].cpu().numpy(), ref) <= 1e-6, k
    B.close()
