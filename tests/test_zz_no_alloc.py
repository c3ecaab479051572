"""gift_bucket_encode_static: the bucket encode without a workspace argument
(its amax slots in the library's per-device scratch array), for callers that
cannot allocate.  Checked through the C ABI against gift_bucket_encode on the
same inputs: two calls in a row, the second on a smaller bucket (the array
keeps the first call's slots and must be cleared), then the size limit."""
import ctypes

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu


def _grad(sizes, seed, dev):
    g = torch.Generator(device=dev).manual_seed(seed)
    parts = []
    for i, n in enumerate(sizes):
        # each tensor its own scale, some blocks far apart in magnitude
        parts.append(torch.randn(n, generator=g, device=dev) * (10.0 ** (i % 5 - 3)))
    return torch.cat(parts).contiguous()


@pytest.mark.parametrize("scaling", ["tensor", "block512"])
@pytest.mark.parametrize("fmt", [0, 1])
def test_static_matches_workspace_encode_twice(scaling, fmt):
    import fac_whitening_amd as fw
    dev = torch.device("cuda:0")
    sc = fw.SCALE_TENSOR if scaling == "tensor" else fw.SCALE_BLOCK512
    cases = [[1536 * 1536, 6144 * 1536, 4096, 1536 * 6144, 520],    # a larger bucket first
             [2048, 1536 * 64, 4]]                                 # then a smaller one
    for k, sizes in enumerate(cases):
        B = fw.Bucket(sizes, scaling=sc, device=dev)
        x = _grad(sizes, 11 + k, dev)
        c_ref, s_ref = B.encode(x, fmt)
        c_st, s_st = B.encode_static(x, fmt)
        # local amax out, and the shared-amax call that needs no slots
        am = torch.empty(B.nscales, dtype=torch.float32, device=dev)
        c_st2, s_st2 = B.encode_static(x, fmt, amax_out=am)
        c_sh, s_sh = B.encode_static(x, fmt, amax_in=am * 2)
        c_shr, s_shr = B.encode(x, fmt, amax_in=am * 2)
        torch.cuda.synchronize()
        assert B.flags() == 0
        assert torch.equal(c_st, c_ref) and torch.equal(s_st, s_ref)
        assert torch.equal(c_st2, c_ref) and torch.equal(s_st2, s_ref)
        assert torch.equal(c_sh, c_shr) and torch.equal(s_sh, s_shr)
        # the local amax: the largest |x| of each scale block
        xs = x.abs()
        if sc == fw.SCALE_TENSOR:
            offs = np.cumsum([0] + sizes)
            want = torch.stack([xs[offs[i]:offs[i + 1]].max() for i in range(len(sizes))])
        else:
            want = torch.cat([torch.nn.functional.pad(xs[o:o + n], (0, (-n) % 512)).view(-1, 512).max(1).values
                              for o, n in zip(np.cumsum([0] + sizes)[:-1], sizes)])
        assert torch.equal(am, want)


def test_static_rejects_a_bucket_beyond_the_scratch():
    import fac_whitening_amd as fw
    dev = torch.device("cuda:0")
    # 262145 blocks of 512: one more than the 1 MiB scratch holds.  The check
    # is made on the host before anything is enqueued, so small dummy
    # buffers are enough.
    B = fw.Bucket([512 * 262145], scaling=fw.SCALE_BLOCK512, device=dev)
    assert B.nscales == 262145
    dummy = torch.zeros(1024, dtype=torch.float32, device=dev)
    codes = torch.zeros(1024, dtype=torch.uint8, device=dev)
    st = fw._lib.gift_bucket_encode_static(B._h, ctypes.c_void_p(dummy.data_ptr()), 0, None, None,
                                           ctypes.c_void_p(codes.data_ptr()), ctypes.c_void_p(dummy.data_ptr()),
                                           ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 2   # GIFT_ERR_WORKSPACE
    # with a shared amax no slots are needed, but this bucket's buffers are
    # not given here: the call is not made
    torch.cuda.synchronize()
    assert torch.count_nonzero(codes).item() == 0
