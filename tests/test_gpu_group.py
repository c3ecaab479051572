"""Grouped rank-k layers: one launch encodes several layers, one launch
decode-reduces them ("GIFT 阅读笔记", Algorithm 1, every selected layer per
step).  Checked against the single-layer calls on the same inputs: codes,
scales and decoded means bit-identical, over two steps (the per-layer call
epochs advance), per tensor and per 128 x 128 block, with layers of
different shapes (ragged tiles included)."""
import pytest
import torch

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _layer(fw, m, d, seed):
    g = torch.Generator(device=DEV).manual_seed(seed)
    L = fw.Layer(m, d, "lowrank", rank=32, device=DEV)
    a = torch.randn(2048, d, generator=g, device=DEV).to(torch.bfloat16)
    L.accumulate_stats(a, fw.SIDE_A, commit=True)
    L.refresh(torch.randn(d, 48, generator=g, device=DEV))
    return L, g


@pytest.mark.parametrize("scaling", [0, 1])
@pytest.mark.parametrize("R", [8, 3])
def test_group_matches_single_layer_calls(scaling, R):
    import fac_whitening_amd as fw
    shapes = [(1536, 6144), (200, 3000), (96, 1536)]
    items, refs = [], []
    for k, (m, d) in enumerate(shapes):
        L, g = _layer(fw, m, d, 40 + k)
        nb = fw.nblocks(m, d, scaling)
        Ws = [torch.randn(m, d, generator=g, device=DEV) * 1e-3 for _ in range(2)]
        rcodes = torch.empty(R, m, d, dtype=torch.uint8, device=DEV)
        rscales = torch.empty(R, nb, dtype=torch.float32, device=DEV)
        for r in range(R):
            W = torch.randn(m, d, generator=g, device=DEV) * 1e-3
            L.encode(W, fw.E4M3, scaling, codes=rcodes[r], scales=rscales[r])
        items.append(dict(layer=L, W=Ws[0].clone(), codes=torch.empty(m, d, dtype=torch.uint8, device=DEV),
                          scales=torch.empty(nb, dtype=torch.float32, device=DEV), rcodes=rcodes, rscales=rscales,
                          out=torch.empty(m, d, dtype=torch.float32, device=DEV)))
        refs.append(Ws)
    G = fw.Group(items, R, fw.E4M3, scaling, device=DEV)
    for step in range(2):
        for it, Ws in zip(items, refs):
            it["W"].copy_(Ws[step])
        G.encode()
        G.decode_reduce()
        torch.cuda.synchronize()
        for it, Ws in zip(items, refs):
            L = it["layer"]
            c, s = L.encode(Ws[step], fw.E4M3, scaling)
            o = L.decode_reduce(it["rcodes"], it["rscales"], fw.E4M3, scaling)
            torch.cuda.synchronize()
            assert L.flags() == 0
            assert torch.equal(it["codes"], c) and torch.equal(it["scales"], s)
            assert torch.equal(it["out"], o)
    G.close()
