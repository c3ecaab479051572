"""Comparison helpers for the GPU-vs-oracle tests."""
import numpy as np


def rel_fro(a, b) -> float:
    """||a - b||_F / ||b||_F in float64."""
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    nb = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / (nb if nb > 0 else 1.0))


def signed_rank(codes) -> np.ndarray:
    """Position of each finite code in the sorted list of finite FP8 values,
    with +0 and -0 sharing rank 0 (code magnitudes increase with value)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    mag = c & 0x7F
    return np.where(c & 0x80, -mag, mag)


def code_agreement(got, want):
    """(fraction identical, largest step distance)."""
    g, w = np.asarray(got), np.asarray(want)
    same = float(np.mean(g == w)) if g.size else 1.0
    steps = np.abs(signed_rank(g) - signed_rank(w))
    return same, int(steps.max()) if steps.size else 0


def assert_codes(got, want, min_same=0.999, max_step=1):
    same, step = code_agreement(got, want)
    assert same >= min_same, f"identical codes {same:.6f} < {min_same}"
    assert step <= max_step, f"code step distance {step} > {max_step}"
    return same, step


def layer_with_factor(fw, m, d, fac, device):
    """A rank-32 layer whose state holds the oracle's factor (basis U and the
    coefficients c_enc, c_dec, rho^-1/2, rho^1/2), marked ready: stage
    isolation of the encode / decode kernels from the refresh."""
    import torch

    L = fw.Layer(m, d, "lowrank", device=device)
    b = L.buffers()
    b["U"].copy_(torch.from_numpy(fac["U"].astype(np.float32)))
    coef = np.zeros(68, np.float32)
    coef[:32] = fac["c_enc"]
    coef[32:64] = fac["c_dec"]
    coef[64], coef[65] = fac["rho"] ** -0.5, fac["rho"] ** 0.5
    b["coef"].copy_(torch.from_numpy(coef))
    L.mark_ready()
    return L
