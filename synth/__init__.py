"""Seeded synthetic workloads for the GIFT encode/decode path.

This module only draws inputs.  It holds none of the method's arithmetic (no
statistics, factor, whitening, scaling or quantisation): the same bytes are
handed to the HIP library and to the CPU oracle, and each of them computes
the method on its own.

Workloads (shapes and distributions of the pages' layers: GIFT 阅读笔记,
§实验设置 -- Llama-300M / Llama-600M MLP layers, fc2 = d_ff -> d_model):

* activations   a ~ N(0, Q diag(i^-alpha) Q^T), Q Haar-orthogonal, i = 1..d
* output grads  delta ~ N(0, diag(j^-beta)) (or rotated by a second Haar Q)
* gradient      W_g = delta^T a / T (the weight gradient of a linear layer),
                one independent (a, delta) draw per data-parallel replica
* test matrix   Omega ~ N(0, 1), [d][k + p]
* stress        W_ji = t_ji c_i, t ~ Student-t(3), c_i = i^-1.5, 0.1 % of the
                columns multiplied by 100

Seeds: numpy SeedSequence(0, spawn_key=(cfg, role, layer, replica, step))
-> a 64-bit seed for a torch.Generator on the target device.  Roles:
0 Haar Q_A, 1 a, 2 delta, 3 Omega, 4 layer exponents, 5 outlier columns,
6 Student-t, 7 Haar Q_G.

Everything is drawn in float32 on ``device`` (the Haar matrix in float64 on
the CPU, so it is the same on every device); bf16 tensors are the RNE cast of
the float32 draw.  The values on a CUDA device differ from those on the CPU
for the same seed; a test always hands the same tensor to both sides.
"""
from __future__ import annotations

import dataclasses

import numpy as np
import torch

ROLE_QA, ROLE_A, ROLE_DELTA, ROLE_OMEGA, ROLE_EXP, ROLE_OUTLIER, ROLE_T, ROLE_QG = range(8)


def seed_for(cfg: int, role: int, layer: int = 0, replica: int = 0, step: int = 0) -> int:
    ss = np.random.SeedSequence(0, spawn_key=(cfg, role, layer, replica, step))
    return int(ss.generate_state(1, dtype=np.uint64)[0] & 0x7FFFFFFFFFFFFFFF)


def generator(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def haar(d: int, seed: int) -> torch.Tensor:
    """Haar-distributed orthogonal [d][d] float64 (CPU): QR of a Gaussian
    matrix with the columns multiplied by sign(diag R) (Mezzadri 2007)."""
    z = torch.randn(d, d, generator=generator(seed, "cpu"), dtype=torch.float64)
    q, r = torch.linalg.qr(z)
    return q * torch.sign(torch.diagonal(r)).unsqueeze(0)


def power_spectrum(n: int, alpha: float) -> torch.Tensor:
    return torch.arange(1, n + 1, dtype=torch.float64) ** (-alpha)


def gaussian_rows(T: int, n: int, alpha: float, Q, seed: int, device, dtype=torch.float32):
    """[T][n] rows ~ N(0, Q diag(i^-alpha) Q^T) (Q None: no rotation)."""
    z = torch.randn(T, n, generator=generator(seed, device), device=device, dtype=torch.float32)
    z = z * power_spectrum(n, alpha).sqrt().to(device=device, dtype=torch.float32)
    if Q is not None:
        z = z @ Q.to(device=device, dtype=torch.float32).T
    return z.to(dtype)


def layer_gradient(delta: torch.Tensor, a: torch.Tensor) -> torch.Tensor:
    """W_g = delta^T a / T in float32 from the stored (possibly bf16) values."""
    T = a.shape[0]
    return (delta.float().T @ a.float()) / T


def omega(d: int, l: int, seed: int, device) -> torch.Tensor:
    return torch.randn(d, l, generator=generator(seed, device), device=device, dtype=torch.float32)


def student_t(shape, nu: int, seed: int, device) -> torch.Tensor:
    """t = z / sqrt(chi2_nu / nu), chi2_nu a sum of nu squared normals."""
    g = generator(seed, device)
    z = torch.randn(*shape, generator=g, device=device)
    c = torch.zeros(*shape, device=device)
    for _ in range(nu):
        c += torch.randn(*shape, generator=g, device=device) ** 2
    return z / torch.sqrt(c / nu)


@dataclasses.dataclass
class LayerCase:
    """One layer of one configuration: R replica gradients, the activations
    (and output grads) of replica 0 for each statistics step, and Omega."""
    W: list            # R tensors [m][d] float32
    a_steps: list      # per step: activations [T][d] (replica 0)
    delta_steps: list  # per step: output grads [T][m] (replica 0)
    omega: torch.Tensor
    cfg: dict


# Configurations (shapes, distributions, replica counts).
CONFIGS = {
    # Tiny single layer, fp32 activations (oracle in seconds).
    1: dict(name="tiny", m=64, d=256, T=1024, alpha=1.5, beta=1.0, rot_G=False,
            act_dtype=torch.float32, R=4, steps=1, ema=0.0, fmt="e4m3", scaling="tensor"),
    # Llama-300M-class fc2 gradient, bf16 activations, EMA over 4 steps.
    2: dict(name="fc2_300m", m=1024, d=4096, T=8192, alpha=1.2, beta=1.0, rot_G=False,
            act_dtype=torch.bfloat16, R=8, steps=4, ema=0.95, fmt="e4m3", scaling="tensor"),
    # Llama-600M-class fc2 layer (two-sided ablation and the throughput unit).
    4: dict(name="fc2_600m", m=1536, d=6144, T=16384, alpha=1.5, beta=1.0, rot_G=True,
            act_dtype=torch.bfloat16, R=8, steps=1, ema=0.0, fmt="e4m3", scaling="block"),
}


def make_layer(cfg_id: int, device="cpu", R=None, steps=None, T=None, m=None, d=None,
               layer: int = 0, k: int = 32, p: int = 16) -> LayerCase:
    """Draw one layer case of configuration ``cfg_id``."""
    c = dict(CONFIGS[cfg_id])
    if R is not None:
        c["R"] = R
    if steps is not None:
        c["steps"] = steps
    if T is not None:
        c["T"] = T
    if m is not None:
        c["m"] = m
    if d is not None:
        c["d"] = d
    m_, d_, T_ = c["m"], c["d"], c["T"]
    QA = haar(d_, seed_for(cfg_id, ROLE_QA, layer))
    QG = haar(m_, seed_for(cfg_id, ROLE_QG, layer)) if c["rot_G"] else None
    a_steps, delta_steps, W = [], [], []
    for s in range(c["steps"]):
        a_steps.append(gaussian_rows(T_, d_, c["alpha"], QA, seed_for(cfg_id, ROLE_A, layer, 0, s),
                                     device, c["act_dtype"]))
        delta_steps.append(gaussian_rows(T_, m_, c["beta"], QG, seed_for(cfg_id, ROLE_DELTA, layer, 0, s),
                                         device, c["act_dtype"]))
    last = c["steps"] - 1
    for r in range(c["R"]):
        if r == 0:
            a, dl = a_steps[last], delta_steps[last]
        else:
            a = gaussian_rows(T_, d_, c["alpha"], QA, seed_for(cfg_id, ROLE_A, layer, r, last), device,
                              c["act_dtype"])
            dl = gaussian_rows(T_, m_, c["beta"], QG, seed_for(cfg_id, ROLE_DELTA, layer, r, last), device,
                               c["act_dtype"])
        W.append(layer_gradient(dl, a).contiguous())
    l = min(k + p, d_)
    om = omega(d_, l, seed_for(cfg_id, ROLE_OMEGA, layer), device)
    return LayerCase(W=W, a_steps=a_steps, delta_steps=delta_steps, omega=om, cfg=c)


# Llama-600M-class selective deployment: 24 decoder layers, each with
# q, k, v, o (1536 x 1536), fc1, fc3 (6144 x 1536: d_out x d_in) and fc2
# (1536 x 6144); 13 fc2 layers take the rank-32 path, the other tensors the
# Euclidean one.  Per-layer anisotropy exponents alpha_l ~ U[0.8, 1.8].
SELECTIVE_SHAPES = {"q": (1536, 1536), "k": (1536, 1536), "v": (1536, 1536), "o": (1536, 1536),
                    "fc1": (6144, 1536), "fc3": (6144, 1536), "fc2": (1536, 6144)}
SELECTIVE_LAYERS, SELECTIVE_GIFT = 24, 13


def selective_alphas(n_layers: int = SELECTIVE_LAYERS) -> np.ndarray:
    """alpha_l ~ U[0.8, 1.8], one per decoder layer."""
    rng = np.random.default_rng(seed_for(3, ROLE_EXP))
    return rng.uniform(0.8, 1.8, n_layers)


def selective_tensors(n_layers: int = SELECTIVE_LAYERS, n_gift: int = SELECTIVE_GIFT):
    """(layer, name, d_out, d_in, alpha, gift) for every weight gradient of the
    selective deployment; the fc2 tensors of layers 0 .. n_gift - 1 are the
    rank-32 ones."""
    al = selective_alphas(n_layers)
    out = []
    for l in range(n_layers):
        for name, (mo, di) in SELECTIVE_SHAPES.items():
            out.append((l, name, mo, di, float(al[l]), name == "fc2" and l < n_gift))
    return out


def direct_gradient(m: int, d: int, alpha: float, T: int, seed: int, device) -> torch.Tensor:
    """The Gaussian limit of delta^T a / T without drawing the T tokens:
    W = diag(sigma) Z diag(i^-alpha/2) / sqrt(T), sigma_j = j^-1/2, Z iid
    N(0, 1) [d_out][d_in] (no input-side rotation: it changes neither the
    sizes nor the value distribution the codec sees)."""
    z = torch.randn(m, d, generator=generator(seed, device), device=device, dtype=torch.float32)
    rs = power_spectrum(m, 1.0).sqrt().to(device=device, dtype=torch.float32)
    cs = power_spectrum(d, alpha).sqrt().to(device=device, dtype=torch.float32)
    return (z * rs.unsqueeze(1) * cs.unsqueeze(0) / float(T) ** 0.5).contiguous()


def stress_gradient(m: int, d: int, seed_layer: int, replica: int, device,
                    outlier_frac: float = 1e-3, outlier_mult: float = 100.0) -> torch.Tensor:
    """Heavy-tailed gradient: W_ji = t_ji c_i, t ~ Student-t(3), c_i = i^-1.5,
    with round(outlier_frac d) seeded outlier columns scaled by outlier_mult."""
    t = student_t((m, d), 3, seed_for(5, ROLE_T, seed_layer, replica), device)
    cscale = power_spectrum(d, 1.5).to(device=device, dtype=torch.float32)
    n_out = max(1, int(round(outlier_frac * d)))
    g = generator(seed_for(5, ROLE_OUTLIER, seed_layer), "cpu")
    cols = torch.randperm(d, generator=g)[:n_out].to(device)
    cscale[cols] *= outlier_mult
    return (t * cscale).contiguous()


def stress_activations(T: int, d: int, seed_layer: int, device, outlier_frac=1e-3, outlier_mult=100.0):
    """Activations for the stress layer: rows z * c with z ~ Student-t(3) and
    the same column scales (and outlier columns) as the gradient, no rotation."""
    z = student_t((T, d), 3, seed_for(5, ROLE_A, seed_layer), device)
    cscale = power_spectrum(d, 1.5).to(device=device, dtype=torch.float32)
    n_out = max(1, int(round(outlier_frac * d)))
    g = generator(seed_for(5, ROLE_OUTLIER, seed_layer), "cpu")
    cols = torch.randperm(d, generator=g)[:n_out].to(device)
    cscale[cols] *= outlier_mult
    return (z * cscale).to(torch.bfloat16)
