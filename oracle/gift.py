"""Plain CPU oracle of the GIFT encode/decode path, in float64.

TEST INFRASTRUCTURE ONLY.  Nothing under ``oracle/`` is part of the product:
only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import, call or execute it.  It shares no code, header,
table or helper with the HIP library, and the HIP library never calls it.

Sources (cited by title and section/equation):

* [Note] "GIFT 阅读笔记:量化用的坐标系,比量化器本身更重要"
  (zhongzhuzhou.org) -- the only technical page.  Sections used:
  前置知识 (Eq. 1-4, FP8 formats), 核心想法 (Eq. 5-14), 简化一 (Eq. 15-16,
  Table I), 简化二 (Eq. 17, Table II), 简化三 (Fig. 3 profiling),
  算法 1 (Algorithm 1), and the toy example (Eq. A1-A3).
* [Abstract] "GIFT: Geometry-Informed Low-precision Gradient Communication
  for LLM Pretraining" (shd-paper.top abstract page).

Every array is float64 internally; fp32 / bf16 inputs are upcast exactly.
Results that the method hands on as fp32 (the whitened tensor, the decoded
gradient) are rounded to float32 with round-to-nearest-even (``astype``).

Readings of points the pages leave open (each repeated where it is used):

R1  Low-rank transform (Note §简化二 Eq. 17 gives only A ~ U_r Lam_r U_r^T):
    T_A = U_k diag(Lt^-1/2 - rho^-1/2) U_k^T + rho^-1/2 I, the exact inverse
    square root of U_k diag(Lt) U_k^T + rho (I - U_k U_k^T); rho is the mean
    of the trailing eigenvalues, (tr A - sum Theta_k)/(d - k), clamped at 0.
R2  Damping (not on the pages): lam = 1e-3 tr(A)/d added to every
    eigenvalue / diagonal (and, for G, 1e-3 tr(G)/m).
R3  Rank-k eigenpairs by randomized subspace iteration: l = min(k+p, d)
    columns, q re-orthonormalised products after Y = A Omega, Rayleigh-Ritz
    on the final basis; iterations use the undamped A.
R4  Scale: r = fp32(FMAX / amax), y = fp32(x * r); stored scale
    s = fp32(amax / FMAX).  amax = 0 gives r = s = 0.  A non-finite amax
    gives s = NaN and every code 0x7F.
R5  "AllReduceSum" of FP8 payloads with per-worker scales (Algorithm 1,
    GIFT branch): each payload is dequantised with its own scale and the
    sum is formed in higher precision, then divided by R.
R6  One factor, from one worker's activations, is shared by all replicas
    (Algorithm 1 applies a single L_A to the reduced sum).
R7  Per-block scaling uses 128x128 tiles; edge tiles use their valid region.
R8  Boundary hit (Note §简化三): upper = code magnitude equal to the largest
    finite code; lower = nonzero input whose code is +-0.
R9  Knee (Note §简化三, "the layers before the sharp drop"): cut after the
    position with the largest ratio s_i / s_{i+1} among the first
    ``max_select`` positions (s_{i+1} = 0 with s_i > 0 counts as an infinite
    ratio; 0/0 counts as 1; ties go to the smallest i).
R10 EMA of A (not on the pages): the first commit sets A to the batch
    statistics, later commits A <- beta A + (1 - beta) A_batch.
R11 Error feedback (Note 算法 1, its error-feedback steps): the residual is added to the
    whitened tensor in float32 (U~ = fp32(W~ + R)), U~ is scaled and
    quantised, and the new residual is the float32 rounding of
    U~ - s dec(q) (one rounding of the exact difference).  The whitened
    tensor itself (W~) is what the inspection output shows; the amax and
    the codes are those of U~.
R13 Per-block Euclidean baseline (Note, experiment setup: block size 512,
    nothing more): blocks of 512 consecutive elements of each tensor's
    row-major order, restarting at every tensor; a tensor's last block may
    be shorter; each block scaled and quantised as R4 with its own amax.
    A model's Euclidean gradients form one flat bucket: the tensors one
    after another, their codes in the same order, their scales tensor by
    tensor.
R12 FP4 payload (the pages name NVFP4 without defining it): E2M1 elements
    (``oracle.fp4``) in blocks of 16 consecutive elements of a row, each
    block with an E4M3 scale, under one fp32 scale per tensor:
      g     = fp32(amax_T / (6 * 448))       (amax_T local or shared; 0 -> 0)
      sig_b = fp32(amax_b / (6 g))           (the block scale before coding)
      sc_b  = E4M3(sig_b)                    (RNE, saturating at 448)
      S_b   = fp32(dec(sc_b) * g)            (the block's effective scale)
      r_b   = fp32(1 / S_b) (0 if S_b = 0),  y = fp32(x * r_b),  q = E2M1(y)
    dequantised value S_b * dec(q).  A non-finite amax_T gives g = NaN,
    every block scale 0x7F and codes 0; a block whose amax is NaN gets scale
    0x7F and codes 0.  Every quotient and product is of float32 values
    computed exactly in float64 and rounded once to float32.
"""
from __future__ import annotations

import numpy as np

from . import fp4 as _fp4
from . import fp8 as _fp8

TRANSFORMS = ("euclid", "diag", "lowrank", "chol", "twosided")
BLOCK = 128  # R7


def _f64(x) -> np.ndarray:
    """Exact upcast of fp32 / bf16 (given as torch-free numpy) to float64."""
    return np.asarray(x).astype(np.float64)


# ---------------------------------------------------------------------------
# Statistics of the input side (and output side, two-sided ablation)
# ---------------------------------------------------------------------------

def second_moment(x) -> np.ndarray:
    """A_batch = (1/T) sum_t x_t x_t^T for x of shape [T][n].

    [Note] §前置知识 Eq. (4): A = E[a a^T] (d_in x d_in) and G = E[delta
    delta^T] (d_out x d_out), estimated over the T tokens of one batch.
    """
    x = _f64(x)
    T = x.shape[0]
    A = x.T @ x / T
    return (A + A.T) * 0.5


def ema_commit(A_prev, A_batch, beta: float) -> np.ndarray:
    """R10: first commit A = A_batch; then A = beta A_prev + (1-beta) A_batch."""
    if A_prev is None:
        return np.array(A_batch, dtype=np.float64)
    return beta * A_prev + (1.0 - beta) * A_batch


def damping(A, rel: float = 1e-3) -> float:
    """R2: lam = rel * tr(A) / n."""
    return rel * float(np.trace(A)) / A.shape[0]


# ---------------------------------------------------------------------------
# Transforms.  Each returns (T, T_inv) acting on the right of a row-major
# gradient:  W~ = W T,  W^ = U T_inv.
# ---------------------------------------------------------------------------

def transform_euclid(d: int):
    """Euclidean baseline: no change of coordinates ([Note] Algorithm 1,
    Euclidean branch)."""
    I = np.eye(d)
    return I, I.copy()


def transform_diag(A, lam: float):
    """Diagonal approximation of A ([Note] §简化二, Table II, "diagonal"):
    T = diag((A_ii + lam)^-1/2), T_inv = diag((A_ii + lam)^1/2)."""
    dg = np.diag(A) + lam
    return np.diag(dg ** -0.5), np.diag(dg ** 0.5)


def cholesky_lower(M) -> np.ndarray:
    """M = L L^T with L lower triangular and a positive diagonal ([Note]
    §核心想法 Eq. (7)); unique for symmetric positive definite M."""
    return np.linalg.cholesky(M)


def transform_cholesky(A, lam: float):
    """Full input-side whitening ([Note] §简化一 Eq. (16) with T_A = L_A^-T,
    the input-side half of Eq. (11); map back with L_A^T as in Eq. (14)).

    Row g of W is sent to L_A^-1 g, as in the toy example Eq. (A3).
    """
    d = A.shape[0]
    L = cholesky_lower(A + lam * np.eye(d))
    Linv = np.linalg.solve(L, np.eye(d))
    return Linv.T, L.T


def orth(Y) -> np.ndarray:
    """Orthonormal basis of the columns of Y (Householder QR)."""
    Q, _ = np.linalg.qr(Y)
    return Q


def lowrank_factor(A, omega, k: int, q: int, lam: float, orth_fn=orth) -> dict:
    """Rank-k factor of A by randomized subspace iteration (R3), then the
    R1 coefficients.  [Note] §简化二 Eq. (17): A ~ U_r Lam_r U_r^T, r = 32.

    omega: [d][l] test matrix, l = min(k + p, d), passed in by the caller.
    Returns U [d][k], theta [k] (Ritz values, descending), lam_t [k]
    (damped, clamped), rho (damped mean trailing eigenvalue) and the
    coefficient vectors c_enc = lam_t^-1/2 - rho^-1/2,
    c_dec = lam_t^1/2 - rho^1/2.
    """
    A = _f64(A)
    d = A.shape[0]
    Y = A @ _f64(omega)
    for _ in range(q):
        Q = orth_fn(Y)
        Y = A @ Q
    Q = orth_fn(Y)
    B = Q.T @ (A @ Q)
    B = (B + B.T) * 0.5
    theta, V = np.linalg.eigh(B)
    order = np.argsort(-theta, kind="stable")
    theta, V = theta[order], V[:, order]
    U = Q @ V[:, :k]
    th = theta[:k]
    lam_t = np.maximum(th, 0.0) + lam
    if k < d:
        rho = max((float(np.trace(A)) - float(th.sum())) / (d - k), 0.0) + lam
    else:
        rho = lam if lam > 0 else 1.0   # unused: U U^T = I when k = d
    return dict(U=U, theta=th, lam_t=lam_t, rho=rho,
                c_enc=lam_t ** -0.5 - rho ** -0.5,
                c_dec=lam_t ** 0.5 - rho ** 0.5)


def transform_lowrank(f: dict):
    """R1 in dense form:
    T = U diag(c_enc) U^T + rho^-1/2 I,  T_inv = U diag(c_dec) U^T + rho^1/2 I.
    """
    U = f["U"]
    d = U.shape[0]
    I = np.eye(d)
    T = (U * f["c_enc"]) @ U.T + f["rho"] ** -0.5 * I
    Tinv = (U * f["c_dec"]) @ U.T + f["rho"] ** 0.5 * I
    return T, Tinv


def output_factor(G, lam_G: float) -> np.ndarray:
    """L_G = chol(G + lam_G I), the output-side factor of [Note] Eq. (7),
    used by the two-sided transform Eq. (11) / Eq. (14)."""
    return cholesky_lower(G + lam_G * np.eye(G.shape[0]))


# ---------------------------------------------------------------------------
# Whitening and mapping back
# ---------------------------------------------------------------------------

def whiten(W, T, L_G=None) -> np.ndarray:
    """W~ = W T ([Note] Eq. (16)); two-sided W~ = L_G^-1 W L_A^-T (Eq. (11)).
    Computed in float64 and rounded to float32 (what is quantised)."""
    W = _f64(W)
    if L_G is not None:
        W = np.linalg.solve(L_G, W)
    return (W @ T).astype(np.float32)


def unwhiten(U, Tinv, L_G=None) -> np.ndarray:
    """W^ = U T_inv ([Note] Eq. (14), input side: U L_A^T); two-sided
    W^ = L_G U L_A^T.  float64, rounded to float32."""
    X = _f64(U) @ Tinv
    if L_G is not None:
        X = L_G @ X
    return X.astype(np.float32)


# ---------------------------------------------------------------------------
# Scale, quantise, dequantise ([Note] §前置知识 FP8: s = amax(X)/FP8_MAX,
# divide, quantise, multiply back; Algorithm 1 Scale / Q / Dequantize)
# ---------------------------------------------------------------------------

def nblocks(m: int, d: int, scaling: str):
    if scaling == "tensor":
        return (1, 1)
    return (-(-m // BLOCK), -(-d // BLOCK))


def amax(X32, scaling: str) -> np.ndarray:
    """max |x| per tensor ([1][1]) or per 128x128 tile (R7)."""
    X = np.abs(_f64(X32))
    m, d = X.shape
    bm, bd = nblocks(m, d, scaling)
    if scaling == "tensor":
        return np.array([[X.max() if X.size else 0.0]])
    out = np.zeros((bm, bd))
    for i in range(bm):
        for j in range(bd):
            out[i, j] = X[i * BLOCK:(i + 1) * BLOCK, j * BLOCK:(j + 1) * BLOCK].max()
    return out


def scale_pair(am: float, fmt: str):
    """R4: (r, s) = (fp32(FMAX/amax), fp32(amax/FMAX)); amax = 0 -> (0, 0);
    non-finite amax -> (nan, nan).  float64 division of two float32 values
    rounded once to float32 is the correctly rounded float32 quotient."""
    fmax = _fp8.FMAX[fmt]
    if not np.isfinite(am):
        return np.float32(np.nan), np.float32(np.nan)
    if am == 0.0:
        return np.float32(0.0), np.float32(0.0)
    am32 = float(np.float32(am))
    return np.float32(fmax / am32), np.float32(am32 / fmax)


def quantize(X32, fmt: str, scaling: str, amax_in=None):
    """Scale and encode a float32 tensor.  Returns (codes uint8 [m][d],
    scales float32 [bm][bd], amax float64 [bm][bd]).

    amax_in: a shared amax (the result of AllReduceMax in [Note]
    Algorithm 1, Euclidean branch); None uses the local amax.
    """
    X32 = np.asarray(X32, dtype=np.float32)
    m, d = X32.shape
    am = amax(X32, scaling) if amax_in is None else np.asarray(amax_in, dtype=np.float64).reshape(nblocks(m, d, scaling))
    bm, bd = am.shape
    codes = np.empty((m, d), dtype=np.uint8)
    scales = np.empty((bm, bd), dtype=np.float32)
    bh = m if scaling == "tensor" else BLOCK
    bw = d if scaling == "tensor" else BLOCK
    for i in range(bm):
        for j in range(bd):
            r, s = scale_pair(float(am[i, j]), fmt)
            tile = X32[i * bh:(i + 1) * bh, j * bw:(j + 1) * bw]
            if np.isnan(r):
                c = np.full(tile.shape, _fp8.NAN_CODE, dtype=np.uint8)
            else:
                y = (tile.astype(np.float64) * float(r)).astype(np.float32)
                c = _fp8.encode(y, fmt)
            codes[i * bh:(i + 1) * bh, j * bw:(j + 1) * bw] = c
            scales[i, j] = s
    return codes, scales, am


def dequantize(codes, scales, fmt: str, scaling: str) -> np.ndarray:
    """s * dec(q) per tile, float64."""
    m, d = codes.shape
    vals = _fp8.decode(codes, fmt)
    bh = m if scaling == "tensor" else BLOCK
    bw = d if scaling == "tensor" else BLOCK
    sc = np.repeat(np.repeat(_f64(scales), bh, axis=0), bw, axis=1)[:m, :d]
    return vals * sc


def dequant_reduce(codes_list, scales_list, fmt: str, scaling: str) -> np.ndarray:
    """U = (1/R) sum_r s_r dec(q_r) (R5; [Note] Eq. (1) and Algorithm 1
    AllReduceSum / Dequantize / divide by N)."""
    R = len(codes_list)
    acc = None
    for c, s in zip(codes_list, scales_list):
        v = dequantize(c, s, fmt, scaling)
        acc = v if acc is None else acc + v
    return acc / R


# ---------------------------------------------------------------------------
# Flat buckets of Euclidean tensors (Algorithm 1, the Euclidean branch; R13)
# ---------------------------------------------------------------------------

FLAT_BLOCK = 512


def quantize_flat(x, fmt: str, block=None, amax_in=None):
    """Euclidean FP8 of one tensor in its row-major order: one scale for the
    tensor (block None) or one per ``block`` consecutive elements (the last
    block may be shorter).  Each block is quantised as a 1 x n tensor with
    R4.  Returns (codes uint8 [n], scales float32 [nb], amax float64 [nb])."""
    v = np.asarray(x, dtype=np.float32).ravel()
    n = v.size
    bl = n if block is None else block
    nb = 1 if block is None else -(-n // block)
    codes = np.empty(n, dtype=np.uint8)
    scales = np.empty(nb, dtype=np.float32)
    am = np.empty(nb)
    for b in range(nb):
        seg = v[b * bl:(b + 1) * bl].reshape(1, -1)
        a_in = None if amax_in is None else np.array([[np.asarray(amax_in, dtype=np.float64).ravel()[b]]])
        c, sc, a = quantize(seg, fmt, "tensor", a_in)
        codes[b * bl:(b + 1) * bl] = c.ravel()
        scales[b] = sc[0, 0]
        am[b] = a[0, 0]
    return codes, scales, am


def dequantize_flat(codes, scales, fmt: str, block=None) -> np.ndarray:
    """s_b dec(q) per element, float64 [n]."""
    c = np.asarray(codes, dtype=np.uint8).ravel()
    n = c.size
    bl = n if block is None else block
    idx = np.arange(n) // max(bl, 1)
    return _fp8.decode(c, fmt) * _f64(scales).ravel()[idx]


def bucket_quantize(tensors, fmt: str, block=None, amax_in=None):
    """A flat bucket: each tensor quantised by ``quantize_flat``; codes and
    scales concatenated in tensor order (amax_in: the concatenated shared
    amax of every scale block, or None)."""
    cs, ss, ams = [], [], []
    off = 0
    for t in tensors:
        n = np.asarray(t).size
        nb = 1 if block is None else -(-n // block)
        a_in = None if amax_in is None else np.asarray(amax_in).ravel()[off:off + nb]
        c, sc, a = quantize_flat(t, fmt, block, a_in)
        cs.append(c)
        ss.append(sc)
        ams.append(a)
        off += nb
    return np.concatenate(cs), np.concatenate(ss), np.concatenate(ams)


def bucket_dequant_reduce(codes_list, scales_list, sizes, fmt: str, block=None) -> np.ndarray:
    """(1/R) sum_r s_r dec(q_r) over a bucket of tensors with the given
    element counts (R5), float64 [sum sizes]."""
    R = len(codes_list)
    out = []
    co = so = 0
    for n in sizes:
        nb = 1 if block is None else -(-n // block)
        acc = None
        for c, sc in zip(codes_list, scales_list):
            v = dequantize_flat(np.asarray(c).ravel()[co:co + n], np.asarray(sc).ravel()[so:so + nb], fmt, block)
            acc = v if acc is None else acc + v
        out.append(acc / R)
        co += n
        so += nb
    return np.concatenate(out) if out else np.zeros(0)


# ---------------------------------------------------------------------------
# FP4 payload (R12)
# ---------------------------------------------------------------------------

FP4_BLOCK = 16
FP4_TSCALE_DIV = _fp4.FMAX * _fp8.FMAX["e4m3"]   # 6 * 448: the largest block scale times the largest element


def quantize_fp4(X32, amax_in=None) -> dict:
    """Two-level FP4 quantiser of a float32 [m][d] tensor (d a multiple of
    16), reading R12.  Returns dict(codes uint8 [m][d] (values 0..15),
    bscales uint8 [m][d/16] (E4M3 codes), tscale float32, amax float64 (the
    amax_T used)).  amax_in: the shared per-tensor amax (AllReduceMax), or
    None for the local one."""
    X32 = np.asarray(X32, dtype=np.float32)
    m, d = X32.shape
    assert d % FP4_BLOCK == 0
    x = _f64(X32).reshape(m, d // FP4_BLOCK, FP4_BLOCK)
    am_t = float(np.abs(x).max()) if amax_in is None else float(np.asarray(amax_in, dtype=np.float64).ravel()[0])
    if x.size == 0 and amax_in is None:
        am_t = 0.0
    if not np.isfinite(am_t):
        g = np.float32(np.nan)
    else:
        g = np.float32(am_t / FP4_TSCALE_DIV)
    amax_b = np.abs(x).max(axis=2) if x.size else np.zeros((m, 0))
    with np.errstate(divide="ignore", invalid="ignore"):
        if np.isnan(g):
            sig = np.full(amax_b.shape, np.nan, dtype=np.float32)
        elif g == 0:
            sig = np.zeros(amax_b.shape, dtype=np.float32)
        else:
            sig = (amax_b / (6.0 * float(g))).astype(np.float32)
        sc = _fp8.encode(sig, "e4m3")
        S = (_fp8.decode(sc, "e4m3") * float(g)).astype(np.float32)
        r = np.where(S > 0, (1.0 / S.astype(np.float64)).astype(np.float32), np.float32(0.0))
        r = np.where(np.isnan(S), np.float32(np.nan), r).astype(np.float32)
        y = (x * r.astype(np.float64)[:, :, None]).astype(np.float32)
    codes = _fp4.encode(y)
    codes = np.where(np.isnan(S)[:, :, None], 0, codes).astype(np.uint8)
    return dict(codes=codes.reshape(m, d), bscales=sc.astype(np.uint8), tscale=g, amax=am_t)


def fp4_block_scales(bscales, tscale) -> np.ndarray:
    """S_b = fp32(dec(sc_b) * g) per block (R12), float32 [m][d/16]."""
    return (_fp8.decode(bscales, "e4m3") * float(np.float32(tscale))).astype(np.float32)


def dequantize_fp4(codes, bscales, tscale) -> np.ndarray:
    """S_b * dec(q) per element, float64 [m][d]."""
    S = fp4_block_scales(bscales, tscale).astype(np.float64)
    return _fp4.decode(codes) * np.repeat(S, FP4_BLOCK, axis=1)


def dequant_reduce_fp4(codes_list, bscales_list, tscales) -> np.ndarray:
    """U = (1/R) sum_r S_{b,r} dec(q_r) (R5 with the FP4 payload)."""
    R = len(codes_list)
    acc = None
    for c, b, t in zip(codes_list, bscales_list, tscales):
        v = dequantize_fp4(c, b, t)
        acc = v if acc is None else acc + v
    return acc / R


def error_feedback_fp4(Wt, R, amax_in=None) -> dict:
    """R11 with the FP4 payload: U~ = fp32(Wt + R), quantise U~ (R12), new
    residual fp32(U~ - S_b dec(q))."""
    Ut = (np.asarray(Wt, dtype=np.float32) + np.asarray(R, dtype=np.float32)).astype(np.float32)
    out = quantize_fp4(Ut, amax_in)
    deq = dequantize_fp4(out["codes"], out["bscales"], out["tscale"])
    out["u_tilde"] = Ut
    out["residual"] = (Ut.astype(np.float64) - deq).astype(np.float32)
    return out


def payload_bytes(m: int, d: int, scaling: str) -> int:
    """FP8: codes (1 B/element) plus one float32 scale per tile.  FP4
    ("block16", R12): half a byte per element, one E4M3 byte per 16
    elements, one float32 tensor scale."""
    if scaling == "block16":
        return m * d // 2 + m * d // FP4_BLOCK + 4
    bm, bd = nblocks(m, d, scaling)
    return m * d + 4 * bm * bd


# ---------------------------------------------------------------------------
# The whole path
# ---------------------------------------------------------------------------

def build_transform(kind: str, A=None, lam=None, omega=None, k=32, q=4,
                    G=None, lam_G=None):
    """(T, T_inv, L_G) for one of TRANSFORMS."""
    if kind == "euclid":
        d = A.shape[0] if A is not None else omega
        T, Ti = transform_euclid(d)
        return T, Ti, None
    if kind == "diag":
        T, Ti = transform_diag(A, lam)
        return T, Ti, None
    if kind == "lowrank":
        T, Ti = transform_lowrank(lowrank_factor(A, omega, k, q, lam))
        return T, Ti, None
    if kind == "chol":
        T, Ti = transform_cholesky(A, lam)
        return T, Ti, None
    if kind == "twosided":
        T, Ti = transform_cholesky(A, lam)
        return T, Ti, output_factor(G, lam_G)
    raise ValueError(kind)


def encode(W, T, fmt: str, scaling: str, L_G=None, amax_in=None):
    """[Note] Algorithm 1 (without error feedback): whiten, scale, quantise.
    Returns dict(whitened, codes, scales, amax)."""
    Wt = whiten(W, T, L_G)
    codes, scales, am = quantize(Wt, fmt, scaling, amax_in)
    return dict(whitened=Wt, codes=codes, scales=scales, amax=am)


def encode_ef(W, T, R, fmt: str, scaling: str, L_G=None, amax_in=None):
    """[Note] Algorithm 1 with error feedback (the geometry branch, R11): whiten,
    add the residual, scale, quantise, and carry the quantisation error of
    U~ to the next step.  R is the float32 residual [m][d] of the previous
    step (zeros at the first).  Returns dict(whitened, u_tilde, codes,
    scales, amax, residual)."""
    Wt = whiten(W, T, L_G)
    out = error_feedback(Wt, R, fmt, scaling, amax_in)
    out["whitened"] = Wt
    return out


def error_feedback(Wt, R, fmt: str, scaling: str, amax_in=None):
    """The error-feedback step of [Note] Algorithm 1 (its error-feedback steps, R11) on
    an already whitened float32 tensor Wt: U~ = fp32(Wt + R), scale and
    quantise U~, new residual fp32(U~ - s dec(q)).  Returns dict(u_tilde,
    codes, scales, amax, residual)."""
    Ut = (np.asarray(Wt, dtype=np.float32) + np.asarray(R, dtype=np.float32)).astype(np.float32)
    codes, scales, am = quantize(Ut, fmt, scaling, amax_in)
    deq = dequantize(codes, scales, fmt, scaling)
    Rn = (Ut.astype(np.float64) - deq).astype(np.float32)
    return dict(u_tilde=Ut, codes=codes, scales=scales, amax=am, residual=Rn)


def decode_reduce(codes_list, scales_list, Tinv, fmt: str, scaling: str, L_G=None):
    """[Note] Algorithm 1: sum the R payloads, dequantise, divide by R, map
    back with T_inv (Eq. (14)).  Returns float32 [m][d]."""
    U = dequant_reduce(codes_list, scales_list, fmt, scaling)
    return unwhiten(U, Tinv, L_G)


# ---------------------------------------------------------------------------
# Fidelity report ([Note] §简化一 Eq. (15)) and the K-FAC metric (Eq. (6))
# ---------------------------------------------------------------------------

def metrics(W_hat, W_ref, A=None) -> dict:
    """RelL2, Cos, MaxErr, MSE of W_hat against W_ref (Eq. (15)); with A,
    also the A-metric relative error sqrt(tr(E A E^T)) / sqrt(tr(W A W^T))
    (Eq. (6) with G = I)."""
    g = _f64(W_ref).ravel()
    gh = _f64(W_hat).ravel()
    e = gh - g
    out = dict(RelL2=np.linalg.norm(e) / np.linalg.norm(g),
               Cos=float(gh @ g) / (np.linalg.norm(gh) * np.linalg.norm(g)),
               MaxErr=float(np.abs(e).max()),
               MSE=float(e @ e) / e.size)
    if A is not None:
        E = _f64(W_hat) - _f64(W_ref)
        Wr = _f64(W_ref)
        A = _f64(A)
        # tr(X A X^T) as the sum of (X A) * X over all entries
        out["ARel"] = float(np.sqrt(np.sum((E @ A) * E) / np.sum((Wr @ A) * Wr)))
    return out


# ---------------------------------------------------------------------------
# Boundary-hit profiler ([Note] §简化三, Fig. 3) and layer selection
# ---------------------------------------------------------------------------

def boundary_hits(grad32, fmt: str, scaling: str = "tensor"):
    """R8: (upper, lower) counts of the Euclidean encode of one gradient
    with its local scale."""
    X = np.asarray(grad32, dtype=np.float32)
    codes, _, _ = quantize(X, fmt, scaling)
    mag = codes & 0x7F
    upper = int(np.count_nonzero(mag == _fp8.FORMATS[fmt]["max_code"]))
    lower = int(np.count_nonzero((mag == 0) & (X != 0)))
    return upper, lower


def layer_scores(counts, numel, n_steps: int) -> np.ndarray:
    """Score = mean over profiled steps of (upper + lower) / numel."""
    counts = np.asarray(counts, dtype=np.float64)
    return (counts[:, 0] + counts[:, 1]) / (np.asarray(numel, dtype=np.float64) * n_steps)


def select_layers(scores, max_select: int):
    """Rank by score (descending, ties to the lower layer index) and cut at
    the knee (R9).  Returns (order, selected)."""
    s = np.asarray(scores, dtype=np.float64)
    n = s.size
    order = sorted(range(n), key=lambda i: (-s[i], i))
    ss = s[order]
    best_i, best_ratio = 1, -1.0
    for i in range(1, min(n - 1, max_select) + 1):   # cut after position i
        a, b = ss[i - 1], ss[i]
        if b > 0:
            ratio = a / b
        elif a > 0:
            ratio = np.inf
        else:
            ratio = 1.0
        if ratio > best_ratio:
            best_i, best_ratio = i, ratio
    if n == 1:
        best_i = 1
    return order, order[:min(best_i, max_select)]


# ---------------------------------------------------------------------------
# Toy quantiser of the worked example ([Note] toy example, step 4)
# ---------------------------------------------------------------------------

def toy_quantize(v) -> np.ndarray:
    """Round every coordinate to the nearest multiple of s/8, s = max|v|."""
    v = _f64(v)
    step = np.abs(v).max() / 8.0
    return np.round(v / step) * step
