"""Python binding of libgift (GIFT encode/decode on MI355X).

Argument marshalling only: every step of the path runs in the HIP kernels of
``libgift.so`` (built from ``csrc/`` by ``build.py``).  PyTorch provides the
device memory and the current stream; nothing here computes on the data.
Importing this module raises if the library has not been built: there is no
fallback.

Function names follow the C ABI in ``include/gift.h``.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libgift.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"libgift.so not built ({LIB_PATH}); run `python -m fac_whitening_amd.build` "
                      "or __graft_entry__.build()")

_lib = ctypes.CDLL(LIB_PATH)

# enums (include/gift.h)
EUCLID, DIAG, LOWRANK, CHOL_INPUT, CHOL_TWOSIDED = range(5)
E4M3, E5M2, E2M1 = 0, 1, 2
SCALE_TENSOR, SCALE_BLOCK128, SCALE_BLOCK16, SCALE_BLOCK512 = 0, 1, 2, 3
BF16, FP32 = 0, 1
SIDE_A, SIDE_G = 0, 1
LAYER_TRANSIENT_STATS = 1   # statistics windows committed in one call, S in the workspace
FLAG_NONFINITE, FLAG_SPIN_TIMEOUT = 1, 2
TRANSFORMS = {"euclid": EUCLID, "diag": DIAG, "lowrank": LOWRANK, "chol": CHOL_INPUT, "twosided": CHOL_TWOSIDED}
FORMATS = {"e4m3": E4M3, "e5m2": E5M2}
SCALINGS = {"tensor": SCALE_TENSOR, "block": SCALE_BLOCK128}
STATUS = {0: "GIFT_OK", 1: "GIFT_ERR_INVALID_ARG", 2: "GIFT_ERR_WORKSPACE", 3: "GIFT_ERR_NOT_READY",
          4: "GIFT_ERR_NUMERICAL", 5: "GIFT_ERR_UNSUPPORTED", 6: "GIFT_ERR_HIP"}

EXPORTS = [
    "gift_layer_state_bytes", "gift_layer_create", "gift_layer_destroy", "gift_layer_get_counters",
    "gift_layer_set_counters", "gift_layer_flags", "gift_layer_buffers", "gift_layer_mark_ready",
    "gift_accumulate_stats", "gift_commit_stats", "gift_refresh_factors", "gift_encode", "gift_encode_ef",
    "gift_decode_reduce", "gift_encode_fp4", "gift_decode_reduce_fp4", "gift_payload_bytes", "gift_profiler_create", "gift_profiler_destroy",
    "gift_profiler_workspace_bytes", "gift_profile_step", "gift_select_layers", "gift_status_string",
    "gift_last_hip_error", "gift_set_fused", "gift_bucket_table_bytes", "gift_bucket_create",
    "gift_bucket_destroy", "gift_bucket_sizes", "gift_bucket_flags", "gift_bucket_amax", "gift_bucket_encode",
    "gift_bucket_decode_reduce", "gift_scale_sync_due", "gift_set_max_resident", "gift_layer_route",
    "gift_bucket_encode_static", "gift_group_table_bytes", "gift_group_create", "gift_group_destroy",
    "gift_group_encode", "gift_group_decode_reduce",
]


class GroupItem(ctypes.Structure):
    _fields_ = [("layer", ctypes.c_void_p), ("d_W", ctypes.c_void_p), ("ldw", ctypes.c_int64),
                ("d_codes", ctypes.c_void_p), ("d_scales", ctypes.c_void_p), ("d_rcodes", ctypes.c_void_p),
                ("code_stride", ctypes.c_int64), ("d_rscales", ctypes.c_void_p), ("scale_stride", ctypes.c_int64),
                ("d_out", ctypes.c_void_p), ("ldo", ctypes.c_int64)]


class LayerDesc(ctypes.Structure):
    _fields_ = [("d_out", ctypes.c_int32), ("d_in", ctypes.c_int32), ("transform", ctypes.c_int32),
                ("rank", ctypes.c_int32), ("oversample", ctypes.c_int32), ("power_iters", ctypes.c_int32),
                ("ema_decay", ctypes.c_float), ("damping_rel", ctypes.c_float), ("flags", ctypes.c_int32)]


_vp, _sz, _i32, _i64 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32, ctypes.c_int64
_P = ctypes.POINTER


def _sig(name, res, *args):
    f = getattr(_lib, name)
    f.restype = res
    f.argtypes = list(args)
    return f


_sig("gift_layer_state_bytes", _i32, _P(LayerDesc), _P(_sz), _P(_sz))
_sig("gift_layer_create", _i32, _P(LayerDesc), _vp, _sz, _vp, _P(_vp))
_sig("gift_layer_destroy", _i32, _vp)
_sig("gift_layer_get_counters", _i32, _vp, _P(_i64))
_sig("gift_layer_set_counters", _i32, _vp, _P(_i64))
_sig("gift_layer_flags", _i32, _vp, _vp, _P(ctypes.c_uint32))
_sig("gift_layer_buffers", _i32, _vp, *[_P(_vp)] * 8)
_sig("gift_layer_mark_ready", _i32, _vp, _vp)
_sig("gift_accumulate_stats", _i32, _vp, _i32, _vp, _i32, _i64, _i64, _i32, _vp, _sz, _vp)
_sig("gift_commit_stats", _i32, _vp, _i32, _vp)
_sig("gift_refresh_factors", _i32, _vp, _vp, _vp, _sz, _vp)
_sig("gift_encode", _i32, _vp, _vp, _i64, _i32, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp)
_sig("gift_encode_ef", _i32, _vp, _vp, _i64, _i32, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp)
_sig("gift_encode_fp4", _i32, _vp, _vp, _i64, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp)
_sig("gift_decode_reduce_fp4", _i32, _vp, _vp, _i64, _vp, _i64, _vp, _i32, _vp, _i64, _vp, _sz, _vp)
_sig("gift_decode_reduce", _i32, _vp, _vp, _i64, _vp, _i64, _i32, _i32, _i32, _vp, _i64, _vp, _sz, _vp)
_sig("gift_payload_bytes", _sz, _i32, _i32, _i32)
_sig("gift_profiler_create", _i32, _i32, _i32, _i32, _vp, _vp, _P(_vp))
_sig("gift_profiler_destroy", _i32, _vp)
_sig("gift_profiler_workspace_bytes", _sz, _i32, _i32, _i64)
_sig("gift_profile_step", _i32, _vp, _i32, _P(_vp), _P(_i64), _vp, _sz, _vp)
_sig("gift_select_layers", _i32, _vp, _i32, _P(ctypes.c_double), _P(_i32), _P(_i32), _P(_i32), _vp)
_sig("gift_status_string", ctypes.c_char_p, _i32)
_sig("gift_last_hip_error", _i32)
_sig("gift_set_fused", _i32, _i32)
_sig("gift_set_max_resident", _i32, _i32)
_sig("gift_layer_route", _i32, _vp, _i32, _i64, _i32, _P(_i32))
_sig("gift_bucket_table_bytes", _sz, _i32)
_sig("gift_bucket_create", _i32, _i32, _P(_i64), _i32, _vp, _sz, _vp, _P(_vp))
_sig("gift_bucket_destroy", _i32, _vp)
_sig("gift_bucket_sizes", _i32, _vp, _P(_i64), _P(_i64), _P(_sz))
_sig("gift_bucket_flags", _i32, _vp, _vp, _P(ctypes.c_uint32))
_sig("gift_bucket_amax", _i32, _vp, _vp, _vp, _vp)
_sig("gift_bucket_encode", _i32, _vp, _vp, _i32, _vp, _vp, _vp, _vp, _vp, _sz, _vp)
_sig("gift_bucket_encode_static", _i32, _vp, _vp, _i32, _vp, _vp, _vp, _vp, _vp)
_sig("gift_bucket_decode_reduce", _i32, _vp, _vp, _i64, _vp, _i64, _i32, _i32, _vp, _vp)
_sig("gift_scale_sync_due", _i32, _i64, _i32)
_sig("gift_group_table_bytes", _sz, _i32)
_sig("gift_group_create", _i32, _i32, _P(GroupItem), _i32, _i32, _i32, _vp, _sz, _vp, _P(_vp))
_sig("gift_group_destroy", _i32, _vp)
_sig("gift_group_encode", _i32, _vp, _vp)
_sig("gift_group_decode_reduce", _i32, _vp, _vp)


def set_fused(enable: bool) -> bool:
    """Select the persistent single-launch rank-k kernels (True, default) or
    the multi-kernel path (False); returns the previous setting."""
    return bool(_lib.gift_set_fused(1 if enable else 0))


def set_max_resident(max_groups: int) -> int:
    """Cap the workgroups persistent launches may count on being resident at
    once (0: the device's own limit); returns the previous cap."""
    return int(_lib.gift_set_max_resident(int(max_groups)))


class GiftError(RuntimeError):
    def __init__(self, status: int, where: str):
        msg = f"{where}: {STATUS.get(status, status)} ({_lib.gift_status_string(status).decode()})"
        if status == 6:
            msg += f", hipError {_lib.gift_last_hip_error()}"
        super().__init__(msg)
        self.status = status


def _check(status: int, where: str):
    if status != 0:
        raise GiftError(status, where)


def _stream(stream=None):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def nblocks(m: int, d: int, scaling: int) -> int:
    return 1 if scaling == SCALE_TENSOR else -(-m // 128) * -(-d // 128)


def payload_bytes(d_out: int, d_in: int, scaling: int) -> int:
    return int(_lib.gift_payload_bytes(d_out, d_in, scaling))


def _alloc(nbytes: int, device) -> torch.Tensor:
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)


class Layer:
    """One layer's state and calls (gift_layer_*)."""

    def __init__(self, d_out: int, d_in: int, transform="lowrank", rank: int = 32, oversample: int = 16,
                 power_iters: int = 4, ema_decay: float = 0.0, damping_rel: float = 1e-3, device="cuda",
                 stream=None, workspace=None, transient_stats: bool = False):
        tr = TRANSFORMS[transform] if isinstance(transform, str) else int(transform)
        self.desc = LayerDesc(d_out, d_in, tr, rank, oversample, power_iters, ema_decay, damping_rel,
                              LAYER_TRANSIENT_STATS if transient_stats else 0)
        sb, wb = _sz(), _sz()
        _check(_lib.gift_layer_state_bytes(ctypes.byref(self.desc), ctypes.byref(sb), ctypes.byref(wb)),
               "gift_layer_state_bytes")
        self.device = torch.device(device)
        self.state = _alloc(sb.value, self.device)
        self.work_bytes = wb.value
        self.work = workspace if workspace is not None else _alloc(wb.value, self.device)
        h = _vp()
        _check(_lib.gift_layer_create(ctypes.byref(self.desc), _ptr(self.state), sb.value, _stream(stream),
                                      ctypes.byref(h)), "gift_layer_create")
        self._h = h
        self.m, self.d, self.k = d_out, d_in, rank

    # -- lifecycle ---------------------------------------------------------
    def close(self):
        if getattr(self, "_h", None):
            _lib.gift_layer_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    @property
    def handle(self):
        return self._h

    def counters(self):
        arr = (_i64 * 8)()
        _check(_lib.gift_layer_get_counters(self._h, arr), "gift_layer_get_counters")
        return list(arr)

    def set_counters(self, vals):
        arr = (_i64 * 8)(*vals)
        _check(_lib.gift_layer_set_counters(self._h, arr), "gift_layer_set_counters")

    def flags(self, stream=None) -> int:
        f = ctypes.c_uint32()
        _check(_lib.gift_layer_flags(self._h, _stream(stream), ctypes.byref(f)), "gift_layer_flags")
        return f.value

    def buffers(self) -> dict:
        """Views into the state buffer (device tensors), by name."""
        ptrs = [_vp() for _ in range(8)]
        _check(_lib.gift_layer_buffers(self._h, *[ctypes.byref(p) for p in ptrs]), "gift_layer_buffers")
        names = ["A", "G", "U", "coef", "tinv_a", "t_a", "lg_inv", "lg"]
        m, d = self.m, self.d
        shapes = {"A": (d, d), "G": (m, m), "U": (d, 32), "tinv_a": (d, d), "t_a": (d, d), "lg_inv": (m, m),
                  "lg": (m, m), "coef": (68,) if self.desc.transform == LOWRANK else (2 * d,)}
        base = self.state.data_ptr()
        out = {}
        for n, p in zip(names, ptrs):
            if not p.value:
                continue
            off = p.value - base
            cnt = 1
            for s in shapes[n]:
                cnt *= s
            out[n] = self.state[off:off + 4 * cnt].view(torch.float32).view(*shapes[n])
        return out

    def route(self, op: str, ld=None, R: int = 1) -> str:
        """'fused' or 'multi': the route gift_encode (op='encode') or
        gift_decode_reduce (op='decode') takes for this layer now."""
        f = _i32()
        _check(_lib.gift_layer_route(self._h, 0 if op == "encode" else 1, self.d if ld is None else ld, R,
                                     ctypes.byref(f)), "gift_layer_route")
        return "fused" if f.value else "multi"

    def mark_ready(self, stream=None):
        _check(_lib.gift_layer_mark_ready(self._h, _stream(stream)), "gift_layer_mark_ready")

    # -- statistics / refresh --------------------------------------------
    def accumulate_stats(self, x: torch.Tensor, side: int = SIDE_A, commit: bool = False, stream=None):
        dtype = BF16 if x.dtype == torch.bfloat16 else FP32
        if x.dtype not in (torch.bfloat16, torch.float32) or x.dim() != 2 or x.stride(1) != 1:
            raise ValueError("x must be a row-major [T][n] bf16 or fp32 tensor")
        _check(_lib.gift_accumulate_stats(self._h, side, _ptr(x), dtype, x.shape[0], x.stride(0), int(commit),
                                          _ptr(self.work), self.work_bytes, _stream(stream)), "gift_accumulate_stats")

    def commit_stats(self, side: int = SIDE_A, stream=None):
        _check(_lib.gift_commit_stats(self._h, side, _stream(stream)), "gift_commit_stats")

    def refresh(self, omega=None, stream=None):
        _check(_lib.gift_refresh_factors(self._h, _ptr(omega), _ptr(self.work), self.work_bytes, _stream(stream)),
               "gift_refresh_factors")

    # -- encode / decode --------------------------------------------------
    def encode(self, W: torch.Tensor, fmt=E4M3, scaling=SCALE_TENSOR, amax_in=None, codes=None, scales=None,
               amax_out=None, whitened=None, want_codes=True, resid=None, stream=None):
        fmt = FORMATS.get(fmt, fmt)
        scaling = SCALINGS.get(scaling, scaling)
        m, d = self.m, self.d
        nb = nblocks(m, d, scaling)
        if W.dtype != torch.float32 or W.shape != (m, d) or W.stride(1) != 1:
            raise ValueError("W must be fp32 [d_out][d_in] with unit column stride")
        if want_codes:
            if codes is None:
                codes = torch.empty(m, d, dtype=torch.uint8, device=W.device)
            if scales is None:
                scales = torch.empty(nb, dtype=torch.float32, device=W.device)
        if resid is None:
            _check(_lib.gift_encode(self._h, _ptr(W), W.stride(0), fmt, scaling, _ptr(amax_in), _ptr(amax_out),
                                    _ptr(codes) if want_codes else None, _ptr(scales) if want_codes else None,
                                    _ptr(whitened), _ptr(self.work), self.work_bytes, _stream(stream)), "gift_encode")
        else:
            if resid.dtype != torch.float32 or resid.shape != (m, d) or not resid.is_contiguous():
                raise ValueError("resid must be a contiguous fp32 [d_out][d_in] tensor")
            _check(_lib.gift_encode_ef(self._h, _ptr(W), W.stride(0), fmt, scaling, _ptr(amax_in), _ptr(amax_out),
                                       _ptr(codes) if want_codes else None, _ptr(scales) if want_codes else None,
                                       _ptr(whitened), _ptr(resid), _ptr(self.work), self.work_bytes,
                                       _stream(stream)), "gift_encode_ef")
        return codes, scales

    def decode_reduce(self, codes: torch.Tensor, scales: torch.Tensor, fmt=E4M3, scaling=SCALE_TENSOR, out=None,
                      R=None, stream=None):
        """codes [R][m][d] uint8, scales [R][nblk] fp32 (contiguous replicas)."""
        fmt = FORMATS.get(fmt, fmt)
        scaling = SCALINGS.get(scaling, scaling)
        m, d = self.m, self.d
        if codes.dim() == 2:
            codes = codes.unsqueeze(0)
            scales = scales.reshape(1, -1)
        R = codes.shape[0] if R is None else R
        if out is None:
            out = torch.empty(m, d, dtype=torch.float32, device=codes.device)
        cs = codes.stride(0) if R > 1 else m * d
        ss = scales.stride(0) if R > 1 else scales.shape[-1]
        _check(_lib.gift_decode_reduce(self._h, _ptr(codes), cs, _ptr(scales), ss, R, fmt, scaling, _ptr(out),
                                       out.stride(0), _ptr(self.work), self.work_bytes, _stream(stream)),
               "gift_decode_reduce")
        return out

    def encode_fp4(self, W: torch.Tensor, amax_in=None, codes=None, bscales=None, tscale=None, amax_out=None,
                   whitened=None, want_codes=True, resid=None, stream=None):
        """FP4 payload: codes [m][d/2] uint8 (two per byte, even column low),
        bscales [m][d/16] uint8 (E4M3), tscale [1] fp32."""
        m, d = self.m, self.d
        if W.dtype != torch.float32 or W.shape != (m, d) or W.stride(1) != 1:
            raise ValueError("W must be fp32 [d_out][d_in] with unit column stride")
        if resid is not None and (resid.dtype != torch.float32 or resid.shape != (m, d) or not resid.is_contiguous()):
            raise ValueError("resid must be a contiguous fp32 [d_out][d_in] tensor")
        if want_codes:
            if codes is None:
                codes = torch.empty(m, d // 2, dtype=torch.uint8, device=W.device)
            if bscales is None:
                bscales = torch.empty(m, d // 16, dtype=torch.uint8, device=W.device)
            if tscale is None:
                tscale = torch.empty(1, dtype=torch.float32, device=W.device)
        _check(_lib.gift_encode_fp4(self._h, _ptr(W), W.stride(0), _ptr(amax_in), _ptr(amax_out),
                                    _ptr(codes) if want_codes else None, _ptr(bscales) if want_codes else None,
                                    _ptr(tscale) if want_codes else None, _ptr(whitened), _ptr(resid),
                                    _ptr(self.work), self.work_bytes, _stream(stream)), "gift_encode_fp4")
        return codes, bscales, tscale

    def decode_reduce_fp4(self, codes: torch.Tensor, bscales: torch.Tensor, tscales: torch.Tensor, out=None,
                          stream=None):
        """codes [R][m][d/2], bscales [R][m][d/16] uint8, tscales [R] fp32."""
        m, d = self.m, self.d
        if codes.dim() == 2:
            codes, bscales = codes.unsqueeze(0), bscales.unsqueeze(0)
        R = codes.shape[0]
        tscales = tscales.reshape(-1)
        if tscales.numel() < R or tscales.dtype != torch.float32 or not tscales.is_contiguous():
            raise ValueError("tscales must be a contiguous fp32 tensor of R entries")
        if out is None:
            out = torch.empty(m, d, dtype=torch.float32, device=codes.device)
        cs = codes.stride(0) if R > 1 else m * d // 2
        bs = bscales.stride(0) if R > 1 else m * d // 16
        _check(_lib.gift_decode_reduce_fp4(self._h, _ptr(codes), cs, _ptr(bscales), bs, _ptr(tscales), R, _ptr(out),
                                           out.stride(0), _ptr(self.work), self.work_bytes, _stream(stream)),
               "gift_decode_reduce_fp4")
        return out


class Profiler:
    """FP8 boundary-hit profiler over a list of layers (gift_profiler_*)."""

    def __init__(self, n_layers: int, fmt=E4M3, scaling=SCALE_TENSOR, device="cuda", stream=None):
        self.n = n_layers
        self.counts = torch.zeros(n_layers, 2, dtype=torch.int64, device=device)
        self.work_bytes = int(_lib.gift_profiler_workspace_bytes(n_layers, scaling, 0))
        self.work = _alloc(self.work_bytes, device)
        h = _vp()
        _check(_lib.gift_profiler_create(n_layers, FORMATS.get(fmt, fmt), SCALINGS.get(scaling, scaling),
                                         _ptr(self.counts), _stream(stream), ctypes.byref(h)), "gift_profiler_create")
        self._h = h

    def step(self, grads, stream=None):
        ptrs = (_vp * self.n)(*[g.data_ptr() for g in grads])
        numel = (_i64 * self.n)(*[g.numel() for g in grads])
        for g in grads:
            if g.dtype != torch.float32 or not g.is_contiguous():
                raise ValueError("gradients must be contiguous fp32")
        _check(_lib.gift_profile_step(self._h, self.n, ptrs, numel, _ptr(self.work), self.work_bytes,
                                      _stream(stream)), "gift_profile_step")

    def select(self, max_select: int, stream=None):
        sc = (ctypes.c_double * self.n)()
        order = (_i32 * self.n)()
        sel = (_i32 * self.n)()
        nsel = _i32()
        _check(_lib.gift_select_layers(self._h, max_select, sc, order, sel, ctypes.byref(nsel), _stream(stream)),
               "gift_select_layers")
        return list(sc), list(order), list(sel[:nsel.value])

    def close(self):
        if getattr(self, "_h", None):
            _lib.gift_profiler_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def scale_sync_due(step: int, period: int) -> bool:
    """Whether `step` is a scale-sync step of a schedule syncing every
    `period` steps (gift_scale_sync_due)."""
    return bool(_lib.gift_scale_sync_due(step, period))


class Bucket:
    """Flat gradient bucket of Euclidean tensors (gift_bucket_*): the tensors
    of `sizes` elements lie one after another in one flat fp32 buffer."""

    def __init__(self, sizes, scaling=SCALE_TENSOR, device="cuda", stream=None):
        self.sizes = [int(n) for n in sizes]
        self.scaling = SCALINGS.get(scaling, scaling)
        n = len(self.sizes)
        tb = int(_lib.gift_bucket_table_bytes(n))
        self.table = _alloc(tb, device)
        arr = (_i64 * n)(*self.sizes)
        h = _vp()
        _check(_lib.gift_bucket_create(n, arr, self.scaling, _ptr(self.table), tb, _stream(stream), ctypes.byref(h)),
               "gift_bucket_create")
        self._h = h
        ne, ns, wb = _i64(), _i64(), _sz()
        _check(_lib.gift_bucket_sizes(h, ctypes.byref(ne), ctypes.byref(ns), ctypes.byref(wb)), "gift_bucket_sizes")
        self.numel, self.nscales, self.work_bytes = ne.value, ns.value, wb.value
        self.work = _alloc(max(self.work_bytes, 256), device)

    def _grad(self, g):
        if g.dtype != torch.float32 or not g.is_contiguous() or g.numel() < self.numel:
            raise ValueError("the bucket needs a contiguous fp32 buffer of all its elements")

    def amax(self, grad, amax_out=None, stream=None):
        self._grad(grad)
        if amax_out is None:
            amax_out = torch.empty(self.nscales, dtype=torch.float32, device=grad.device)
        _check(_lib.gift_bucket_amax(self._h, _ptr(grad), _ptr(amax_out), _stream(stream)), "gift_bucket_amax")
        return amax_out

    def encode(self, grad, fmt=E4M3, amax_in=None, amax_out=None, codes=None, scales=None, stream=None):
        self._grad(grad)
        if codes is None:
            codes = torch.empty(self.numel, dtype=torch.uint8, device=grad.device)
        if scales is None:
            scales = torch.empty(self.nscales, dtype=torch.float32, device=grad.device)
        _check(_lib.gift_bucket_encode(self._h, _ptr(grad), FORMATS.get(fmt, fmt), _ptr(amax_in), _ptr(amax_out),
                                       _ptr(codes), _ptr(scales), _ptr(self.work), self.work_bytes, _stream(stream)),
               "gift_bucket_encode")
        return codes, scales

    def encode_static(self, grad, fmt=E4M3, amax_in=None, amax_out=None, codes=None, scales=None, stream=None):
        """gift_bucket_encode_static: the encode without a workspace (the
        library's per-device scratch array holds the amax slots)."""
        self._grad(grad)
        if codes is None:
            codes = torch.empty(self.numel, dtype=torch.uint8, device=grad.device)
        if scales is None:
            scales = torch.empty(self.nscales, dtype=torch.float32, device=grad.device)
        _check(_lib.gift_bucket_encode_static(self._h, _ptr(grad), FORMATS.get(fmt, fmt), _ptr(amax_in),
                                              _ptr(amax_out), _ptr(codes), _ptr(scales), _stream(stream)),
               "gift_bucket_encode_static")
        return codes, scales

    def decode_reduce(self, codes, scales, fmt=E4M3, out=None, stream=None):
        """codes [R][numel] uint8, scales [R][nscales] fp32."""
        if codes.dim() == 1:
            codes, scales = codes.unsqueeze(0), scales.unsqueeze(0)
        R = codes.shape[0]
        if out is None:
            out = torch.empty(self.numel, dtype=torch.float32, device=codes.device)
        cs = codes.stride(0) if R > 1 else self.numel
        ss = scales.stride(0) if R > 1 else self.nscales
        _check(_lib.gift_bucket_decode_reduce(self._h, _ptr(codes), cs, _ptr(scales), ss, R, FORMATS.get(fmt, fmt),
                                              _ptr(out), _stream(stream)), "gift_bucket_decode_reduce")
        return out

    def flags(self, stream=None) -> int:
        f = ctypes.c_uint32()
        _check(_lib.gift_bucket_flags(self._h, _stream(stream), ctypes.byref(f)), "gift_bucket_flags")
        return f.value

    def close(self):
        if getattr(self, "_h", None):
            _lib.gift_bucket_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


class Group:
    """Grouped rank-k layers (gift_group_*): one launch encodes all of them,
    one launch decode-reduces all of them.  items: a list of dicts with the
    layer (a Layer), W, codes, scales (this worker's payload), rcodes
    [R][m][d], rscales [R][nblk] (the payloads to decode) and out."""

    def __init__(self, items, R, fmt=E4M3, scaling=SCALE_TENSOR, device="cuda", stream=None):
        n = len(items)
        arr = (GroupItem * n)()
        self._keep = items
        for k, it in enumerate(items):
            L = it["layer"]
            rc, rs = it["rcodes"], it["rscales"]
            arr[k] = GroupItem(L.handle, it["W"].data_ptr(), it["W"].stride(0), it["codes"].data_ptr(),
                               it["scales"].data_ptr(), rc.data_ptr(), rc.stride(0) if R > 1 else L.m * L.d,
                               rs.data_ptr(), rs.stride(0) if R > 1 else rs.shape[-1], it["out"].data_ptr(),
                               it["out"].stride(0))
        tb = int(_lib.gift_group_table_bytes(n))
        self.table = _alloc(tb, device)
        h = _vp()
        _check(_lib.gift_group_create(n, arr, R, FORMATS.get(fmt, fmt), SCALINGS.get(scaling, scaling),
                                      _ptr(self.table), tb, _stream(stream), ctypes.byref(h)), "gift_group_create")
        self._h = h

    def encode(self, stream=None):
        _check(_lib.gift_group_encode(self._h, _stream(stream)), "gift_group_encode")

    def decode_reduce(self, stream=None):
        _check(_lib.gift_group_decode_reduce(self._h, _stream(stream)), "gift_group_decode_reduce")

    def close(self):
        if getattr(self, "_h", None):
            _lib.gift_group_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
