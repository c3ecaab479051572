"""The C-ABI library loads and exports every entry point include/gift.h
declares; host-side argument checks that need no GPU."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    text = open(os.path.join(ROOT, "include", "gift.h"), encoding="utf-8").read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gift_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = _declared()
    for required in ("gift_accumulate_stats", "gift_refresh_factors", "gift_encode", "gift_decode_reduce",
                     "gift_select_layers"):
        assert required in names


def test_library_exports_every_declared_symbol():
    import fac_whitening_amd as fw
    lib = ctypes.CDLL(fw.LIB_PATH)
    for name in _declared():
        assert hasattr(lib, name), name
    assert sorted(fw.EXPORTS) == _declared()


def test_host_side_checks_without_gpu():
    import fac_whitening_amd as fw
    lib = fw._lib
    sb, wb = ctypes.c_size_t(), ctypes.c_size_t()
    good = fw.LayerDesc(1536, 6144, fw.LOWRANK, 32, 16, 4, 0.0, 1e-3)
    assert lib.gift_layer_state_bytes(ctypes.byref(good), ctypes.byref(sb), ctypes.byref(wb)) == 0
    assert sb.value % 256 == 0 and wb.value % 256 == 0
    assert sb.value >= 2 * 6144 * 6144 * 4 + 6144 * 32 * 4
    for bad in [fw.LayerDesc(1536, 6145, fw.LOWRANK, 32, 16, 4, 0.0, 1e-3),     # d_in % 8
                fw.LayerDesc(0, 6144, fw.LOWRANK, 32, 16, 4, 0.0, 1e-3),        # d_out
                fw.LayerDesc(1536, 6144, 9, 32, 16, 4, 0.0, 1e-3),              # transform
                fw.LayerDesc(1536, 6144, fw.LOWRANK, 33, 16, 4, 0.0, 1e-3),     # rank > 32
                fw.LayerDesc(1536, 6144, fw.LOWRANK, 32, 40, 4, 0.0, 1e-3),     # l > 64
                fw.LayerDesc(1536, 6144, fw.LOWRANK, 32, 16, 4, 1.0, 1e-3),     # beta = 1
                fw.LayerDesc(1536, 6144, fw.LOWRANK, 32, 16, 4, 0.0, -1.0)]:    # damping < 0
        assert lib.gift_layer_state_bytes(ctypes.byref(bad), ctypes.byref(sb), ctypes.byref(wb)) == 1
    # transient statistics: the window sums leave the state (d^2 fp32, and
    # m^2 more for the two-sided variant) and the workspace holds one of them
    for tr, n_s in ((fw.LOWRANK, 6144 * 6144 * 4), (fw.CHOL_TWOSIDED, (6144 * 6144 + 1536 * 1536) * 4)):
        base = fw.LayerDesc(1536, 6144, tr, 32, 16, 4, 0.0, 1e-3)
        tra = fw.LayerDesc(1536, 6144, tr, 32, 16, 4, 0.0, 1e-3, fw.LAYER_TRANSIENT_STATS)
        sb2, wb2 = ctypes.c_size_t(), ctypes.c_size_t()
        assert lib.gift_layer_state_bytes(ctypes.byref(base), ctypes.byref(sb), ctypes.byref(wb)) == 0
        assert lib.gift_layer_state_bytes(ctypes.byref(tra), ctypes.byref(sb2), ctypes.byref(wb2)) == 0
        assert sb.value - sb2.value == n_s
        assert wb2.value >= max(wb.value, 6144 * 6144 * 4)
    unknown = fw.LayerDesc(1536, 6144, fw.LOWRANK, 32, 16, 4, 0.0, 1e-3, 2)   # unknown flag bit
    assert lib.gift_layer_state_bytes(ctypes.byref(unknown), ctypes.byref(sb), ctypes.byref(wb)) == 1
    # payload = 1 byte per element + one fp32 scale per tile
    assert fw.payload_bytes(1536, 6144, fw.SCALE_TENSOR) == 1536 * 6144 + 4
    assert fw.payload_bytes(1536, 6144, fw.SCALE_BLOCK128) == 1536 * 6144 + 4 * 12 * 48
    assert fw.payload_bytes(100, 300, fw.SCALE_BLOCK128) == 100 * 300 + 4 * 1 * 3
    assert lib.gift_status_string(3) == b"not ready (no committed statistics or no factor yet)"
    # calls with a NULL handle fail before touching the device
    assert lib.gift_encode(None, None, 0, 0, 0, None, None, None, None, None, None, 0, None) == 1
    assert lib.gift_profiler_create(0, 0, 0, None, None, None) == 1
    # FP4 payload: half a byte per code, one E4M3 byte per 16 elements, the tensor scale
    assert fw.payload_bytes(4096, 16384, fw.SCALE_BLOCK16) == 4096 * 16384 // 2 + 4096 * 1024 + 4
    assert lib.gift_encode_fp4(None, None, 0, None, None, None, None, None, None, None, None, 0, None) == 1
    # buckets: table size, argument checks before any device work
    assert lib.gift_bucket_table_bytes(0) == 0 and lib.gift_bucket_table_bytes(168) % 256 == 0
    h = ctypes.c_void_p()
    sizes = (ctypes.c_int64 * 2)(1024, 6)                          # 6 is not a multiple of 4
    assert lib.gift_bucket_create(2, sizes, fw.SCALE_TENSOR, None, 0, None, ctypes.byref(h)) == 1
    assert lib.gift_bucket_create(2, sizes, fw.SCALE_BLOCK128, None, 0, None, ctypes.byref(h)) == 1


def test_scale_sync_schedule():
    """Algorithm 1, its scale-sync step: local scales by default, a shared scale on
    every period-th step from step 0; period <= 0 never syncs."""
    import fac_whitening_amd as fw
    assert [fw.scale_sync_due(t, 4) for t in range(9)] == [True, False, False, False, True, False, False, False, True]
    assert not any(fw.scale_sync_due(t, 0) for t in range(5))
    assert not any(fw.scale_sync_due(t, -3) for t in range(5))
    assert all(fw.scale_sync_due(t, 1) for t in range(5))


def test_product_path_has_no_oracle_or_cpu_fallback():
    """The package never imports the oracle and has no CPU code path."""
    pkg = os.path.join(ROOT, "fac_whitening_amd")
    for fn in os.listdir(pkg):
        if fn.endswith(".py"):
            src = open(os.path.join(pkg, fn), encoding="utf-8").read()
            assert "oracle" not in src.replace("never imports the oracle", ""), fn
