"""Host-side checks of liblores.so that need no GPU: the library loads, exports
every entry point include/lores.h declares, plans the documented layout, and
its host algorithms agree with the oracle.  Invalid arguments return error
codes without touching the device."""
import ctypes
import math
import os
import re
import subprocess

import numpy as np
import pytest

import quantized_linear_recurrence_amd as lores
from oracle import assign as oassign

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lores.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(lores_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol(lores_lib):
    declared = _declared()
    assert len(declared) >= 10
    out = subprocess.run(["nm", "-D", "--defined-only", lores.__path__[0] + "/liblores.so"],
                         capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r"\sT\s+(lores_\w+)", out))
    missing = [s for s in declared if s not in exported]
    assert not missing, missing
    for s in declared:
        assert hasattr(lores_lib, s)
    assert set(declared) == set(lores._lib.EXPORTS)


def test_spec_version(lores_lib):
    hdr = open(os.path.join(ROOT, "include", "lores.h")).read()
    v = int(re.search(r"#define LORES_SPEC_VERSION (\d+)", hdr).group(1))
    assert lores.lores_spec_version() == v == lores._lib.SPEC_VERSION == 8


def _layout_bytes(B, H, dk, dv, head_prec, key=False, window=1):
    """Segment sizes as include/lores.h documents them."""
    bits = {0: 32, 1: 16, 2: 8, 3: 4, 4: 6, 5: 8}
    dvp = (dv + 63) // 64 * 64
    off = 0
    for c in range(6):
        hc = sum(1 for p in head_prec if p == c)
        if not hc:
            continue
        off = (off + 255) // 256 * 256
        # whole 16-byte chunks per row; above d_k = 128 per half row
        chunks = 2 * -(-(dk // 2 * bits[c]) // 128) if dk > 128 else -(-(dk * bits[c]) // 128)
        off += B * hc * chunks * 16 * dvp
        if c in (2, 3, 4, 5):                      # one fp32 scale per value row / key column
            off = (off + 255) // 256 * 256
            off += B * hc * (dk if key else dvp) * 4
            if window > 1:                         # W - 1 slots of g, k, alpha per unit
                off = (off + 255) // 256 * 256
                off += B * hc * (((window - 1) * (dvp + 2 * dk) * 4 + 15) // 16 * 16)
    return (off + 255) // 256 * 256


@pytest.mark.parametrize("B,H,dk,dv,prec", [
    (1, 2, 64, 64, [2, 2]), (64, 32, 128, 128, [2] * 32), (256, 128, 128, 64, [2] * 128),
    (128, 32, 128, 128, [1] * 8 + [2] * 24), (2048, 32, 128, 128, [2] * 16 + [3] * 16),
    (3, 4, 96, 100, [0, 1, 2, 3]), (1, 1, 32, 1, [3]), (2048, 32, 128, 128, [4] * 16 + [3] * 16),
    (3, 5, 96, 65, [4, 0, 1, 2, 3]), (2, 1, 32, 1, [4]), (4, 6, 64, 100, [5, 4, 3, 2, 1, 0]),
    (3, 6, 256, 100, [5, 4, 3, 2, 1, 0]), (2, 2, 256, 1, [2, 3]),
    (3, 6, 160, 100, [5, 4, 3, 2, 1, 0]), (3, 6, 192, 65, [5, 4, 3, 2, 1, 0]),
    (3, 6, 224, 33, [5, 4, 3, 2, 1, 0])])
def test_size_query_matches_documented_layout(lores_lib, B, H, dk, dv, prec):
    assert lores.lores_state_alloc(B, H, dk, dv, prec) == _layout_bytes(B, H, dk, dv, prec)


def test_assign_precision_matches_oracle(lores_lib):
    g = np.random.default_rng(0)
    for trial in range(200):
        H = int(g.integers(1, 70))
        stat = -g.uniform(0, 1, H)
        if trial % 3 == 0:
            stat = np.round(stat, 1)                  # many ties
        nt = int(g.integers(1, 4))
        frac = g.uniform(0, 1, nt)
        prec = g.integers(0, 4, nt)
        assert lores.lores_assign_precision(stat, frac, prec) == \
            oassign.assign_precision(stat, frac, prec)


def test_decay_stat_matches_oracle(lores_lib):
    g = np.random.default_rng(1)
    a = np.exp(-np.log1p(np.exp(g.normal(-3, 1, (50, 7))))).astype(np.float32)
    np.testing.assert_allclose(lores.lores_decay_stat(a), oassign.decay_stat(a), rtol=1e-12)
    a3 = g.uniform(0.1, 1, (20, 5, 16)).astype(np.float32)
    np.testing.assert_allclose(lores.lores_decay_stat(a3), oassign.decay_stat(a3), rtol=1e-12)


def _rc(fn, *args):
    return fn(*args)


def test_invalid_arguments_return_codes_without_gpu(lores_lib):
    L = lores_lib
    hp = (ctypes.c_uint8 * 4)(2, 2, 2, 2)
    nb = ctypes.c_size_t(0)
    bad_dims = [(0, 4, 64, 64), (1, 0, 64, 64), (1, 4, 48, 64), (1, 4, 64, 0), (1, 4, 64, 257),
                (1, 513, 64, 64)]
    for B, H, dk, dv in bad_dims:
        assert L.lores_state_alloc(B, H, dk, dv, hp, None, ctypes.byref(nb), None, None) == -1
        assert lores.lores_last_error()
    # d_k above 128 (split rows) takes either scale axis, with or without windows
    for dk in (160, 192, 224):
        assert L.lores_state_alloc(1, 4, dk, 64, hp, None, ctypes.byref(nb), None, None) == 0
    assert L.lores_state_alloc(1, 4, 288, 64, hp, None, ctypes.byref(nb), None, None) == -1
    assert L.lores_state_alloc(1, 4, 256, 64, hp, None, ctypes.byref(nb), None, None) == 0
    assert L.lores_state_alloc_axis(1, 4, 256, 64, hp, 1, None, ctypes.byref(nb), None,
                                    None) == 0
    assert L.lores_state_alloc_window(1, 4, 256, 64, hp, 0, 4, None, ctypes.byref(nb), None,
                                      None) == 0
    assert L.lores_state_alloc_window(1, 4, 256, 64, hp, 1, 4, None, ctypes.byref(nb), None,
                                      None) == 0
    assert L.lores_state_alloc_window(1, 4, 256, 64, hp, 0, 1, None, ctypes.byref(nb), None,
                                      None) == 0
    bad = (ctypes.c_uint8 * 4)(2, 2, 9, 2)
    assert L.lores_state_alloc(1, 4, 64, 64, bad, None, ctypes.byref(nb), None, None) == -1
    assert L.lores_state_alloc(1, 4, 64, 64, None, None, ctypes.byref(nb), None, None) == -1
    # misaligned device buffer is rejected before any device work
    out = ctypes.c_void_p()
    nb.value = 1 << 20
    assert L.lores_state_alloc(1, 4, 64, 64, hp, ctypes.c_void_p(0x1001), ctypes.byref(nb), None,
                               ctypes.byref(out)) == -1
    # too small a buffer
    nb.value = 16
    assert L.lores_state_alloc(1, 4, 64, 64, hp, ctypes.c_void_p(0x10000), ctypes.byref(nb), None,
                               ctypes.byref(out)) == -3
    # decode step and dequant on a NULL handle
    p = ctypes.c_void_p(0x10000)
    assert L.lores_decode_step(None, p, p, p, 0, p, 0, p, 1, 0, 1, 0, 0, p, None) == -1
    assert L.lores_dequant_state(None, p, None) == -1
    # host algorithms
    stat = (ctypes.c_double * 2)(0.0, float("nan"))
    fr = (ctypes.c_double * 1)(1.0)
    tp = (ctypes.c_uint8 * 1)(2)
    o = (ctypes.c_uint8 * 2)()
    assert L.lores_assign_precision(stat, 2, fr, tp, 1, o) == -1
    tp_bad = (ctypes.c_uint8 * 1)(7)
    stat_ok = (ctypes.c_double * 2)(0.0, -1.0)
    assert L.lores_assign_precision(stat_ok, 2, fr, tp_bad, 1, o) == -1
    assert L.lores_assign_precision(stat_ok, 2, fr, tp, 0, o) == -1
    neg = (ctypes.c_float * 2)(0.5, -0.5)
    st = (ctypes.c_double * 2)()
    assert L.lores_decay_stat(neg, 1, 2, 1, st) == -1


def test_key_axis_layout_and_limits(lores_lib):
    """Key-column scales: d_k scales per unit of a scaled class at every
    built d_k and d_v, an unknown axis EINVAL (size queries only: no device
    work)."""
    L = lores._lib.lib()
    hp = (ctypes.c_uint8 * 3)(2, 3, 1)
    n = ctypes.c_size_t(0)
    assert L.lores_state_alloc_axis(4, 3, 128, 100, hp, 1, None, ctypes.byref(n), None, None) == 0
    key_bytes = n.value
    assert L.lores_state_alloc_axis(4, 3, 128, 100, hp, 0, None, ctypes.byref(n), None, None) == 0
    val_bytes = n.value
    want = _layout_bytes(4, 3, 128, 100, [2, 3, 1], key=True)
    assert key_bytes == want, (key_bytes, want)
    assert val_bytes == _layout_bytes(4, 3, 128, 100, [2, 3, 1])
    for dk, dv in ((96, 64), (32, 64), (96, 200), (32, 1)):
        assert L.lores_state_alloc_axis(2, 3, dk, dv, hp, 1, None, ctypes.byref(n), None,
                                        None) == 0, (dk, dv)
        assert n.value == _layout_bytes(2, 3, dk, dv, [2, 3, 1], key=True), (dk, dv)
    for dv in (1, 64, 65, 128, 150, 192, 193, 256):
        assert L.lores_state_alloc_axis(2, 3, 64, dv, hp, 1, None, ctypes.byref(n), None,
                                        None) == 0, dv
    assert L.lores_state_alloc_axis(2, 3, 64, 64, hp, 2, None, ctypes.byref(n), None,
                                    None) == lores._lib.LORES_EINVAL
    assert "scale_axis" in lores.lores_last_error()


def test_window_layout_and_limits(lores_lib):
    """Windowed states: the window segment per scaled class, W in [1, 16],
    with value-row or key-column scales at every built d_k (size queries
    only)."""
    L = lores._lib.lib()
    hp = (ctypes.c_uint8 * 4)(2, 3, 1, 5)
    n = ctypes.c_size_t(0)
    for W in (1, 2, 8, 16):
        assert L.lores_state_alloc_window(5, 4, 128, 100, hp, 0, W, None, ctypes.byref(n), None,
                                          None) == 0
        assert n.value == _layout_bytes(5, 4, 128, 100, [2, 3, 1, 5], window=W), W
    for W in (0, 17, -1):
        assert L.lores_state_alloc_window(5, 4, 128, 100, hp, 0, W, None, ctypes.byref(n), None,
                                          None) == lores._lib.LORES_EINVAL
    for dk in (32, 96):
        assert L.lores_state_alloc_window(5, 4, dk, 100, hp, 0, 4, None, ctypes.byref(n), None,
                                          None) == 0
        assert n.value == _layout_bytes(5, 4, dk, 100, [2, 3, 1, 5], window=4)
    assert L.lores_state_alloc_window(5, 4, 96, 100, hp, 1, 4, None, ctypes.byref(n), None,
                                      None) == 0
    assert n.value == _layout_bytes(5, 4, 96, 100, [2, 3, 1, 5], key=True, window=4)
    assert L.lores_state_alloc_window(5, 4, 96, 100, hp, 0, 1, None, ctypes.byref(n), None,
                                      None) == 0
    # key-column windows: d_k scales per unit plus the window block
    assert L.lores_state_alloc_window(5, 4, 128, 100, hp, 1, 4, None, ctypes.byref(n), None,
                                      None) == 0
    assert n.value == _layout_bytes(5, 4, 128, 100, [2, 3, 1, 5], key=True, window=4)
    assert L.lores_state_alloc_window(5, 4, 128, 150, hp, 1, 4, None, ctypes.byref(n), None,
                                      None) == 0
    assert n.value == _layout_bytes(5, 4, 128, 150, [2, 3, 1, 5], key=True, window=4)


def test_error_message_is_thread_local_and_cleared(lores_lib):
    lores.lores_assign_precision([0.0], [1.0], [2])
    assert lores.lores_last_error() == ""
    with pytest.raises(lores.LoresError):
        lores.lores_assign_precision([0.0], [1.0], [9])
    assert "precision" in lores.lores_last_error()
