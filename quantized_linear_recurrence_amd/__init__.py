"""Python binding of liblores (the LoReS quantized recurrent-state decode step on
MI355X / gfx950).

The functions carry the C ABI's names (include/lores.h) and only marshal
arguments: torch tensors become device pointers, the current torch stream
becomes the hipStream_t, shapes and dtypes are checked so that no raw pointer
is handed over with too few elements.  All computation happens in the HIP
kernels of liblores.so; if the library is missing, calls raise.

PyTorch serves only as the device allocator and stream provider.
"""
import ctypes

import numpy as np

from . import _lib
from ._lib import (LORES_BF16, LORES_FP8, LORES_FP32, LORES_INT4, LORES_INT6, LORES_INT8,
                   LORES_MAX_WINDOW, LORES_ROUND_NEAREST, LORES_ROUND_STOCHASTIC, LORES_SCALE_KEY,
                   LORES_SCALE_VALUE, LoresLayout, LoresLibraryMissing)

__all__ = ["LORES_FP32", "LORES_BF16", "LORES_INT8", "LORES_INT4", "LORES_INT6", "LORES_FP8",
           "LORES_ROUND_STOCHASTIC", "LORES_ROUND_NEAREST", "LORES_SCALE_VALUE", "LORES_SCALE_KEY",
           "LoresError", "lores_state_set_rounding",
           "LORES_MAX_WINDOW", "LoresLibraryMissing", "LoresState", "lores_state_alloc",
           "lores_state_alloc_axis", "lores_state_alloc_window",
           "lores_state_layout",
           "lores_state_head_map", "lores_decay_stat", "lores_assign_precision",
           "lores_decode_step", "lores_step_launches", "lores_quant_state", "lores_dequant_state",
           "lores_last_error", "lores_spec_version"]


class LoresError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(f"{_lib.STATUS_NAMES.get(status, status)}: {msg}")
        self.status = status


def _check(rc):
    if rc != 0:
        raise LoresError(rc, _lib.lib().lores_last_error().decode())


def _stream_ptr(stream, device):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return ctypes.c_void_p(stream.cuda_stream)


def _dev_ptr(t, name, dtype, numel, device):
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, the state is on {device}")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.numel() != numel:
        raise ValueError(f"{name} must have {numel} elements, got {t.numel()}")
    return ctypes.c_void_p(t.data_ptr())


def _host_array(x, dtype):
    a = np.ascontiguousarray(np.asarray(x, dtype=dtype))
    return a, a.ctypes.data_as(ctypes.c_void_p)


def lores_spec_version():
    return _lib.lib().lores_spec_version()


def lores_last_error():
    return _lib.lib().lores_last_error().decode()


class LoresState:
    """A quantized recurrent state: the library handle plus its device buffer.

    The buffer is a torch uint8 tensor (caller-owned device memory); the handle
    is freed when this object is garbage-collected.
    """

    def __init__(self, handle, buf, B, H, d_k, d_v, head_prec, scale_axis=LORES_SCALE_VALUE,
                 window=1):
        self._h = handle
        self.buf = buf
        self.device = buf.device
        self.B, self.H, self.d_k, self.d_v = B, H, d_k, d_v
        self.head_prec = list(head_prec)
        self.rounding = LORES_ROUND_STOCHASTIC
        self.scale_axis = scale_axis
        self.window = window

    @property
    def handle(self):
        return self._h

    def __del__(self):
        h = getattr(self, "_h", None)
        if h:
            try:
                _lib.lib().lores_state_free(h)
            except Exception:
                pass
            self._h = None


def lores_state_alloc(B, H, d_k, d_v, head_prec, device=None, stream=None, buf=None,
                      scale_axis=LORES_SCALE_VALUE, window=1):
    """Plan the packed layout; size query if device and buf are both None.

    Returns the byte size (size query) or a LoresState whose buffer (a new
    torch uint8 tensor on `device`, or the given `buf`) is cleared to S_0 = 0
    on `stream`.  scale_axis: LORES_SCALE_VALUE (one scale per value row,
    lores_state_alloc) or LORES_SCALE_KEY (one per key column,
    lores_state_alloc_axis).  window > 1: requantize the scaled heads once per
    window of that many steps (lores_state_alloc_window).
    """
    L = _lib.lib()
    hp, hp_ptr = _host_array(head_prec, np.uint8)
    if hp.size != H:
        raise ValueError(f"head_prec must have H = {H} entries")
    window = int(window)

    def alloc(ptr, size, stream_ptr, out):
        if window != 1:
            return L.lores_state_alloc_window(B, H, d_k, d_v, hp_ptr, int(scale_axis), window, ptr,
                                              size, stream_ptr, out)
        return L.lores_state_alloc_axis(B, H, d_k, d_v, hp_ptr, int(scale_axis), ptr, size,
                                        stream_ptr, out)
    nbytes = ctypes.c_size_t(0)
    _check(alloc(None, ctypes.byref(nbytes), None, None))
    if device is None and buf is None:
        return nbytes.value
    import torch
    if buf is None:
        buf = torch.empty(nbytes.value, dtype=torch.uint8, device=device)
    device = buf.device
    size = ctypes.c_size_t(buf.numel() * buf.element_size())
    out = ctypes.c_void_p()
    _check(alloc(ctypes.c_void_p(buf.data_ptr()), ctypes.byref(size), _stream_ptr(stream, device),
                 ctypes.byref(out)))
    return LoresState(out.value, buf, B, H, d_k, d_v, hp.tolist(), int(scale_axis), window)


lores_state_alloc_axis = lores_state_alloc
lores_state_alloc_window = lores_state_alloc


def lores_state_layout(state):
    lay = LoresLayout()
    _check(_lib.lib().lores_state_layout(ctypes.c_void_p(state.handle), ctypes.byref(lay)))
    return {"B": lay.B, "H": lay.H, "d_k": lay.d_k, "d_v": lay.d_v, "d_v_pad": lay.d_v_pad,
            "n_class": list(lay.n_class), "codes_offset": list(lay.codes_offset),
            "scales_offset": list(lay.scales_offset),
            "unit_code_bytes": list(lay.unit_code_bytes), "total_bytes": lay.total_bytes,
            "scale_axis": lay.scale_axis, "unit_scales": lay.unit_scales,
            "window": lay.window, "window_fill": lay.window_fill,
            "window_offset": list(lay.window_offset),
            "unit_window_bytes": list(lay.unit_window_bytes)}


def lores_state_head_map(state):
    prec = np.zeros(state.H, np.uint8)
    slot = np.zeros(state.H, np.int32)
    _check(_lib.lib().lores_state_head_map(ctypes.c_void_p(state.handle),
                                           prec.ctypes.data_as(ctypes.c_void_p),
                                           slot.ctypes.data_as(ctypes.c_void_p)))
    return prec, slot


def lores_state_set_rounding(state, mode):
    """LORES_ROUND_STOCHASTIC (default) or LORES_ROUND_NEAREST for later steps."""
    _check(_lib.lib().lores_state_set_rounding(ctypes.c_void_p(state.handle), int(mode)))
    state.rounding = int(mode)


def lores_step_launches(state):
    """Kernel launches one lores_decode_step on `state` enqueues."""
    n = ctypes.c_int32(0)
    _check(_lib.lib().lores_step_launches(ctypes.c_void_p(state.handle), ctypes.byref(n)))
    return n.value


def lores_decay_stat(alpha):
    """Mean log(alpha) per head; alpha host array [n, H] or [n, H, width] (fp32)."""
    a = np.ascontiguousarray(np.asarray(alpha, dtype=np.float32))
    if a.ndim == 2:
        a = a[:, :, None]
    if a.ndim != 3:
        raise ValueError("alpha must be [n, H] or [n, H, width]")
    n, H, W = a.shape
    stat = np.zeros(H, np.float64)
    _check(_lib.lib().lores_decay_stat(a.ctypes.data_as(ctypes.c_void_p), n, H, W,
                                       stat.ctypes.data_as(ctypes.c_void_p)))
    return stat


def lores_assign_precision(stat, tier_frac, tier_prec):
    s, sp = _host_array(stat, np.float64)
    f, fp = _host_array(tier_frac, np.float64)
    p, pp = _host_array(tier_prec, np.uint8)
    if f.size != p.size:
        raise ValueError("tier_frac and tier_prec must have the same length")
    out = np.zeros(s.size, np.uint8)
    _check(_lib.lib().lores_assign_precision(sp, s.size, fp, pp, f.size,
                                             out.ctypes.data_as(ctypes.c_void_p)))
    return out.tolist()


def lores_decode_step(state, q, k, v, alpha, beta, delta, seed, t, o=None, seq_base=0,
                      head_base=0, stream=None):
    """One decode step t for all B x H units; returns o [B, H, d_v] fp32."""
    import torch
    B, H, dk, dv, dev = state.B, state.H, state.d_k, state.d_v, state.device
    in_bf16 = q.dtype == torch.bfloat16
    in_dt = torch.bfloat16 if in_bf16 else torch.float32
    per_channel = alpha.numel() == B * H * dk and dk != 1
    if o is None:
        o = torch.empty((B, H, dv), dtype=torch.float32, device=dev)
    args = (_dev_ptr(q, "q", in_dt, B * H * dk, dev), _dev_ptr(k, "k", in_dt, B * H * dk, dev),
            _dev_ptr(v, "v", in_dt, B * H * dv, dev))
    a_ptr = _dev_ptr(alpha, "alpha", torch.float32, B * H * dk if per_channel else B * H, dev)
    b_ptr = _dev_ptr(beta, "beta", torch.float32, B * H, dev)
    o_ptr = _dev_ptr(o, "o", torch.float32, B * H * dv, dev)
    _check(_lib.lib().lores_decode_step(ctypes.c_void_p(state.handle), *args, int(in_bf16), a_ptr,
                                        int(per_channel), b_ptr, int(delta), int(seed), int(t),
                                        int(seq_base), int(head_base), o_ptr,
                                        _stream_ptr(stream, dev)))
    return o


def lores_quant_state(state, X, seed, seq_base=0, head_base=0, stream=None):
    """fp32 [B, H, d_v, d_k] -> the packed state (requantized, draws keyed at t = 0)."""
    import torch
    shape = (state.B, state.H, state.d_v, state.d_k)
    ptr = _dev_ptr(X, "X", torch.float32, int(np.prod(shape)), state.device)
    _check(_lib.lib().lores_quant_state(ctypes.c_void_p(state.handle), ptr, int(seed),
                                        int(seq_base), int(head_base),
                                        _stream_ptr(stream, state.device)))


def lores_dequant_state(state, out=None, stream=None):
    """Packed state -> fp32 [B, H, d_v, d_k]."""
    import torch
    shape = (state.B, state.H, state.d_v, state.d_k)
    if out is None:
        out = torch.empty(shape, dtype=torch.float32, device=state.device)
    ptr = _dev_ptr(out, "out", torch.float32, int(np.prod(shape)), state.device)
    _check(_lib.lib().lores_dequant_state(ctypes.c_void_p(state.handle), ptr,
                                          _stream_ptr(stream, state.device)))
    return out
