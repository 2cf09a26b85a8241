"""ctypes declarations of liblores.so (include/lores.h).

The library is loaded on first use.  If it has not been built, every entry
point raises LoresLibraryMissing: there is no fallback implementation.
"""
import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "liblores.so")

SPEC_VERSION = 8                     # LORES_SPEC_VERSION of include/lores.h
LORES_FP32, LORES_BF16, LORES_INT8, LORES_INT4, LORES_INT6, LORES_FP8 = 0, 1, 2, 3, 4, 5
NUM_PREC = 6
LORES_ROUND_STOCHASTIC, LORES_ROUND_NEAREST = 0, 1
LORES_SCALE_VALUE, LORES_SCALE_KEY = 0, 1
LORES_MAX_WINDOW = 16
LORES_OK, LORES_EINVAL, LORES_EUNSUPPORTED, LORES_ESIZE, LORES_EHIP, LORES_ENOMEM = 0, -1, -2, -3, -4, -5
STATUS_NAMES = {0: "LORES_OK", -1: "LORES_EINVAL", -2: "LORES_EUNSUPPORTED", -3: "LORES_ESIZE",
                -4: "LORES_EHIP", -5: "LORES_ENOMEM"}

# every symbol include/lores.h declares
EXPORTS = ("lores_state_alloc", "lores_state_alloc_axis", "lores_state_alloc_window",
           "lores_state_free", "lores_state_layout", "lores_state_head_map",
           "lores_decay_stat", "lores_assign_precision", "lores_decode_step",
           "lores_step_launches", "lores_state_set_rounding", "lores_quant_state",
           "lores_dequant_state",
           "lores_last_error", "lores_spec_version")


class LoresLibraryMissing(RuntimeError):
    pass


class LoresLayout(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("H", ctypes.c_int32), ("d_k", ctypes.c_int32),
                ("d_v", ctypes.c_int32), ("d_v_pad", ctypes.c_int32),
                ("n_class", ctypes.c_int32 * NUM_PREC), ("codes_offset", ctypes.c_int64 * NUM_PREC),
                ("scales_offset", ctypes.c_int64 * NUM_PREC),
                ("unit_code_bytes", ctypes.c_int64 * NUM_PREC),
                ("total_bytes", ctypes.c_uint64),
                ("scale_axis", ctypes.c_int32), ("unit_scales", ctypes.c_int32),
                ("window", ctypes.c_int32), ("window_fill", ctypes.c_int32),
                ("window_offset", ctypes.c_int64 * NUM_PREC),
                ("unit_window_bytes", ctypes.c_int64 * NUM_PREC)]


_lib = None


def lib():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise LoresLibraryMissing(
            f"{LIB_PATH} is not built; run `python -m quantized_linear_recurrence_amd.build` "
            "(there is no non-HIP fallback)")
    L = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, u64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_uint64
    L.lores_state_alloc.argtypes = [i32, i32, i32, i32, vp, vp, ctypes.POINTER(ctypes.c_size_t),
                                    vp, ctypes.POINTER(vp)]
    L.lores_state_alloc.restype = ctypes.c_int
    L.lores_state_alloc_axis.argtypes = [i32, i32, i32, i32, vp, i32, vp,
                                         ctypes.POINTER(ctypes.c_size_t), vp, ctypes.POINTER(vp)]
    L.lores_state_alloc_axis.restype = ctypes.c_int
    L.lores_state_alloc_window.argtypes = [i32, i32, i32, i32, vp, i32, i32, vp,
                                           ctypes.POINTER(ctypes.c_size_t), vp, ctypes.POINTER(vp)]
    L.lores_state_alloc_window.restype = ctypes.c_int
    L.lores_state_free.argtypes = [vp]
    L.lores_state_free.restype = None
    L.lores_state_layout.argtypes = [vp, ctypes.POINTER(LoresLayout)]
    L.lores_state_layout.restype = ctypes.c_int
    L.lores_state_head_map.argtypes = [vp, vp, vp]
    L.lores_state_head_map.restype = ctypes.c_int
    L.lores_decay_stat.argtypes = [vp, i64, i32, i32, vp]
    L.lores_decay_stat.restype = ctypes.c_int
    L.lores_assign_precision.argtypes = [vp, i32, vp, vp, i32, vp]
    L.lores_assign_precision.restype = ctypes.c_int
    L.lores_decode_step.argtypes = [vp, vp, vp, vp, i32, vp, i32, vp, i32, u64, u64, i64, i64,
                                    vp, vp]
    L.lores_decode_step.restype = ctypes.c_int
    L.lores_state_set_rounding.argtypes = [vp, i32]
    L.lores_state_set_rounding.restype = ctypes.c_int
    L.lores_step_launches.argtypes = [vp, ctypes.POINTER(i32)]
    L.lores_step_launches.restype = ctypes.c_int
    L.lores_quant_state.argtypes = [vp, vp, u64, i64, i64, vp]
    L.lores_quant_state.restype = ctypes.c_int
    L.lores_dequant_state.argtypes = [vp, vp, vp]
    L.lores_dequant_state.restype = ctypes.c_int
    L.lores_last_error.argtypes = []
    L.lores_last_error.restype = ctypes.c_char_p
    L.lores_spec_version.argtypes = []
    L.lores_spec_version.restype = ctypes.c_int
    _lib = L
    return L
