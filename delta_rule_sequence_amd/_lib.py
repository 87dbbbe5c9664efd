"""ctypes view of libefla.so (the C ABI declared in include/efla.h).

Loading fails loudly when the library has not been built: there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
# Debug builds of the same sources (python -m delta_rule_sequence_amd.build --sanitize or
# --lds-poison) are loaded instead when EFLA_LIBRARY_VARIANT names them: "hostsan" (host code
# under AddressSanitizer/UndefinedBehaviorSanitizer, for the host-side checks of the C ABI) or
# "ldspoison" (kernels that fill their LDS with NaN before they start).
_VARIANTS = {"": "libefla.so", "hostsan": "libefla_hostsan.so", "ldspoison": "libefla_ldspoison.so"}
LIB_PATH = os.path.join(_PKG, _VARIANTS[os.environ.get("EFLA_LIBRARY_VARIANT", "")])

EFLA_F32 = 0
EFLA_BF16 = 1
EFLA_EXACT = 0
EFLA_EULER = 1
MODES = {"exact": EFLA_EXACT, "euler": EFLA_EULER}

STATUS = {0: "EFLA_OK", 1: "EFLA_ERR_NULL", 2: "EFLA_ERR_SHAPE", 3: "EFLA_ERR_DTYPE",
          4: "EFLA_ERR_UNSUPPORTED", 5: "EFLA_ERR_WORKSPACE", 6: "EFLA_ERR_HIP",
          7: "EFLA_ERR_ALIGN"}

NOALLOC_WS_BYTES = 64 << 20  # EFLA_NOALLOC_WS_BYTES: static workspace of efla_fwd_noalloc

# Every symbol include/efla.h declares.
EXPORTS = ["efla_abi_version", "efla_status_str", "efla_check_problem", "efla_workspace_bytes",
           "efla_saved_bytes", "efla_get_saved_layout", "efla_prep", "efla_chunk_ut",
           "efla_fwd", "efla_fwd_state", "efla_fwd_noalloc", "efla_fwd_gated", "efla_bwd", "efla_bwd_state",
           "efla_bwd_gated",
           "efla_decode", "efla_decode_gated",
           "efla_profile_enable", "efla_profile_read", "efla_profile_reset"]


class EflaProblem(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("H", ctypes.c_int32), ("T", ctypes.c_int32),
                ("dk", ctypes.c_int32), ("dv", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("chunk", ctypes.c_int32), ("scale", ctypes.c_float),
                ("cu_seqlens", ctypes.c_void_p), ("n_seqs", ctypes.c_int32), ("mode", ctypes.c_int32),
                ("segments", ctypes.c_int32)]


class EflaSavedLayout(ctypes.Structure):
    _fields_ = [("w", ctypes.c_size_t), ("ut", ctypes.c_size_t), ("states", ctypes.c_size_t),
                ("table", ctypes.c_size_t), ("m", ctypes.c_size_t), ("x", ctypes.c_size_t),
                ("coef", ctypes.c_size_t), ("cum", ctypes.c_size_t), ("segp", ctypes.c_size_t),
                ("total", ctypes.c_size_t), ("n_chunk_slots", ctypes.c_int64)]


class EflaError(RuntimeError):
    def __init__(self, fn, code):
        self.code = code
        super().__init__("%s failed: %s (%d)" % (fn, STATUS.get(code, "?"), code))


_lib = None


def lib():
    """The loaded library (raises if libefla.so is missing)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError("libefla.so is not built (%s); run python -m delta_rule_sequence_amd.build"
                          % LIB_PATH)
    L = ctypes.CDLL(LIB_PATH)
    P = ctypes.POINTER(EflaProblem)
    vp, sz, st = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int
    fp = ctypes.POINTER(ctypes.c_float)
    L.efla_abi_version.restype = ctypes.c_int
    L.efla_abi_version.argtypes = []
    L.efla_status_str.restype = ctypes.c_char_p
    L.efla_status_str.argtypes = [st]
    L.efla_check_problem.restype = st
    L.efla_check_problem.argtypes = [P]
    L.efla_workspace_bytes.restype = sz
    L.efla_workspace_bytes.argtypes = [P, ctypes.c_int]
    L.efla_saved_bytes.restype = sz
    L.efla_saved_bytes.argtypes = [P]
    L.efla_get_saved_layout.restype = st
    L.efla_get_saved_layout.argtypes = [P, ctypes.POINTER(EflaSavedLayout)]
    L.efla_prep.restype = st
    L.efla_prep.argtypes = [P, vp, vp, fp, fp, fp, fp, vp]
    L.efla_chunk_ut.restype = st
    L.efla_chunk_ut.argtypes = [P, vp, vp, vp, vp, vp, vp, sz, vp]
    L.efla_fwd.restype = st
    L.efla_fwd.argtypes = [P, vp, vp, vp, vp, vp, vp, sz, vp, sz, vp]
    L.efla_bwd.restype = st
    L.efla_bwd.argtypes = [P, vp, vp, vp, vp, vp, vp, sz, vp, vp, vp, vp, vp, sz, vp]
    L.efla_fwd_state.restype = st
    L.efla_fwd_state.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp, sz, vp]
    L.efla_bwd_state.restype = st
    L.efla_bwd_state.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp, vp, vp, vp, vp, vp,
                                 sz, vp]
    L.efla_fwd_noalloc.restype = st
    L.efla_fwd_noalloc.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp]
    L.efla_decode.restype = st
    L.efla_decode.argtypes = [P, vp, vp, vp, vp, vp, vp, vp]
    L.efla_fwd_gated.restype = st
    L.efla_fwd_gated.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp, sz, vp]
    L.efla_bwd_gated.restype = st
    L.efla_bwd_gated.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp, vp, vp, vp, vp, vp,
                                 vp, sz, vp]
    L.efla_decode_gated.restype = st
    L.efla_decode_gated.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp]
    L.efla_profile_enable.restype = st
    L.efla_profile_enable.argtypes = [ctypes.c_int]
    L.efla_profile_read.restype = ctypes.c_int
    L.efla_profile_read.argtypes = [ctypes.c_char_p, ctypes.c_int, ctypes.POINTER(ctypes.c_int64),
                                    ctypes.POINTER(ctypes.c_double), ctypes.c_int]
    L.efla_profile_reset.restype = None
    L.efla_profile_reset.argtypes = []
    _lib = L
    return L


def check(fn, code):
    if code != 0:
        raise EflaError(fn, code)


def problem(B, H, T, dk, dv, dtype, scale=1.0, cu_seqlens_ptr=None, n_seqs=0, chunk=64,
            mode=EFLA_EXACT, segments=0):
    return EflaProblem(B, H, T, dk, dv, dtype, chunk, scale, cu_seqlens_ptr, n_seqs, mode, segments)
