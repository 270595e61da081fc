"""ctypes view of libhmm.so (declarations mirror include/hmm.h).

The library is built in-tree by ``mixture_experts_ffn_int32_amd.build``.  If it
is missing, every call raises: there is no fallback path.
"""

import ctypes
import os
import threading

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libhmm.so")

HMM_OK = 0
HMM_ERR_NULL_POINTER = 1
HMM_ERR_BAD_SHAPE = 2
HMM_ERR_BAD_DTYPE = 3
HMM_ERR_MISALIGNED = 4
HMM_ERR_UNSUPPORTED = 5
HMM_ERR_WORKSPACE_TOO_SMALL = 6
HMM_ERR_EXPERT_ID_OUT_OF_RANGE = 7
HMM_ERR_HIP = 8
HMM_ERR_TIMEOUT = 9

HMM_BF16, HMM_F32, HMM_FP8_E4M3, HMM_MXFP8_E4M3, HMM_FP8_E4M3_GROUP = 0, 1, 2, 3, 4
HMM_FLAG_VALIDATE_IDS = 1
HMM_FLAG_TILES_LARGE = 2
HMM_FLAG_TILES_NARROW = 4
HMM_FLAG_FUSED_FORWARD = 8
HMM_FLAG_SERIAL_BACKWARD = 16
HMM_FLAG_FP8_BACKWARD = 32
TILE_FLAGS = {"auto": 0, "large": HMM_FLAG_TILES_LARGE, "narrow": HMM_FLAG_TILES_NARROW}

# every symbol include/hmm.h declares
EXPORTS = (
    "hmm_forward_sizes", "hmm_saved_layout_of", "hmm_forward", "hmm_backward_sizes", "hmm_backward",
    "hmm_route_workspace_size", "hmm_route", "hmm_status_string", "hmm_last_error_message", "hmm_build_info",
    "hmm_profile_enable", "hmm_profile_read", "hmm_quant_rows_fp8", "hmm_quant_cols_workspace_size",
    "hmm_quant_cols_fp8", "hmm_forward_shared", "hmm_backward_shared", "hmm_quant_rows_mx", "hmm_quant_cols_mx",
    "hmm_quant_rows_group", "hmm_quant_cols_group", "hmm_set_fused_spin_limit", "hmm_forward_noalloc",
)


class Problem(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int64), ("H", ctypes.c_int64), ("I", ctypes.c_int64), ("E", ctypes.c_int64),
                ("K", ctypes.c_int64), ("out_dtype", ctypes.c_int32), ("gmm1_dtype", ctypes.c_int32),
                ("flags", ctypes.c_uint32), ("shared_I", ctypes.c_uint32)]


class SavedLayout(ctypes.Structure):
    _fields_ = [(n, ctypes.c_size_t) for n in
                ("counts", "offsets", "sorted_slot", "row_of_slot", "tok_of_row", "tiles", "h", "a", "aw", "id_error",
                 "shared_offsets", "shared_idx", "shared_ones", "shared_tiles", "shared_h", "shared_a", "total")]


class StageTime(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char * 32), ("launches", ctypes.c_int32), ("ms", ctypes.c_double)]


_lock = threading.Lock()
_lib = None

_P = ctypes.c_void_p
_SZ = ctypes.c_size_t
_PROB = ctypes.POINTER(Problem)
_SIGS = {
    "hmm_forward_sizes": [_PROB, ctypes.POINTER(_SZ), ctypes.POINTER(_SZ)],
    "hmm_saved_layout_of": [_PROB, ctypes.POINTER(SavedLayout)],
    "hmm_forward": [_PROB, _P, _P, _P, _P, _P, _P, _P, _SZ, _P, _SZ, _P],
    "hmm_backward_sizes": [_PROB, ctypes.POINTER(_SZ)],
    "hmm_backward": [_PROB, _P, _P, _P, _P, _P, _P, _P, _SZ, _P, _P, _P, _P, _P, _SZ, _P],
    "hmm_forward_noalloc": [_PROB, _P, _P, _P, _P, _P, _P, _P, _SZ, _P],
    "hmm_forward_shared": [_PROB, _P, _P, _P, _P, _P, _P, _P, _P, _P, _SZ, _P, _SZ, _P],
    "hmm_backward_shared": [_PROB, _P, _P, _P, _P, _P, _P, _P, _P, _P, _SZ, _P, _P, _P, _P, _P, _P, _P, _SZ, _P],
    "hmm_route_workspace_size": [_PROB, ctypes.POINTER(_SZ)],
    "hmm_route": [_PROB, _P, _P, _P, _P, _P, _P, _SZ, _P],
    "hmm_quant_rows_fp8": [_P, ctypes.c_int64, ctypes.c_int64, _P, _P, _P],
    "hmm_quant_cols_workspace_size": [ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.POINTER(_SZ)],
    "hmm_quant_cols_fp8": [_P, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, _P, _P, _P, _SZ, _P],
    "hmm_quant_rows_mx": [_P, ctypes.c_int64, ctypes.c_int64, _P, _P, _P],
    "hmm_quant_cols_mx": [_P, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, _P, _P, _P],
    "hmm_quant_rows_group": [_P, ctypes.c_int64, ctypes.c_int64, _P, _P, _P],
    "hmm_quant_cols_group": [_P, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, _P, _P, _P],
    "hmm_status_string": [ctypes.c_int],
    "hmm_set_fused_spin_limit": [ctypes.c_uint32],
    "hmm_last_error_message": [],
    "hmm_build_info": [],
    "hmm_profile_enable": [ctypes.c_int32],
    "hmm_profile_read": [ctypes.POINTER(StageTime), ctypes.c_int32, ctypes.POINTER(ctypes.c_int32),
                         ctypes.POINTER(ctypes.c_int32)],
}


def load(path=None):
    """Load libhmm.so once; raise RuntimeError if it is absent or incomplete."""
    global _lib
    with _lock:
        if _lib is not None and path is None:
            return _lib
        p = path or LIB_PATH
        if not os.path.exists(p):
            raise RuntimeError("libhmm.so is not built (%s missing); run "
                               "`python -m mixture_experts_ffn_int32_amd.build`" % p)
        lib = ctypes.CDLL(p)
        for name in EXPORTS:
            fn = getattr(lib, name)  # AttributeError if a declared symbol is missing
            fn.argtypes = _SIGS[name]
            fn.restype = ctypes.c_char_p if name in ("hmm_status_string", "hmm_last_error_message",
                                                     "hmm_build_info") else ctypes.c_int
        if path is None:
            _lib = lib
        return lib


class HmmError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(message)
        self.status = status


def profile_enable(on=True):
    check(load().hmm_profile_enable(1 if on else 0))


def profile_read():
    """{stage name: (launches, total ms)} since the last read; clears the record."""
    lib = load()
    n, dropped = ctypes.c_int32(), ctypes.c_int32()
    buf = (StageTime * 64)()
    check(lib.hmm_profile_read(buf, 64, ctypes.byref(n), ctypes.byref(dropped)))
    return {buf[i].name.decode(): (buf[i].launches, buf[i].ms) for i in range(min(n.value, 64))}, dropped.value


def check(status):
    """Turn a non-zero hmm_status into a Python exception."""
    if status == HMM_OK:
        return
    lib = load()
    name = lib.hmm_status_string(status).decode()
    msg = "%s: %s" % (name, lib.hmm_last_error_message().decode())
    if status in (HMM_ERR_BAD_SHAPE, HMM_ERR_EXPERT_ID_OUT_OF_RANGE, HMM_ERR_NULL_POINTER, HMM_ERR_MISALIGNED):
        err = ValueError(msg)
    elif status == HMM_ERR_BAD_DTYPE:
        err = TypeError(msg)
    elif status == HMM_ERR_UNSUPPORTED:
        err = NotImplementedError(msg)
    else:
        err = HmmError(status, msg)
    err.status = status
    raise err
