"""ctypes view of libmla_verify.so (the C ABI declared in include/mla_verify.h).

Argument marshalling only.  Loading fails loudly if the library is not built.
"""
from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmla_verify.so")
# the same library with the device-side argument checks (MLA_VERIFY_DEBUG; include/mla_verify.h)
DEBUG_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmla_verify_debug.so")
DEBUG_SLOT_OUT_OF_RANGE = 1
DEBUG_NEGATIVE_LENGTH = 2
DEBUG_Q_LEN_OUT_OF_RANGE = 4

MLA_OK = 0
MLA_ERR_INVALID_ARGUMENT = -1
MLA_ERR_UNSUPPORTED = -2
MLA_ERR_OUT_OF_MEMORY = -3
MLA_ERR_HIP = -4
MLA_ERR_SCRATCH_TOO_SMALL = -5
NOALLOC_SCRATCH_BYTES = 40 << 20  # MLA_VERIFY_NOALLOC_SCRATCH_BYTES

FORM_AUTO = 0        # kernel-1 layouts (include/mla_verify.h)
FORM_128ROW = 1
FORM_TWO_STREAM = 2
FORM_FOUR_STREAM = 3
FLAG_BATCH_INVARIANT = 1  # create flags (include/mla_verify.h)

D_QK = 576
D_V = 512

# Every function the header declares, with its ctypes signature.
_P = ctypes.c_void_p
_I32 = ctypes.c_int32


class MlaVerifyConfig(ctypes.Structure):
    _fields_ = [
        ("num_heads", ctypes.c_int32),
        ("d_qk", ctypes.c_int32),
        ("d_v", ctypes.c_int32),
        ("batch", ctypes.c_int32),
        ("max_q_len", ctypes.c_int32),
        ("max_nsplit", ctypes.c_int32),
        ("num_slots", ctypes.c_int64),
        ("sm_scale", ctypes.c_float),
        ("form", ctypes.c_int32),
        ("flags", ctypes.c_int32),
    ]


SIGNATURES = {
    "mla_verify_create": (ctypes.c_int, [ctypes.POINTER(MlaVerifyConfig), ctypes.POINTER(_P)]),
    "mla_verify_run": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _P, _P, _I32, _P]),
    "mla_verify_run_noalloc": (ctypes.c_int, [ctypes.POINTER(MlaVerifyConfig), _P, _P, _P, _P, _P, _P, _P, _I32,
                                              _P]),
    "mla_verify_partials": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _I32, _P]),
    "mla_verify_merge": (ctypes.c_int, [_P, _P, _P, _I32, _I32, _I32, _I32, _P, _P, _P]),
    "mla_verify_compact": (ctypes.c_int, [_P, _P, ctypes.c_int64, _P, ctypes.c_int64, ctypes.c_int64, _P, _P]),
    "mla_verify_build_metadata": (ctypes.c_int, [_P, _I32, _I32, ctypes.c_int64, _P, _P, _P, _I32, _P,
                                                  ctypes.c_int64, _P, _P, _P, _P]),
    "mla_verify_workspace": (ctypes.c_int, [_P, ctypes.POINTER(_P), ctypes.POINTER(ctypes.c_int64),
                                            ctypes.POINTER(_P), ctypes.POINTER(ctypes.c_int64)]),
    "mla_verify_debug_flags": (ctypes.c_int, [_P, ctypes.POINTER(ctypes.c_int32), _I32]),
    "mla_verify_destroy": (ctypes.c_int, [_P]),
    "mla_verify_error_string": (ctypes.c_char_p, [ctypes.c_int]),
}

_libs = {}


class MlaVerifyError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} failed: {error_string(status)} ({status})")
        self.status = status


def load(debug: bool = False) -> ctypes.CDLL:
    """Load the library once (the debug build with debug=True).  Import torch before calling this
    on a GPU so that the library binds to the HIP runtime torch already loaded."""
    path = DEBUG_LIB_PATH if debug else LIB_PATH
    if path not in _libs:
        if not os.path.exists(path):
            raise ImportError(
                f"{path} is not built; run `python -m speculative_decode_mla_amd.build` "
                "(there is no fallback implementation)")
        lib = ctypes.CDLL(path)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _libs[path] = lib
    return _libs[path]


def error_string(status: int) -> str:
    return load().mla_verify_error_string(status).decode()


def check(fn: str, status: int) -> None:
    if status != MLA_OK:
        raise MlaVerifyError(fn, status)
