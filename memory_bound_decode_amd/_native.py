"""ctypes declarations of the libmbd C ABI (include/mbd.h).  Marshalling only."""
from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, Structure, c_char_p, c_double, c_int32, c_int64, c_uint16, c_uint64, c_void_p

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmbd.so")

MBD_OK, MBD_EINVAL, MBD_ESHAPE, MBD_EALIGN, MBD_ERANGE, MBD_EFORMAT, MBD_EHIP, MBD_ENOMEM = range(8)
MBD_TERNARY_B128, MBD_INT4_G128, MBD_CASSANDRA, MBD_MX32, MBD_TERNARY_SKIP, MBD_CASSANDRA_MX = 1, 2, 3, 4, 5, 6
MBD_MAX_SECTIONS = 8


class MbdPackParams(Structure):
    _fields_ = [("keep_num", c_int32), ("keep_den", c_int32), ("n_mats", c_int64)]


class MbdSection(Structure):
    _fields_ = [("name", c_char_p), ("data", c_void_p), ("bytes", c_uint64), ("padded_bytes", c_uint64)]


class MbdStats(Structure):
    _fields_ = [
        ("fmt", c_int32), ("n_sym", c_int32), ("M", c_int64), ("K", c_int64),
        ("n_kept", c_int64), ("unary_bits", c_int64), ("n_tiles", c_int64),
        ("bpw", c_double), ("spec_bpw", c_double), ("exp_entropy_bits", c_double),
        ("unary_avg_bits", c_double), ("zero_fraction", c_double),
    ]


class MbdDWeights(Structure):
    _fields_ = [
        ("fmt", c_int32), ("n_sym", c_int32), ("M", c_int64), ("K", c_int64),
        ("n_kept", c_int64), ("n_mats", c_int64), ("sec", c_void_p * MBD_MAX_SECTIONS),
    ]


# name -> (restype, argtypes); every symbol include/mbd.h declares
class MbdEncodePlan(Structure):
    _fields_ = [("n_kept", c_int64), ("unary_bits", c_int64), ("n_tiles", c_int64), ("n_sym", c_int32),
                ("reserved", c_int32), ("bytes", c_uint64 * 8), ("padded_bytes", c_uint64 * 8)]


SIGNATURES = {
    "mbd_pack": (c_int32, [c_int32, POINTER(c_uint16), c_int64, c_int64, c_void_p,
                           POINTER(MbdPackParams), POINTER(c_void_p)]),
    "mbd_packed_sections": (c_int32, [c_void_p, POINTER(MbdSection), c_int32, POINTER(c_int32)]),
    "mbd_packed_stats": (c_int32, [c_void_p, POINTER(MbdStats)]),
    "mbd_validate": (c_int32, [c_void_p]),
    "mbd_packed_free": (None, [c_void_p]),
    "mbd_dequant": (c_int32, [POINTER(MbdDWeights), c_void_p, c_void_p]),
    "mbd_gemv": (c_int32, [POINTER(MbdDWeights), c_void_p, c_int32, c_void_p, c_void_p]),
    "mbd_moe_workspace_bytes": (c_int32, [c_int64, c_int32, c_int32, POINTER(c_uint64)]),
    "mbd_moe_gemv": (c_int32, [POINTER(MbdDWeights), c_void_p, c_int32, c_int32, c_void_p, c_int32,
                               c_void_p, c_void_p, c_uint64, c_void_p]),
    "mbd_moe_gemv_noalloc": (c_int32, [POINTER(MbdDWeights), c_void_p, c_int32, c_int32, c_void_p, c_int32,
                                       c_void_p, c_void_p]),
    "mbd_spec_decode": (c_int32, [POINTER(MbdDWeights), c_void_p, c_void_p]),
    "mbd_spec_gemv": (c_int32, [POINTER(MbdDWeights), c_void_p, c_int32, c_void_p, c_void_p]),
    "mbd_verify_restore": (c_int32, [POINTER(MbdDWeights), c_void_p, c_void_p]),
    "mbd_encode_workspace_bytes": (c_int32, [c_int64, POINTER(c_uint64)]),
    "mbd_encode_plan": (c_int32, [c_void_p, c_void_p, c_int64, c_int64, c_int32, c_int32, c_void_p, c_uint64,
                                  POINTER(MbdEncodePlan), c_void_p]),
    "mbd_encode_cassandra": (c_int32, [c_void_p, c_void_p, c_int64, c_int64, c_int32, c_int32,
                                       POINTER(MbdEncodePlan), POINTER(c_void_p), c_void_p, c_uint64, c_void_p]),
    "mbd_probe_stream_read": (c_int32, [c_void_p, c_uint64, c_void_p, c_int32, c_int32, c_void_p]),
    "mbd_status_str": (c_char_p, [c_int32]),
    "mbd_last_error": (c_char_p, []),
}

_lib = None


def lib() -> ctypes.CDLL:
    """The loaded libmbd; raises if it has not been built (there is no fallback)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError("libmbd.so is not built (%s); run __graft_entry__.build()" % LIB_PATH)
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


class MbdError(RuntimeError):
    def __init__(self, status: int, where: str):
        L = lib()
        self.status = status
        msg = L.mbd_last_error().decode(errors="replace")
        super().__init__("%s: %s (%s)" % (where, L.mbd_status_str(status).decode(), msg))


def check(status: int, where: str) -> None:
    if status != MBD_OK:
        raise MbdError(status, where)
