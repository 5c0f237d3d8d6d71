"""ctypes declarations of the C ABI in include/cfr.h (argument marshalling only)."""
from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, c_char_p, c_int32, c_int64, c_uint8, c_uint16, c_uint64, c_void_p

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libcfr.so")

CFR_OK, CFR_EINVAL, CFR_ENOMEM, CFR_EHIP, CFR_EUNSUPPORTED, CFR_ESOLVER = 0, -1, -2, -3, -4, -5


class CfrConfig(ctypes.Structure):
    _fields_ = [("hidden", c_int32), ("n_experts", c_int32), ("inter", c_int32), ("top", c_int32),
                ("rank", c_int32), ("n_screen", c_int32), ("max_batch", c_int32),
                ("device", c_int32), ("rot_seed", c_uint64), ("ranking", c_int32),
                ("exact_bits", c_int32)]


class CfrSizes(ctypes.Structure):
    _fields_ = [("n_blocks", c_int32), ("half_bytes", c_int32), ("unit_bytes", c_int32),
                ("n_cand", c_int32), ("codes_bytes", c_int64), ("scales_count", c_int64),
                ("norms_count", c_int64), ("u_count", c_int64), ("b_count", c_int64),
                ("weights_bytes", c_int64)]


class CfrReadStats(ctypes.Structure):
    _fields_ = [("codes", c_int64), ("scales", c_int64), ("norms", c_int64), ("rho", c_int64),
                ("exact", c_int64), ("b", c_int64), ("u", c_int64), ("total", c_int64),
                ("dense", c_int64)]


_P = c_void_p
# name -> (restype, argtypes); every symbol declared in include/cfr.h
SIGNATURES = {
    "cfr_sizes_of": (c_int32, [POINTER(CfrConfig), POINTER(CfrSizes)]),
    "cfr_read_bytes": (c_int32, [POINTER(CfrConfig), c_int32, POINTER(CfrReadStats)]),
    "cfr_read_bytes_batch": (c_int32, [POINTER(CfrConfig), c_int32, c_int32, _P, _P, _P,
                                       POINTER(CfrReadStats)]),
    "cfr_read_bytes_shared": (c_int32, [POINTER(CfrConfig), c_int32, _P, _P, c_int32, POINTER(CfrReadStats)]),
    "cfr_build_reader": (c_int32, [POINTER(CfrConfig), _P, _P, _P, _P, POINTER(c_void_p)]),
    "cfr_build_reader_q4": (c_int32, [POINTER(CfrConfig), _P, _P, POINTER(c_void_p)]),
    "cfr_reader_decode": (c_int32, [_P, _P, _P, _P, c_int32, c_int32, _P, _P]),
    "cfr_reader_decode_residual": (c_int32, [_P, _P, _P, _P, c_int32, c_int32, _P, _P, _P]),
    "cfr_reader_decode_noalloc": (c_int32, [_P, _P, _P, _P, c_int32, c_int32, _P, _P]),
    "cfr_reader_decode_shared": (c_int32, [_P, _P, _P, _P, c_int32, c_int32, _P, _P, _P, _P, _P]),
    "cfr_reader_decode_debug": (c_int32, [_P, _P, _P, _P, c_int32, c_int32, _P, _P, _P, _P, _P,
                                          _P, _P, _P]),
    "cfr_reader_decode_profile": (c_int32, [_P, _P, _P, _P, c_int32, c_int32, _P, _P, _P]),
    "cfr_reader_decode_stage": (c_int32, [_P, c_int32, _P, _P, _P, c_int32, c_int32, _P, _P]),
    "cfr_reader_route": (c_int32, [_P, _P, c_int32, ctypes.c_float, _P, _P, _P, _P]),
    "cfr_dense_decode": (c_int32, [_P, _P, _P, _P, c_int32, _P, _P]),
    "cfr_dense_decode_residual": (c_int32, [_P, _P, _P, _P, c_int32, _P, _P, _P]),
    "cfr_reader_export": (c_int32, [_P, _P, _P, _P, _P, _P, _P, _P]),
    "cfr_pack_host": (c_int32, [POINTER(CfrConfig), _P, _P, _P, _P, _P, _P, _P]),
    "cfr_reader_clone": (c_int32, [_P, POINTER(c_void_p)]),
    "cfr_reader_config": (c_int32, [_P, POINTER(CfrConfig)]),
    "cfr_reader_status": (c_int32, [_P, POINTER(c_int32)]),
    "cfr_reader_free": (None, [_P]),
    "cfr_last_error": (c_char_p, []),
}

_lib = None


class CfrError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"cfr error {code}: {msg}")
        self.code = code


def load():
    """Load the in-tree libcfr.so; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                           "`python -m calibration_free_channel_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def check(rc):
    if rc != CFR_OK:
        raise CfrError(rc, load().cfr_last_error().decode("utf-8", "replace"))
    return rc
