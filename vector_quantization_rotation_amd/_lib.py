"""ctypes binding of libtq.so: argument marshalling only.

Every computation runs inside the HIP library.  PyTorch supplies device memory
(tensors) and the current HIP stream; nothing here falls back to the CPU: a
missing library raises.
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libtq.so")

TQ_OK, TQ_ERR_INVALID, TQ_ERR_UNSUPPORTED, TQ_ERR_HIP, TQ_ERR_NOMEM, TQ_ERR_WORKSPACE = 0, -1, -2, -3, -4, -5
TQ_MSE, TQ_PROD = 0, 1
TQ_F32, TQ_BF16, TQ_F16 = 0, 1, 2
TQ_LAYOUT_ROWS, TQ_LAYOUT_TILE32 = 0, 1
TQ_NOALLOC_SCRATCH_BYTES = 16 << 20  # the library's fixed workspace of tq_attn_decode_noalloc

# (name, restype, argtypes) for every symbol declared in include/tq.h
_P, _I, _I64, _SZ, _F, _D = C.c_void_p, C.c_int, C.c_int64, C.c_size_t, C.c_float, C.c_double
SIGNATURES = [
    ("tq_codebook_build", _I, [_I, _I, C.POINTER(_D), C.POINTER(_D)]),
    ("tq_quantizer_create", _I, [C.POINTER(_P), _I, _I, _I, C.POINTER(_F), C.POINTER(_F)]),
    ("tq_quantizer_destroy", None, [_P]),
    ("tq_quantizer_info", _I, [_P, C.POINTER(_I), C.POINTER(_I), C.POINTER(_I), C.POINTER(_I), C.POINTER(_SZ)]),
    ("tq_encode_mse", _I, [_P, _P, _I, _I64, _I64, _P, _P, _P]),
    ("tq_encode_prod", _I, [_P, _P, _I, _I64, _I64, _P, _P, _P, _P]),
    ("tq_encode_cache", _I, [_P, _P, _I, _I64, _I64, _I64, _I64, _I64, _I, _P, _P, _P, _P]),
    ("tq_decode", _I, [_P, _P, _P, _P, _I64, _P, _I64, _P]),
    ("tq_score", _I, [_P, _P, _I64, _I64, _P, _P, _P, _I64, _I, _P, _P, _P, _SZ, _P]),
    ("tq_score_ws_bytes", _SZ, [_P, _I64, _I64, _I]),
    ("tq_tile_records", _I, [_P, _P, _I64, _I64, _P, _P]),
    ("tq_attn_decode", _I, [_P, _P, _P, _I, _I, _I, _I, _P, _P, _P, _P, _P, _P, _I, _I64, _P, _F, _P, _P, _SZ, _P]),
    ("tq_attn_decode_ws_bytes", _SZ, [_P, _I, _I, _I, _I64, _I]),
    ("tq_attn_prefill", _I, [_P, _P, _P, _I, _I, _I, _I, _I, _P, _P, _P, _P, _P, _P, _I, _I64, _P, _F, _P, _P, _SZ,
                             _P]),
    ("tq_attn_prefill_ws_bytes", _SZ, [_P, _I, _I, _I, _I, _I64, _I]),
    ("tq_attn_decode_append", _I, [_P, _P, _P, _I, _I, _I, _I, _P, _P, _I, _P, _P, _P, _P, _P, _P, _I, _I64, _P, _F,
                                   _P, _P, _SZ, _P]),
    ("tq_attn_decode_noalloc", _I, [_P, _P, _P, _I, _I, _I, _I, _P, _P, _P, _P, _P, _P, _I, _I64, _P, _F, _P, _P]),
    ("tq_profile_enable", _I, [_I]),
    ("tq_profile_select", _I, [C.c_char_p]),
    ("tq_profile_query", _I, [C.c_char_p, C.POINTER(C.c_double), C.POINTER(C.c_int64)]),
    ("tq_profile_reset", _I, []),
    ("tq_status_str", C.c_char_p, [_I]),
    ("tq_last_hip_error", _I, []),
    ("tq_version", C.c_char_p, []),
]

_lib = None


class TQError(RuntimeError):
    def __init__(self, fn: str, status: int):
        lib = load()
        name = lib.tq_status_str(status).decode()
        extra = f" (hipError {lib.tq_last_hip_error()})" if status == TQ_ERR_HIP else ""
        super().__init__(f"{fn} failed: {name}{extra}")
        self.status = status


def load():
    """Load libtq.so (built in-tree by vector_quantization_rotation_amd.build)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} not found: build it with `python -m vector_quantization_rotation_amd.build`")
    lib = C.CDLL(LIB_PATH)
    for name, res, args in SIGNATURES:
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    _lib = lib
    return lib


def _check(fn: str, status: int):
    if status != TQ_OK:
        raise TQError(fn, status)


def codebook_build(d: int, bits: int):
    """Host Lloyd-Max codebook from the library: (centroids[2^bits], bounds[2^bits-1]) fp64."""
    lib = load()
    L = 1 << bits
    c = np.zeros(L, dtype=np.float64)
    t = np.zeros(max(L - 1, 1), dtype=np.float64)
    _check("tq_codebook_build", lib.tq_codebook_build(d, bits, c.ctypes.data_as(C.POINTER(_D)),
                                                      t.ctypes.data_as(C.POINTER(_D))))
    return c, t[:L - 1]


def profile_enable(on: bool = True):
    _check("tq_profile_enable", load().tq_profile_enable(1 if on else 0))


def profile_select(name: str = ""):
    """Record only launches whose kernel name contains `name` ("" = all)."""
    _check("tq_profile_select", load().tq_profile_select(name.encode()))


def profile_reset():
    _check("tq_profile_reset", load().tq_profile_reset())


def profile_query(name: str = ""):
    """(total milliseconds, launches) of the library kernels whose name contains `name`."""
    ms, n = C.c_double(), C.c_int64()
    _check("tq_profile_query", load().tq_profile_query(name.encode(), C.byref(ms), C.byref(n)))
    return ms.value, n.value
