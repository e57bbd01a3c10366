"""ctypes declarations for libtq.so (the C ABI in include/tq.h).

Loading fails loudly: there is no fallback implementation.  Build the library
first with ``python -m kv_cache_vector_05_amd.build``.
"""
from __future__ import annotations

import ctypes as C
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libtq.so")

TQ_OK, TQ_EINVAL, TQ_EUNSUPPORTED, TQ_ENOMEM, TQ_EHIP = 0, -1, -2, -3, -4
TQ_F32, TQ_BF16 = 0, 1
TQ_ROT_AUTO, TQ_ROT_HADAMARD, TQ_ROT_DENSE, TQ_ROT_NONE = 0, 1, 2, 3
TQ_CORR_QJL, TQ_CORR_SIGN = 0, 1
TQ_OP_ENCODE, TQ_OP_LOGITS, TQ_OP_DECODE = 0, 1, 2


class tq_spec(C.Structure):
    _fields_ = [("d", C.c_int32), ("bits", C.c_int32), ("m", C.c_int32), ("rotation", C.c_int32),
                ("seed", C.c_uint64), ("correction", C.c_int32), ("block", C.c_int32)]


class tq_draws(C.Structure):
    _fields_ = [("sigma", C.c_void_p), ("rot_gauss", C.c_void_p), ("sketch", C.c_void_p)]


class tq_packed(C.Structure):
    _fields_ = [("norm", C.c_void_p), ("rnorm", C.c_void_p), ("codes", C.c_void_p), ("signs", C.c_void_p),
                ("n", C.c_int64)]


class tq_pages(C.Structure):
    _fields_ = [("pages", C.c_void_p), ("page_size", C.c_int32), ("max_pages", C.c_int32), ("n_pages", C.c_int64)]


# exported symbols and their signatures (restype, argtypes)
SIGNATURES = {
    "tq_codebook_tables": (C.c_int32, [C.POINTER(tq_spec), C.POINTER(tq_draws), C.c_void_p, C.c_void_p,
                                       C.c_void_p, C.c_void_p]),
    "tq_codebook_init": (C.c_int32, [C.POINTER(tq_spec), C.POINTER(tq_draws), C.c_void_p,
                                     C.POINTER(C.c_void_p)]),
    "tq_codebook_init_calibrated": (C.c_int32, [C.POINTER(tq_spec), C.POINTER(tq_draws), C.c_void_p, C.c_void_p,
                                                C.c_int32, C.c_void_p, C.POINTER(C.c_void_p)]),
    "tq_calibrate": (C.c_int32, [C.POINTER(tq_spec), C.POINTER(tq_draws), C.c_void_p, C.c_int64, C.c_int32,
                                 C.c_int32, C.c_void_p, C.c_void_p, C.c_int32, C.c_void_p, C.c_void_p]),
    "tq_codebook_get_mu": (C.c_int32, [C.c_void_p, C.c_void_p, C.POINTER(C.c_int32)]),
    "tq_decode_vectors": (C.c_int32, [C.c_void_p, C.POINTER(tq_packed), C.c_int64, C.c_int64, C.c_void_p,
                                      C.c_void_p]),
    "tq_codebook_destroy": (C.c_int32, [C.c_void_p]),
    "tq_codebook_get_spec": (C.c_int32, [C.c_void_p, C.POINTER(tq_spec)]),
    "tq_codebook_export": (C.c_int32, [C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p]),
    "tq_encode_kv": (C.c_int32, [C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, C.c_int32, C.c_int32,
                                 C.c_int32, C.c_int32, C.POINTER(C.c_int64), C.POINTER(C.c_int64), C.c_int32,
                                 C.c_int32, C.c_void_p, C.c_void_p, C.c_int32, C.POINTER(tq_packed),
                                 C.POINTER(tq_packed), C.c_void_p, C.c_size_t, C.c_void_p]),
    "tq_encode_kv_paged": (C.c_int32, [C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, C.c_int32, C.c_int32,
                                       C.c_int32, C.c_int32, C.POINTER(C.c_int64), C.POINTER(C.c_int64), C.c_int32,
                                       C.POINTER(tq_pages), C.c_void_p, C.c_void_p, C.c_int32, C.POINTER(tq_packed),
                                       C.POINTER(tq_packed), C.c_void_p]),
    "tq_append_kv": (C.c_int32, [C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, C.c_int32, C.c_int32, C.c_int32,
                                 C.POINTER(C.c_int64), C.POINTER(C.c_int64), C.c_void_p, C.POINTER(tq_pages),
                                 C.c_int32, C.c_void_p, C.c_void_p, C.c_int32, C.POINTER(tq_packed),
                                 C.POINTER(tq_packed), C.c_void_p]),
    "tq_attn_logits_paged": (C.c_int32, [C.c_void_p, C.c_void_p, C.c_int32, C.POINTER(tq_packed), C.c_int32,
                                         C.c_int32, C.c_int32, C.c_void_p, C.c_void_p, C.POINTER(tq_pages), C.c_void_p,
                                         C.c_void_p, C.c_int32, C.c_int32, C.c_void_p, C.c_void_p, C.c_void_p,
                                         C.c_size_t, C.c_void_p]),
    "tq_attn_decode_paged": (C.c_int32, [C.c_void_p, C.c_void_p, C.c_void_p, C.c_int32, C.POINTER(tq_packed),
                                         C.POINTER(tq_packed), C.c_int32, C.c_int32, C.c_int32, C.c_void_p,
                                         C.c_void_p, C.POINTER(tq_pages), C.c_void_p, C.c_void_p, C.c_int32, C.c_float,
                                         C.c_void_p, C.c_void_p, C.c_size_t, C.c_void_p]),
    "tq_attn_logits": (C.c_int32, [C.c_void_p, C.c_void_p, C.c_int32, C.POINTER(tq_packed), C.c_int32,
                                   C.c_int32, C.c_int32, C.c_int32, C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p,
                                   C.c_int32, C.c_int32, C.c_void_p, C.c_void_p, C.c_void_p, C.c_size_t,
                                   C.c_void_p]),
    "tq_attn_decode": (C.c_int32, [C.c_void_p, C.c_void_p, C.c_void_p, C.c_int32, C.POINTER(tq_packed),
                                   C.POINTER(tq_packed), C.c_int32, C.c_int32, C.c_int32, C.c_int32,
                                   C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, C.c_int32, C.c_float, C.c_void_p,
                                   C.c_void_p, C.c_size_t, C.c_void_p]),
    "tq_attn_decode_noalloc": (C.c_int32, [C.c_void_p, C.c_void_p, C.c_void_p, C.c_int32, C.POINTER(tq_packed),
                                           C.POINTER(tq_packed), C.c_int32, C.c_int32, C.c_int32, C.c_int32,
                                           C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, C.c_int32, C.c_float,
                                           C.c_void_p, C.c_void_p]),
    "tq_workspace_bytes": (C.c_size_t, [C.c_void_p, C.c_void_p, C.c_int32, C.c_int64, C.c_int32, C.c_int32,
                                        C.c_int32, C.c_int32]),
    "tq_plane_words": (C.c_int64, [C.POINTER(tq_spec), C.c_int32]),
    "tq_rope_table": (C.c_int32, [C.c_double, C.c_int32, C.c_int32, C.c_void_p, C.c_void_p]),
    "tq_last_error": (C.c_char_p, []),
    "tq_version": (C.c_char_p, []),
}

_lib = None


def lib():
    """The loaded library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        # TQ_LIBRARY names another build of the same ABI (side-by-side timing)
        path = os.environ.get("TQ_LIBRARY", LIB_PATH)
        if not os.path.exists(path):
            raise ImportError(f"libtq.so is not built ({path}); run python -m kv_cache_vector_05_amd.build")
        L = C.CDLL(path)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


class TQError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"libtq error {code}: {msg}")
        self.code = code


def check(code: int):
    if code != TQ_OK:
        raise TQError(code, lib().tq_last_error().decode())
    return code
