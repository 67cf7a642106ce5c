"""ctypes binding of ``libtq.so`` (the C ABI in include/tq.h).

Argument marshalling only.  Loading fails loudly when the library has not
been built: there is no fallback implementation.
"""

from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libtq.so")

TQ_F32, TQ_F16, TQ_BF16 = 0, 1, 2

_STATUS = {
    0: "ok",
    1: "invalid argument",
    2: "unsupported configuration",
    3: "misaligned pointer",
    4: "workspace too small",
    5: "HIP runtime error",
    6: "no gfx950 device",
}

#: every function include/tq.h declares, with (restype, argtypes)
_c = ctypes
SIGNATURES = {
    "tq_status_string": (_c.c_char_p, [_c.c_int]),
    "tq_last_hip_error": (_c.c_int, []),
    "tq_row_bytes": (_c.c_size_t, [_c.c_int, _c.c_int]),
    "tq_codebook": (_c.c_int, [_c.c_int, _c.c_int, _c.c_void_p, _c.c_void_p]),
    "tq_rht_signs": (_c.c_int, [_c.c_uint64, _c.c_int, _c.c_void_p]),
    "tq_ctx_create": (_c.c_int, [_c.c_int, _c.c_uint64, _c.POINTER(_c.c_void_p)]),
    "tq_ctx_destroy": (_c.c_int, [_c.c_void_p]),
    "tq_write_kv": (
        _c.c_int,
        [_c.c_void_p, _c.c_void_p, _c.c_int, _c.c_int64, _c.c_int, _c.c_void_p, _c.c_int64,
         _c.c_int, _c.c_void_p, _c.c_int, _c.c_void_p, _c.c_void_p],
    ),
    "tq_write_kv_pair": (
        _c.c_int,
        [_c.c_void_p, _c.c_void_p, _c.c_void_p, _c.c_int, _c.c_int64, _c.c_int, _c.c_void_p, _c.c_int,
         _c.c_void_p, _c.c_int, _c.c_int64, _c.c_int, _c.c_void_p, _c.c_void_p, _c.c_void_p],
    ),
    "tq_prod_row_bytes": (_c.c_size_t, [_c.c_int, _c.c_int]),
    "tq_write_kv_prod": (
        _c.c_int,
        [_c.c_void_p, _c.c_void_p, _c.c_int, _c.c_int64, _c.c_int, _c.c_void_p, _c.c_int64,
         _c.c_int, _c.c_void_p, _c.c_int, _c.c_void_p, _c.c_void_p, _c.c_void_p],
    ),
    "tq_prod_scores_workspace_bytes": (_c.c_size_t, [_c.c_int, _c.c_int]),
    "tq_prod_scores": (
        _c.c_int,
        [_c.c_void_p, _c.c_void_p, _c.c_int, _c.c_int, _c.c_int, _c.c_int, _c.c_void_p, _c.c_int,
         _c.c_int64, _c.c_int, _c.c_void_p, _c.c_int, _c.c_void_p, _c.c_int, _c.c_void_p,
         _c.c_void_p, _c.c_void_p, _c.c_size_t, _c.c_void_p],
    ),
    "tq_decompress_kv": (
        _c.c_int,
        [_c.c_void_p, _c.c_void_p, _c.c_int64, _c.c_int, _c.c_int, _c.c_int, _c.c_void_p, _c.c_int64,
         _c.c_void_p, _c.c_int, _c.c_void_p, _c.c_void_p],
    ),
    "tq_decode_kernel": (_c.c_char_p, [_c.c_int, _c.c_int, _c.c_int, _c.c_int, _c.c_int, _c.c_int]),
    "tq_decode_workspace_bytes": (
        _c.c_size_t, [_c.c_void_p, _c.c_int, _c.c_int, _c.c_int, _c.c_int, _c.c_int]),
    "tq_paged_decode": (
        _c.c_int,
        [_c.c_void_p, _c.c_void_p, _c.c_int, _c.c_int, _c.c_int, _c.c_int,
         _c.c_void_p, _c.c_int, _c.c_void_p, _c.c_int, _c.c_int64, _c.c_int,
         _c.c_void_p, _c.c_int, _c.c_void_p, _c.c_int, _c.c_float,
         _c.c_void_p, _c.c_void_p, _c.c_size_t, _c.c_void_p],
    ),
    "tq_paged_decode_append": (
        _c.c_int,
        [_c.c_void_p, _c.c_void_p, _c.c_int, _c.c_int, _c.c_int, _c.c_int,
         _c.c_void_p, _c.c_void_p, _c.c_int,
         _c.c_void_p, _c.c_int, _c.c_void_p, _c.c_int, _c.c_int64, _c.c_int,
         _c.c_void_p, _c.c_int, _c.c_void_p, _c.c_int, _c.c_float,
         _c.c_void_p, _c.c_void_p, _c.c_size_t, _c.c_void_p, _c.c_void_p],
    ),
    "tq_hybrid_workspace_bytes": (
        _c.c_size_t, [_c.c_void_p, _c.c_int, _c.c_int, _c.c_int, _c.c_int, _c.c_int]),
    "tq_paged_decode_hybrid": (
        _c.c_int,
        [_c.c_void_p, _c.c_void_p, _c.c_int, _c.c_int, _c.c_int, _c.c_int,
         _c.c_void_p, _c.c_int, _c.c_void_p, _c.c_int, _c.c_int64, _c.c_int,
         _c.c_void_p, _c.c_int, _c.c_void_p, _c.c_int,
         _c.c_void_p, _c.c_void_p, _c.c_int, _c.c_int, _c.c_void_p, _c.c_float,
         _c.c_void_p, _c.c_void_p, _c.c_size_t, _c.c_void_p],
    ),
    "tq_prefill_workspace_bytes": (
        _c.c_size_t, [_c.c_void_p, _c.c_int, _c.c_int, _c.c_int, _c.c_int, _c.c_int, _c.c_int]),
    "tq_paged_prefill": (
        _c.c_int,
        [_c.c_void_p, _c.c_void_p, _c.c_int, _c.c_int, _c.c_int, _c.c_void_p, _c.c_int, _c.c_int,
         _c.c_void_p, _c.c_int, _c.c_void_p, _c.c_int, _c.c_int64, _c.c_int,
         _c.c_void_p, _c.c_int, _c.c_void_p, _c.c_int, _c.c_float,
         _c.c_void_p, _c.c_void_p, _c.c_size_t, _c.c_void_p],
    ),
    "tq_paged_decode_noalloc": (
        _c.c_int,
        [_c.c_void_p, _c.c_void_p, _c.c_int, _c.c_int, _c.c_int, _c.c_int,
         _c.c_void_p, _c.c_int, _c.c_void_p, _c.c_int, _c.c_int64, _c.c_int,
         _c.c_void_p, _c.c_int, _c.c_void_p, _c.c_int, _c.c_float,
         _c.c_void_p, _c.c_void_p],
    ),
}


class TQError(RuntimeError):
    """A call into the library failed (mirrors the pages' IntegrationError)."""


_lib = None


def lib():
    """The loaded library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise TQError(
                f"{LIB_PATH} is missing: build it with `python -m paged_decode_attention_tq_amd.build`"
            )
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def check(status: int, what: str):
    if status != 0:
        msg = _STATUS.get(status, f"status {status}")
        if status == 5:
            msg += f" (hipError {lib().tq_last_hip_error()})"
        if status in (1, 2, 3):
            raise ValueError(f"{what}: {msg}")
        raise TQError(f"{what}: {msg}")
