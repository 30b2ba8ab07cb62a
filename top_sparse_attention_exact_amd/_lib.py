"""ctypes loader for libatopk.so (the C ABI of include/atopk.h)."""

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libatopk.so")

_c_i64 = ctypes.c_int64
_c_vp = ctypes.c_void_p
_c_int = ctypes.c_int
_c_size_p = ctypes.POINTER(ctypes.c_size_t)

_SIGNATURES = {
    "atopk_status_str": (ctypes.c_char_p, [_c_int]),
    "atopk_version": (_c_int, []),
    "atopk_stage_events": (_c_int, [ctypes.POINTER(_c_vp), _c_int]),
    "atopk_stage_count": (_c_int, []),
    "atopk_exact_workspace": (_c_int, [_c_int, _c_i64, _c_i64, _c_i64, _c_i64, _c_size_p]),
    "atopk_exact": (_c_int, [_c_vp, _c_int, _c_i64, _c_i64, _c_i64, _c_i64, _c_vp, _c_vp, _c_vp, ctypes.c_size_t, _c_vp]),
    "atopk_bucketed_workspace": (_c_int, [_c_int, _c_i64, _c_i64, _c_i64, _c_i64, _c_i64, _c_i64, _c_int, _c_size_p]),
    "atopk_bucketed": (
        _c_int,
        [_c_vp, _c_int, _c_i64, _c_i64, _c_i64, _c_i64, _c_i64, _c_i64, _c_int, _c_vp, _c_vp, _c_vp, ctypes.c_size_t, _c_vp],
    ),
    "atopk_bucketed_noalloc": (
        _c_int,
        [_c_vp, _c_int, _c_i64, _c_i64, _c_i64, _c_i64, _c_i64, _c_i64, _c_int, _c_vp, _c_vp, _c_vp],
    ),
    "atopk_bucketed_ex_workspace": (
        _c_int, [_c_int, _c_i64, _c_i64, _c_i64, _c_i64, _c_i64, _c_i64, _c_int, _c_int, _c_size_p]
    ),
    "atopk_bucketed_ex": (
        _c_int,
        [_c_vp, _c_int, _c_i64, _c_i64, _c_i64, _c_i64, _c_i64, _c_i64, _c_int, _c_int, _c_vp, _c_vp, _c_vp,
         ctypes.c_size_t, _c_vp],
    ),
    "atopk_sparse_attn_decode_workspace": (
        _c_int,
        [_c_i64, _c_i64, _c_i64, _c_i64, _c_i64, _c_i64, _c_i64, _c_i64, _c_size_p],
    ),
    "atopk_sparse_attn_decode": (
        _c_int,
        [_c_vp, _c_vp, _c_vp, _c_i64, _c_i64, _c_i64, _c_i64, _c_i64, _c_i64, ctypes.c_float, _c_i64, _c_i64, _c_i64,
         _c_vp, _c_vp, _c_vp, _c_vp, ctypes.c_size_t, _c_vp],
    ),
    "atopk_sparse_attn_rerank_workspace": (
        _c_int, [_c_i64, _c_i64, _c_i64, _c_i64, _c_i64, _c_i64, ctypes.POINTER(ctypes.c_size_t)]),
    "atopk_sparse_attn_rerank": (
        _c_int,
        [_c_vp, _c_vp, _c_vp, _c_i64, _c_i64, _c_i64, _c_i64, _c_i64, _c_i64, ctypes.c_float, _c_vp, _c_i64, _c_i64,
         _c_i64, _c_i64, _c_vp, _c_vp, _c_vp, _c_vp, ctypes.c_size_t, _c_vp],
    ),
    "atopk_expected_recall": (_c_int, [_c_i64, _c_i64, _c_i64, _c_i64, ctypes.POINTER(ctypes.c_double)]),
    "atopk_choose_workspace": (
        _c_int,
        [_c_int, _c_i64, _c_i64, _c_i64, _c_i64, ctypes.c_double, ctypes.POINTER(ctypes.c_size_t)],
    ),
    "atopk_choose": (
        _c_int,
        [_c_vp, _c_int, _c_i64, _c_i64, _c_i64, _c_i64, ctypes.c_double, _c_vp, _c_vp, _c_vp, ctypes.c_size_t, _c_vp,
         ctypes.POINTER(ctypes.c_int64), ctypes.POINTER(ctypes.c_int64), ctypes.POINTER(ctypes.c_double),
         ctypes.POINTER(ctypes.c_float)],
    ),
}

EXPORTED = tuple(_SIGNATURES)

_lib = None


class AtopkError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        super().__init__("%s failed: %s (status %d)" % (where, status_str(status), status))


def lib():
    """The loaded library.  Raises if it was never built: there is no
    fallback implementation."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                "libatopk.so is not built (%s); run `python -m top_sparse_attention_exact_amd.build`" % LIB_PATH
            )
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def status_str(status):
    return lib().atopk_status_str(int(status)).decode()


def check(status, where):
    if status != 0:
        raise AtopkError(status, where)
