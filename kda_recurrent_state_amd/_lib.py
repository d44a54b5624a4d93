"""ctypes view of libkda's C ABI (include/kda.h).  Argument marshalling only."""
from __future__ import annotations

import ctypes
import os

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG_DIR, "libkda.so")

KDA_F32, KDA_BF16 = 0, 1
KDA_I32, KDA_I64 = 0, 1
KDA_OK = 0
STATUS_NAMES = {0: "KDA_OK", 1: "KDA_E_NULL", 2: "KDA_E_DTYPE", 3: "KDA_E_SHAPE", 4: "KDA_E_LAYOUT",
                5: "KDA_E_OVERLAP", 6: "KDA_E_UNSUPPORTED", 7: "KDA_E_WORKSPACE", 8: "KDA_E_ALIAS",
                9: "KDA_E_HIP"}
EXPORTED = ("kda_state_gather", "kda_state_scatter", "kda_chunk_prefill", "kda_chunk_prefill_workspace_size",
            "kda_chunk_prefill_noalloc",
            "kda_recurrent_decode", "kda_ckpt_quantize_scatter", "kda_ckpt_dequantize_gather",
            "kda_status_string", "kda_last_error_detail")


class StateCache(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("dtype", ctypes.c_int), ("num_rows", ctypes.c_int64),
                ("H", ctypes.c_int64), ("V", ctypes.c_int64), ("K", ctypes.c_int64),
                ("stride", ctypes.c_int64 * 4)]


class PrefillArgs(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int64), ("N", ctypes.c_int64), ("H", ctypes.c_int64), ("K", ctypes.c_int64),
                ("V", ctypes.c_int64),
                ("q", ctypes.c_void_p), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p), ("qkv_dtype", ctypes.c_int),
                ("g", ctypes.c_void_p), ("beta", ctypes.c_void_p), ("beta_dtype", ctypes.c_int),
                ("cu_seqlens", ctypes.c_void_p),
                ("initial_state", ctypes.c_void_p), ("initial_dtype", ctypes.c_int),
                ("out", ctypes.c_void_p),
                ("final_state", ctypes.c_void_p), ("final_dtype", ctypes.c_int),
                ("scale", ctypes.c_float), ("use_qk_l2norm", ctypes.c_int),
                ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_size_t),
                ("ckpt_interval", ctypes.c_int64), ("ckpt_cu", ctypes.c_void_p), ("ckpt_states", ctypes.c_void_p),
                ("num_ckpt", ctypes.c_int64), ("ckpt_dtype", ctypes.c_int)]


class DecodeArgs(ctypes.Structure):
    _fields_ = [("N", ctypes.c_int64), ("H", ctypes.c_int64), ("K", ctypes.c_int64), ("V", ctypes.c_int64),
                ("q", ctypes.c_void_p), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p), ("qkv_dtype", ctypes.c_int),
                ("g", ctypes.c_void_p), ("beta", ctypes.c_void_p), ("beta_dtype", ctypes.c_int),
                ("state_indices", ctypes.c_void_p), ("index_type", ctypes.c_int),
                ("out", ctypes.c_void_p), ("scale", ctypes.c_float), ("use_qk_l2norm", ctypes.c_int)]


class Int8Store(ctypes.Structure):
    _fields_ = [("qdata", ctypes.c_void_p), ("scale", ctypes.c_void_p), ("num_slots", ctypes.c_int64),
                ("H", ctypes.c_int64), ("V", ctypes.c_int64), ("K", ctypes.c_int64),
                ("qdata_stride0", ctypes.c_int64), ("scale_stride0", ctypes.c_int64)]


class KDAError(RuntimeError):
    def __init__(self, func: str, status: int, detail: str = ""):
        self.status = status
        msg = "%s failed: %s" % (func, STATUS_NAMES.get(status, str(status)))
        if detail:
            msg += " (%s)" % detail
        super().__init__(msg)


_lib = None


def load_library(path: str = LIB_PATH):
    """Load libkda.so.  There is no fallback: a missing library is an error."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError("libkda.so not found at %s; build it with `python -m kda_recurrent_state_amd.build` "
                          "(or __graft_entry__.build())" % path)
    lib = ctypes.CDLL(path)
    vp, i64 = ctypes.c_void_p, ctypes.c_int64
    lib.kda_state_gather.argtypes = [ctypes.POINTER(StateCache), vp, ctypes.c_int, i64, vp, vp, vp]
    lib.kda_state_gather.restype = ctypes.c_int
    lib.kda_state_scatter.argtypes = [ctypes.POINTER(StateCache), vp, ctypes.c_int, i64, vp, vp]
    lib.kda_state_scatter.restype = ctypes.c_int
    lib.kda_chunk_prefill.argtypes = [ctypes.POINTER(PrefillArgs), vp]
    lib.kda_chunk_prefill.restype = ctypes.c_int
    lib.kda_chunk_prefill_noalloc.argtypes = [ctypes.POINTER(PrefillArgs), vp]
    lib.kda_chunk_prefill_noalloc.restype = ctypes.c_int
    lib.kda_recurrent_decode.argtypes = [ctypes.POINTER(StateCache), ctypes.POINTER(DecodeArgs), vp]
    lib.kda_recurrent_decode.restype = ctypes.c_int
    lib.kda_ckpt_quantize_scatter.argtypes = [ctypes.POINTER(Int8Store), vp, ctypes.c_int, i64, vp, ctypes.c_int, vp]
    lib.kda_ckpt_quantize_scatter.restype = ctypes.c_int
    lib.kda_ckpt_dequantize_gather.argtypes = [ctypes.POINTER(Int8Store), vp, ctypes.c_int, i64, vp, vp, ctypes.c_int,
                                               vp]
    lib.kda_ckpt_dequantize_gather.restype = ctypes.c_int
    lib.kda_chunk_prefill_workspace_size.argtypes = [i64, i64, i64, i64, i64]
    lib.kda_chunk_prefill_workspace_size.restype = ctypes.c_size_t
    lib.kda_status_string.argtypes = [ctypes.c_int]
    lib.kda_status_string.restype = ctypes.c_char_p
    lib.kda_last_error_detail.argtypes = []
    lib.kda_last_error_detail.restype = ctypes.c_char_p
    _lib = lib
    return lib


def check(func: str, status: int) -> None:
    if status != KDA_OK:
        detail = ""
        if status == 9:
            detail = (_lib.kda_last_error_detail() or b"").decode(errors="replace")
        raise KDAError(func, status, detail)
