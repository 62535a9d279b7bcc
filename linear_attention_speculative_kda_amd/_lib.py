"""ctypes binding of libkda.so (the HIP kernels and their C ABI, include/kda.h).

Argument marshalling only: every step of the computation runs in the HIP
kernels. torch tensors supply device memory and the current stream.
The library must be built (``python -m linear_attention_speculative_kda_amd.build``);
there is no fallback of any kind when it is missing.
"""

from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("KDA_LIB", os.path.join(_HERE, "libkda.so"))

KDA_OK = 0
KDA_ERR_METADATA = 8
STATUS_NAMES = {
    0: "KDA_OK", 1: "KDA_ERR_NULL", 2: "KDA_ERR_SHAPE", 3: "KDA_ERR_CAPACITY",
    4: "KDA_ERR_ALIGN", 5: "KDA_ERR_ALIAS", 6: "KDA_ERR_UNSUPPORTED", 7: "KDA_ERR_LAUNCH",
    8: "KDA_ERR_METADATA",
}
ROW_ISSUES = {
    0: "ok", 1: "malformed span", 2: "window longer than max_seqlen", 3: "slot >= num_slots",
    4: "slot shared with an earlier row", 5: "record row out of range",
    6: "record row shared with an earlier row",
}

c_ptr = ctypes.c_void_p


class KdaLayer(ctypes.Structure):
    _fields_ = [
        ("num_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("scale", ctypes.c_float),
        ("has_lower_bound", ctypes.c_int32),
        ("lower_bound", ctypes.c_float),
        ("a_log", c_ptr),
        ("g_bias", c_ptr),
    ]


class KdaTokens(ctypes.Structure):
    _fields_ = [
        ("q", c_ptr), ("k", c_ptr), ("v", c_ptr), ("g", c_ptr), ("beta", c_ptr),
        ("stride_q", ctypes.c_int64), ("stride_k", ctypes.c_int64),
        ("stride_v", ctypes.c_int64), ("stride_g", ctypes.c_int64),
        ("stride_beta", ctypes.c_int64),
        ("cu_seqlens", c_ptr),
        ("num_rows", ctypes.c_int32),
        ("num_tokens", ctypes.c_int32),
        ("max_seqlen", ctypes.c_int32),
    ]


class KdaPool(ctypes.Structure):
    _fields_ = [
        ("state", c_ptr),
        ("slot_stride", ctypes.c_int64),
        ("num_slots", ctypes.c_int32),
        ("state_indices", c_ptr),
    ]


class KdaRecords(ctypes.Structure):
    _fields_ = [
        ("k", c_ptr), ("v", c_ptr), ("g", c_ptr), ("beta", c_ptr),
        ("rows", ctypes.c_int32),
        ("window", ctypes.c_int32),
    ]


class KdaAlign(ctypes.Structure):
    _fields_ = [
        ("block_table", c_ptr),
        ("row_stride", ctypes.c_int64),
        ("width", ctypes.c_int32),
        ("num_computed", c_ptr),
        ("block_size", ctypes.c_int32),
    ]


class KdaSpecTable(ctypes.Structure):
    _fields_ = [
        ("indices", c_ptr),
        ("row_stride", ctypes.c_int64),
        ("cols", ctypes.c_int32),
        ("num_accepted", c_ptr),
    ]


class KdaConvState(ctypes.Structure):
    _fields_ = [
        ("state", c_ptr),
        ("block_stride", ctypes.c_int64), ("dim_stride", ctypes.c_int64),
        ("token_stride", ctypes.c_int64),
        ("num_blocks", ctypes.c_int32),
    ]


class KdaError(RuntimeError):
    def __init__(self, call: str, status: int, message: str):
        super().__init__(f"{call}: {message}")
        self.status = status


_lib = None


def load() -> ctypes.CDLL:
    """Load libkda.so once. Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"libkda.so not found at {LIB_PATH}: build it with "
            "`python -m linear_attention_speculative_kda_amd.build` (hipcc, gfx950)")
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.POINTER
    lib.kda_recurrent.argtypes = [P(KdaLayer), P(KdaTokens), P(KdaPool), c_ptr, c_ptr]
    lib.kda_verify.argtypes = [P(KdaLayer), P(KdaTokens), P(KdaPool), P(KdaRecords), c_ptr,
                               c_ptr, c_ptr]
    lib.kda_recurrent_spec.argtypes = [P(KdaLayer), P(KdaTokens), P(KdaPool), P(KdaSpecTable),
                                       c_ptr, c_ptr]
    lib.kda_commit.argtypes = [P(KdaLayer), c_ptr, ctypes.c_int32, P(KdaPool), P(KdaRecords),
                               c_ptr, c_ptr, c_ptr, c_ptr, c_ptr]
    lib.kda_verify_deferred.argtypes = [P(KdaLayer), P(KdaTokens), P(KdaPool), P(KdaRecords),
                                        c_ptr, P(KdaRecords), c_ptr, c_ptr, c_ptr]
    lib.kda_commit_layers.argtypes = [P(KdaLayer), P(KdaPool), P(KdaRecords), ctypes.c_int32,
                                      c_ptr, ctypes.c_int32, c_ptr, c_ptr, c_ptr, c_ptr,
                                      P(KdaAlign), c_ptr]
    lib.kda_conv_compact.argtypes = [P(KdaConvState), ctypes.c_int32, ctypes.c_int32,
                                     ctypes.c_int32, ctypes.c_int32, c_ptr, ctypes.c_int32, c_ptr,
                                     c_ptr, ctypes.c_int32, P(KdaAlign), c_ptr]
    lib.kda_flush_layers.argtypes = [P(KdaLayer), P(KdaPool), P(KdaRecords), ctypes.c_int32,
                                     ctypes.c_int32, c_ptr, c_ptr, c_ptr]
    for fn in ("kda_recurrent", "kda_recurrent_spec", "kda_verify", "kda_commit", "kda_verify_deferred",
               "kda_commit_layers", "kda_flush_layers", "kda_conv_compact"):
        getattr(lib, fn).restype = ctypes.c_int
    lib.kda_check_rows.argtypes = [c_ptr, ctypes.c_int32, ctypes.c_int32, c_ptr, ctypes.c_int32,
                                   c_ptr, ctypes.c_int32, ctypes.c_int32,
                                   ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_int32)]
    lib.kda_check_rows.restype = ctypes.c_int
    lib.kda_status_string.argtypes = [ctypes.c_int]
    lib.kda_status_string.restype = ctypes.c_char_p
    lib.kda_build_info.argtypes = []
    lib.kda_build_info.restype = ctypes.c_char_p
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load().kda_status_string(int(status)).decode()


def check(call: str, status: int) -> None:
    if status != KDA_OK:
        raise KdaError(call, status, status_string(status))
