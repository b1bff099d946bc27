"""ctypes loader for libspecache.so (the C ABI in include/specache.h).

The library is built in-tree by `python -m decode_attention_bit_kivi_amd.build`
(SPECACHE_LIB may point at another build of the same library).
There is no fallback: if the shared object is missing or does not load, every
call raises.
"""
from __future__ import annotations

import ctypes
import os
import threading

LIB_PATH = os.environ.get("SPECACHE_LIB") or os.path.join(os.path.dirname(os.path.abspath(__file__)),
                                                         "libspecache.so")

ABI_VERSION = 6

SPECACHE_OK = 0
SPECACHE_ERR_INVALID = 1
SPECACHE_ERR_UNSUPPORTED = 2
SPECACHE_ERR_WORKSPACE = 3
SPECACHE_ERR_NOT_PINNED = 4
SPECACHE_ERR_HIP = 5
SPECACHE_ERR_TOO_LARGE = 6
NOALLOC_SCRATCH_BYTES = 128 * 1024 * 1024  # SPECACHE_NOALLOC_SCRATCH_BYTES

EXPORTED = (
    "specache_lowbit_bytes",
    "specache_quantize_pack",
    "specache_quantize_append",
    "specache_offload_fp16",
    "specache_score_topk_workspace_size",
    "specache_score_topk",
    "specache_gather_fp16",
    "specache_gather_reuse",
    "specache_gather_fp16_missing",
    "specache_decode_attn_workspace_size",
    "specache_decode_attn",
    "specache_decode_attn_fp16_workspace_size",
    "specache_decode_attn_fp16",
    "specache_decode_step_workspace_size",
    "specache_decode_step",
    "specache_decode_step_noalloc",
    "specache_gather_stream_create",
    "specache_compute_stream_create",
    "specache_stream_destroy",
    "specache_flag_set",
    "specache_flag_wait",
    "specache_status_string",
    "specache_abi_version",
)


class Shape(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("n_q_heads", ctypes.c_int32),
        ("n_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("seq_len", ctypes.c_int64),
        ("bits", ctypes.c_int32),
        ("group", ctypes.c_int32),
        ("seq_capacity", ctypes.c_int64),
        ("v_bits", ctypes.c_int32),
        ("reserved", ctypes.c_int32),
    ]


class LowBit(ctypes.Structure):
    _fields_ = [
        ("k_codes", ctypes.c_void_p),
        ("k_meta", ctypes.c_void_p),
        ("v_codes", ctypes.c_void_p),
        ("v_meta", ctypes.c_void_p),
    ]


class SpecacheError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {status_string(status)} (status {status})")


_lock = threading.Lock()
_lib = None


def load() -> ctypes.CDLL:
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing; build it with "
                               "`python -m decode_attention_bit_kivi_amd.build`")
        lib = ctypes.CDLL(LIB_PATH)
        P, I, I64, F, SZ = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
        SP, LP = ctypes.POINTER(Shape), ctypes.POINTER(LowBit)
        PSZ = ctypes.POINTER(SZ)
        sig = {
            "specache_lowbit_bytes": (SZ, [SP, PSZ, PSZ, PSZ, PSZ]),
            "specache_quantize_pack": (I, [SP, P, P, LP, P]),
            "specache_quantize_append": (I, [SP, P, P, I64, LP, P]),
            "specache_offload_fp16": (I, [SP, P, P, I64, I64, P, P, P]),
            "specache_score_topk_workspace_size": (SZ, [SP, I, I]),
            "specache_score_topk": (I, [SP, P, I, I, LP, F, I, P, P, P, SZ, P]),
            "specache_gather_fp16": (I, [SP, P, I, P, P, P, P, P]),
            "specache_gather_reuse": (I, [SP, P, I, P, I, P, P, P, P, P, P]),
            "specache_gather_fp16_missing": (I, [SP, P, I, P, P, P, P, P]),
            "specache_decode_attn_workspace_size": (SZ, [SP, I, I, I]),
            "specache_decode_attn": (I, [SP, P, I, LP, P, I, P, P, P, P, I, F, P, P, SZ, P]),
            "specache_decode_attn_fp16_workspace_size": (SZ, [SP, I, I]),
            "specache_decode_attn_fp16": (I, [SP, P, I, P, P, P, P, I, F, P, P, SZ, P]),
            "specache_decode_step_workspace_size": (SZ, [SP, I, I, I, I]),
            "specache_decode_step": (I, [SP, P, I, I, I, LP, P, I, P, P, P, P, I, F, P, I, P, P, P, SZ, P]),
            "specache_decode_step_noalloc": (I, [SP, P, I, I, I, LP, P, I, P, P, P, P, I, F, P, I, P, P, P]),
            "specache_gather_stream_create": (I, [I, ctypes.POINTER(P)]),
            "specache_compute_stream_create": (I, [I, ctypes.POINTER(P)]),
            "specache_stream_destroy": (I, [P]),
            "specache_flag_set": (I, [P, ctypes.c_uint32, P]),
            "specache_flag_wait": (I, [P, ctypes.c_uint32, ctypes.c_uint32, P, P]),
            "specache_status_string": (ctypes.c_char_p, [I]),
            "specache_abi_version": (I, []),
        }
        for name, (res, args) in sig.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        got = lib.specache_abi_version()
        if got != ABI_VERSION:
            raise RuntimeError(f"libspecache ABI version {got}, binding expects {ABI_VERSION}")
        _lib = lib
        return lib


def status_string(status: int) -> str:
    try:
        return load().specache_status_string(status).decode()
    except Exception:
        return "unknown"


def check(status: int, what: str) -> None:
    if status != SPECACHE_OK:
        raise SpecacheError(status, what)
