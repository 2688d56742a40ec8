"""ctypes loader for libsepattn.so and the argument marshalling of its C ABI.

Nothing here computes any part of the method: every step runs in the HIP
kernels behind the C entry points. PyTorch only supplies device memory and
the current HIP stream. If the library is missing or fails to load, every
call raises; there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
import threading

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libsepattn.so")

c_int = ctypes.c_int
c_float = ctypes.c_float
c_vp = ctypes.c_void_p

SEP_OK = 0
SEP_ERR_NULL = -1
SEP_ERR_SHAPE = -2
SEP_ERR_PARAM = -3
SEP_ERR_DTYPE = -4
SEP_ERR_WORKSPACE = -5
SEP_ERR_HIP = -6
SEP_ERR_ALIGN = -7
SEP_F32 = 0
SEP_BF16 = 1


class SepCacheStruct(ctypes.Structure):
    """Mirror of ``sep_cache`` in include/sepattn.h."""
    _fields_ = [
        ("a", ctypes.c_int32), ("s", ctypes.c_int32), ("p", ctypes.c_int32), ("w", ctypes.c_int32),
        ("B", ctypes.c_int32), ("Hkv", ctypes.c_int32), ("D", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
        ("k", c_vp), ("v", c_vp), ("pos", c_vp), ("tok", c_vp), ("state", c_vp),
        ("policy", ctypes.c_int32),
        ("work", c_vp), ("work_bytes", ctypes.c_size_t),
    ]


SIGNATURES = {
    "sep_mask_build": (c_int, [c_vp, c_int, c_int, c_vp, c_int, c_int, c_int, c_vp, c_vp, c_int,
                               c_int, c_vp, c_vp]),
    "sep_index_compact": (c_int, [c_vp, c_int, c_int, c_vp, c_vp, c_vp, c_vp]),
    "sep_attn_prefill": (c_int, [c_vp, c_vp, c_vp, c_int, c_int, c_int, c_int, c_int, c_int, c_vp,
                                 c_vp, c_vp, c_int, c_int, c_float, c_vp, c_vp, c_vp]),
    "sep_attn_prefill_backward": (c_int, [c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_int, c_int, c_int, c_int,
                                          c_int, c_int, c_vp, c_vp, c_vp, c_int, c_int, c_float, c_vp,
                                          c_vp, c_vp, c_vp, c_vp]),
    "sep_attn_prefill_backward_noalloc": (c_int, [c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_int, c_int, c_int, c_int,
                                                  c_int, c_int, c_vp, c_vp, c_vp, c_int, c_int, c_float, c_vp,
                                                  c_vp, c_vp, c_vp]),
    "sep_cache_reset": (c_int, [ctypes.POINTER(SepCacheStruct), c_vp]),
    "sep_cache_update": (c_int, [ctypes.POINTER(SepCacheStruct), c_vp, c_vp, c_vp, c_int, c_vp,
                                 c_int, c_vp]),
    "sep_mask_compact": (c_int, [c_vp, c_int, c_int, c_vp, c_int, c_vp, c_vp, c_vp, c_vp, c_vp]),
    "sep_chunk_workspace_bytes": (ctypes.c_size_t, [ctypes.POINTER(SepCacheStruct), c_int]),
    "sep_decode_work_bytes": (ctypes.c_size_t, [ctypes.POINTER(SepCacheStruct), c_int]),
    "sep_attn_prefill_chunk": (c_int, [c_vp, c_vp, c_vp, c_vp, c_int, c_vp, c_int, ctypes.POINTER(SepCacheStruct),
                                       c_int, c_int, c_float, c_vp, ctypes.c_size_t, c_vp, c_vp, c_vp]),
    "sep_rope_table": (c_int, [ctypes.c_double, c_int, c_int, c_vp, c_vp]),
    "sep_attn_decode_rope": (c_int, [c_vp, c_vp, c_vp, ctypes.POINTER(SepCacheStruct), c_int, c_float, c_vp,
                                     c_int, c_vp, c_vp, c_vp]),
    "sep_attn_decode": (c_int, [c_vp, c_vp, c_vp, ctypes.POINTER(SepCacheStruct), c_int, c_float,
                                c_vp, c_vp, c_vp]),
    "sep_decode_update": (c_int, [c_vp, c_vp, c_vp, c_vp, c_vp, c_int, ctypes.POINTER(SepCacheStruct), c_int,
                                  c_float, c_vp, c_int, c_vp, c_vp, c_vp]),
    "sep_status_string": (ctypes.c_char_p, [c_int]),
    "sep_version": (c_int, []),
}

_lock = threading.Lock()
_lib = None


class SepError(RuntimeError):
    def __init__(self, fn: str, code: int, msg: str):
        super().__init__(f"{fn} returned {code}: {msg}")
        self.code = code


def load() -> ctypes.CDLL:
    """Load the package's own libsepattn.so once; raise if it is not there."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        p = LIB_PATH
        if not os.path.exists(p):
            raise RuntimeError(
                f"libsepattn.so not found at {p}; build it with "
                "`python -m kv_cache_compression_sep_amd.build` (hipcc, gfx950)")
        lib = ctypes.CDLL(p)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
        return lib


def check(fn: str, code: int) -> None:
    if code != SEP_OK:
        msg = load().sep_status_string(code).decode()
        raise SepError(fn, code, msg)
