"""ctypes loader for libspattn.so (the gfx950 HIP library built in-tree)."""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libspattn.so")
HEADER_PATH = os.path.join(os.path.dirname(HERE), "include", "spattn.h")

_lib = None

c_int, c_float, c_size_t, c_int64, c_void_p = (ctypes.c_int, ctypes.c_float, ctypes.c_size_t,
                                               ctypes.c_int64, ctypes.c_void_p)

_SIGNATURES = {
    "prepare_seqlens": (c_int, [c_void_p, c_void_p, c_int, c_int, c_void_p, c_void_p, c_void_p,
                                c_void_p, c_void_p, c_void_p]),
    "kv_cache_append": (c_int, [c_void_p, c_void_p, c_int, c_void_p, c_void_p, c_int, c_int,
                                c_void_p, c_void_p, c_int, c_void_p, c_int, c_int, c_int,
                                c_void_p, c_void_p, c_int, c_int, c_void_p, c_void_p, c_void_p]),
    "prepare_and_append": (c_int, [c_void_p, c_void_p, c_int, c_int, c_void_p, c_void_p, c_void_p,
                                   c_void_p, c_void_p, c_void_p, c_int, c_void_p, c_void_p, c_int,
                                   c_void_p, c_int, c_int, c_int, c_void_p, c_void_p, c_int, c_int,
                                   c_void_p, c_void_p, c_void_p]),
    "qkv_prologue": (c_int, [c_void_p, c_void_p, c_void_p, c_void_p, c_int, c_void_p, c_void_p,
                             c_int, c_int, c_int, c_int, c_int, c_int, c_void_p, c_void_p,
                             c_float, c_int, c_int, c_void_p, c_void_p, c_int, c_void_p,
                             c_void_p, c_void_p, c_void_p, c_void_p, c_int, c_void_p, c_int,
                             c_int, c_int, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p]),
    "topk_select": (c_int, [c_void_p, c_int, c_void_p, c_void_p, c_int, c_int, c_int, c_int, c_int,
                            c_void_p, c_int, c_void_p, c_void_p, c_void_p]),
    "attention_workspace_bytes": (c_size_t, [c_int, c_int, c_int, c_int, c_int, c_int, c_int,
                                             c_int, c_int, c_int, c_int]),
    "paged_attention_fwd": (c_int, [c_void_p, c_int, c_void_p, c_void_p, c_int, c_void_p, c_int,
                                    c_int, c_int, c_void_p, c_void_p, c_void_p, c_void_p, c_int,
                                    c_int, c_int, c_int, c_int, c_int, c_int, c_float, c_int,
                                    c_int, c_void_p, c_void_p, c_void_p, c_size_t, c_void_p,
                                    c_void_p]),
    "paged_decode_step": (c_int, [c_void_p, c_void_p, c_int, c_int, c_void_p, c_void_p, c_void_p,
                                  c_void_p, c_void_p, c_int, c_void_p, c_void_p, c_int, c_void_p,
                                  c_int, c_int, c_int, c_void_p, c_void_p, c_int, c_int, c_int,
                                  c_int, c_int, c_float, c_int, c_void_p, c_void_p, c_void_p,
                                  c_size_t, c_void_p, c_void_p, c_void_p]),
    "paged_decode_step_noalloc": (c_int, [c_void_p, c_void_p, c_int, c_int, c_void_p, c_void_p,
                                          c_void_p, c_void_p, c_void_p, c_int, c_void_p, c_void_p,
                                          c_int, c_void_p, c_int, c_int, c_int, c_void_p, c_void_p,
                                          c_int, c_int, c_int, c_int, c_int, c_float, c_int,
                                          c_void_p, c_void_p, c_void_p, c_void_p, c_void_p]),
    "sparse_attention_fwd": (c_int, [c_void_p, c_int, c_int, c_void_p, c_void_p, c_int, c_void_p,
                                     c_int, c_int, c_int, c_void_p, c_void_p, c_void_p, c_void_p,
                                     c_int, c_int, c_int, c_void_p, c_void_p, c_int, c_int,
                                     c_void_p, c_void_p, c_int, c_int, c_int64, c_int, c_int,
                                     c_int, c_float, c_void_p, c_void_p, c_void_p, c_size_t,
                                     c_void_p, c_void_p]),
}


def load():
    """Load libspattn.so; raises if it has not been built (there is no fallback)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with `python -m selected_token_sparse_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in _SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib
