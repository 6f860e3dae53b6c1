"""ctypes loader of libdsa.so (the C ABI declared in include/dsa.h).

Loading fails loudly when the library has not been built: there is no other
implementation to fall back to.
"""

from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libdsa.so")

c_int, c_int64, c_size_t, c_uint64, c_float = (
    ctypes.c_int, ctypes.c_int64, ctypes.c_size_t, ctypes.c_uint64, ctypes.c_float)
c_void_p, c_char_p = ctypes.c_void_p, ctypes.c_char_p

DSA_OK, DSA_ERR_INVALID_ARG, DSA_ERR_UNSUPPORTED, DSA_ERR_WORKSPACE, DSA_ERR_HIP = range(5)
NOALLOC_SCRATCH_BYTES = 16 << 20          # DSA_NOALLOC_SCRATCH_BYTES of include/dsa.h

# name -> (restype, argtypes); the order follows include/dsa.h
SIGNATURES = {
    "dsa_status_str": (c_char_p, [c_int]),
    "dsa_last_error": (c_char_p, []),
    "dsa_abi_version": (c_int, []),
    "dsa_index_scores": (c_int, [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                 c_int, c_int, c_int, c_int, c_int, c_int, c_int64, c_void_p]),
    "dsa_topk_workspace_size": (c_size_t, [c_int, c_int, c_int64, c_int]),
    "dsa_topk": (c_int, [c_void_p, c_void_p, c_int, c_int, c_int64, c_int, c_void_p,
                         c_void_p, c_size_t, c_void_p]),
    "dsa_sparse_attn_workspace_size": (c_size_t, [c_int, c_int, c_int, c_int, c_int, c_int, c_int]),
    "dsa_sparse_attn": (c_int, [c_void_p, c_void_p, c_void_p, c_int64, c_int64, c_int64,
                                c_void_p, c_void_p, c_int, c_int, c_int, c_int, c_int, c_int,
                                c_int, c_int, c_int, c_int, c_float, c_void_p, c_void_p,
                                c_void_p, c_size_t, c_void_p]),
    "dsa_sparse_attn_noalloc": (c_int, [c_void_p, c_void_p, c_void_p, c_int64, c_int64, c_int64,
                                        c_void_p, c_void_p, c_int, c_int, c_int, c_int, c_int, c_int,
                                        c_int, c_int, c_int, c_int, c_float, c_void_p, c_void_p,
                                        c_void_p]),
    "spec_verify_workspace_size": (c_size_t, [c_int, c_int, c_int]),
    "spec_verify": (c_int, [c_void_p, c_void_p, c_void_p, c_int, c_int, c_int, c_void_p,
                            c_uint64, c_uint64, c_void_p, c_void_p, c_void_p, c_void_p,
                            c_size_t, c_void_p]),
    "spec_verify_greedy_workspace_size": (c_size_t, [c_int, c_int, c_int]),
    "spec_verify_greedy": (c_int, [c_void_p, c_void_p, c_int, c_int, c_int, c_void_p, c_void_p, c_void_p,
                                   c_size_t, c_void_p]),
}

_lib = None


class DSAError(RuntimeError):
    def __init__(self, fn, status, message):
        super().__init__(f"{fn} failed with status {status}: {message}")
        self.status = status


def load(path: str = LIB_PATH):
    """Returns the loaded library (cached).  Raises if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(
            f"libdsa.so not found at {path}; build it first "
            "(python dsa_sparse_attention_lightning_amd/build.py or __graft_entry__.build())")
    lib = ctypes.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def check(fn_name: str, status: int):
    if status != DSA_OK:
        lib = load()
        raise DSAError(fn_name, status, lib.dsa_last_error().decode())
