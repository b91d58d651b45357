"""ctypes declarations of libtv.so (the C ABI in include/tv.h)."""
from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libtv.so")

TV_OK = 0
TV_ERR_INVALID_ARG = 1
TV_ERR_BAD_TREE = 2
TV_ERR_CAPACITY = 3
TV_ERR_UNSUPPORTED = 4
TV_ERR_HIP = 5
TV_ERR_BAD_PAGE = 6
TV_ERR_SCRATCH = 7

TV_F32 = 0
TV_BF16 = 1
TV_MAX_NODES = 64
TV_MAX_PAGES_PER_SEQ = 256
PAGE = 64

# every function the header declares, with (restype, argtypes)
_P = ctypes.c_void_p
_I = ctypes.c_int32


class TvAttnArgs(ctypes.Structure):
    """Mirror of tv_attn_args."""
    _fields_ = [
        ("q", _P), ("k_new", _P), ("v_new", _P), ("k_cache", _P), ("v_cache", _P),
        ("prefix_len", _P), ("n_nodes", _P), ("anc", _P), ("depth", _P), ("err", _P),
        ("out", _P), ("workspace", _P), ("workspace_bytes", ctypes.c_size_t),
        ("B", _I), ("n_max", _I), ("Hq", _I), ("Hkv", _I), ("D", _I), ("cap", _I),
        ("dtype", _I), ("rope_theta", ctypes.c_float), ("softmax_scale", ctypes.c_float),
    ]


class TvPagedKv(ctypes.Structure):
    """Mirror of tv_paged_kv."""
    _fields_ = [("block_table", _P), ("max_pages", _I), ("num_pages", _I)]


SIGNATURES = {
    "tv_status_string": (ctypes.c_char_p, [_I]),
    "tv_version": (ctypes.c_char_p, []),
    "tv_build_tree": (_I, [_P, _P, _I, _I, _P, _P, _P, _P]),
    "tv_tree_attention_workspace_size": (ctypes.c_size_t, [ctypes.POINTER(TvAttnArgs)]),
    "tv_tree_attention": (_I, [ctypes.POINTER(TvAttnArgs), _P]),
    "tv_tree_attention_noalloc": (_I, [ctypes.POINTER(TvAttnArgs), _P]),
    "tv_tree_attention_from_parents": (_I, [ctypes.POINTER(TvAttnArgs), _P, _P, _P, _P]),
    "tv_tree_attention_paged": (_I, [ctypes.POINTER(TvAttnArgs), ctypes.POINTER(TvPagedKv), _P]),
    "tv_tree_attention_paged_from_parents": (_I, [ctypes.POINTER(TvAttnArgs), ctypes.POINTER(TvPagedKv), _P, _P, _P,
                                                  _P]),
    "tv_accept": (_I, [_P, _P, _P, _P, _P, _P, _P, _I, _I, _P, _P, _P, _P, _P]),
    "tv_eagle2_tree": (_I, [_P, _P, _P, _I, _I, _I, _I, _I, _P, _P, _P, _P, _P]),
    "tv_speculative_sample_workspace_size": (ctypes.c_size_t, [_I, _I]),
    "tv_speculative_sample": (_I, [_P, _P, _I, _I, _P, _P, _P, _I, _I, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]),
    "tv_accept_typical": (_I, [_P, _I, _I, _P, _P, _P, _P, _P, _P, _I, _I, ctypes.c_float,
                               ctypes.c_float, _P, _P, _P, _P, _P, _P, _P, _P]),
    "tv_commit": (_I, [_P, _P, _I, _I, _I, _I, _I, _P, _P, _P, _I, _P, _P]),
    "tv_accept_commit": (_I, [_P, _P, _P, _P, _P, _P, _P, _I, _I, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _P, _P,
                              _P]),
    "tv_commit_paged": (_I, [_P, _P, ctypes.POINTER(TvPagedKv), _I, _I, _I, _I, _P, _P, _P, _I, _P, _P]),
    "tv_accept_commit_paged": (_I, [_P, _P, _P, _P, _P, _P, _P, _I, _I, _P, _P, _P, _P, _P, _P,
                                    ctypes.POINTER(TvPagedKv), _I, _I, _I, _P, _P, _P]),
    "tv_v_cache_layout": (_I, [_P, _P, ctypes.c_int64, _I, _I, _I, _I, _P]),
}

_lib = None


def load() -> ctypes.CDLL:
    """Loads libtv.so from the package directory; raises if it is not built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with `python -m tree_attention_verification_tv_amd.build` "
            "(or __graft_entry__.build()); there is no fallback implementation")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


class TvError(RuntimeError):
    def __init__(self, fn: str, status: int):
        msg = load().tv_status_string(status).decode()
        super().__init__(f"{fn} returned {status} ({msg})")
        self.status = status


def check(fn: str, status: int) -> None:
    if status != TV_OK:
        raise TvError(fn, status)
