"""ctypes loader for liblongstraw.so: declarations mirror include/longstraw.h one for one."""
from __future__ import annotations

import ctypes as C
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "liblongstraw.so")

LS_OK = 0
LS_ERR_INVALID = -1
LS_ERR_UNSUPPORTED = -2
LS_ERR_WORKSPACE = -3
LS_ERR_HIP = -4
LS_DTYPE_F32 = 0
LS_DTYPE_BF16 = 1

ERROR_NAMES = {LS_ERR_INVALID: "LS_ERR_INVALID", LS_ERR_UNSUPPORTED: "LS_ERR_UNSUPPORTED",
               LS_ERR_WORKSPACE: "LS_ERR_WORKSPACE", LS_ERR_HIP: "LS_ERR_HIP"}


class LongStrawError(RuntimeError):
    """A non-zero return code of the C library, with its ls_last_error() message."""

    def __init__(self, code: int, message: str):
        self.code = code
        super().__init__(f"{ERROR_NAMES.get(code, code)}: {message}")


class ls_prefix_t(C.Structure):
    _fields_ = [
        ("hq", C.c_int), ("hkv", C.c_int), ("d", C.c_int), ("page_size", C.c_int),
        ("dtype", C.c_int), ("n_shards", C.c_int),
        ("prefix_len", C.c_int64), ("n_phys_pages", C.c_int64),
        ("page_table", C.c_void_p), ("k_pages", C.c_void_p), ("v_pages", C.c_void_p),
        ("shard_page_bounds", C.POINTER(C.c_int64)),
        ("softmax_scale", C.c_float),
    ]


class ls_kernel_stat_t(C.Structure):
    _fields_ = [("name", C.c_char * 48), ("launches", C.c_int64), ("total_ms", C.c_double)]


_P = C.c_void_p
_I64 = C.c_int64
_I = C.c_int
_SIG = {
    "ls_version": (_I, []),
    "ls_last_error": (C.c_char_p, []),
    "ls_capture_pages": (_I, [_P, _P, _I, _I64, _I64, _P, _I64, _P, _P, _I, _I64, _I, _I, _I, _P]),
    "ls_gather_pages": (_I, [_P, _I, _P, _I64, _I64, _I64, _I64, _I, _I, _I, _P, _P]),
    "ls_fwd_workspace_bytes": (C.c_size_t, [C.POINTER(ls_prefix_t), _I64]),
    "ls_bwd_workspace_bytes": (C.c_size_t, [C.POINTER(ls_prefix_t), _I64]),
    "ls_bwd_ds_workspace_bytes": (C.c_size_t, [C.POINTER(ls_prefix_t), _I64, _I64]),
    "ls_bwd_ds_chunk_workspace_bytes": (C.c_size_t, [C.POINTER(ls_prefix_t), _I64, _I64, _I, _I]),
    "ls_check_page_table": (_I, [_P, _I64, _I64]),
    "ls_replay_fwd": (_I, [C.POINTER(ls_prefix_t), _P, _I64, _I64, _P, _P, _I64, _P, _P, _P, C.c_size_t, _P]),
    "ls_replay_fwd_noalloc": (_I, [C.POINTER(ls_prefix_t), _P, _I64, _I64, _P, _P, _I64, _P, _P, _P]),
    "ls_score_workspace_bytes": (C.c_size_t, [C.POINTER(ls_prefix_t), _I64, _I64]),
    "ls_score_fwd": (_I, [C.POINTER(ls_prefix_t), _I64, _P, _I64, _P, _P, _P, _P, _P, C.c_size_t, _P]),
    "ls_replay_bwd": (_I, [C.POINTER(ls_prefix_t), _P, _I64, _I64, _P, _P, _I64, _P, _P, _P, _P, _P, _P, _I,
                           _P, _P, _P, _P, C.c_size_t, _P]),
    "ls_fwd_dq_workspace_bytes": (C.c_size_t, [C.POINTER(ls_prefix_t), _I64]),
    "ls_replay_fwd_dq": (_I, [C.POINTER(ls_prefix_t), _P, _I64, _I64, _P, _P, _I64, _P, _P, _P, _P, _P, C.c_size_t,
                              _P]),
    "ls_lse_merge": (_I, [_I, _I64, _I, _P, _P, _P, _I, _P, _P]),
    "ls_lse_merge_bf16num": (_I, [_I, _I64, _I, _P, _P, _P, _I, _P, _P]),
    "ls_debug_owner_slots": (C.c_size_t, [C.POINTER(ls_prefix_t), _I64, _I64]),
    "ls_debug_set_owner_counts": (_I, [_P, C.c_size_t]),
    "ls_profile_begin": (_I, []),
    "ls_profile_end": (_I, [C.POINTER(ls_kernel_stat_t), _I, C.POINTER(_I)]),
}

_lib = None


def lib():
    """The loaded library.  Raises if liblongstraw.so has not been built: there is no
    fallback implementation."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing; build it with `python -m suffix_attention_amd.build`")
        h = C.CDLL(LIB_PATH)
        for name, (res, args) in _SIG.items():
            fn = getattr(h, name)
            fn.restype = res
            fn.argtypes = args
        _lib = h
    return _lib


def check(rc: int) -> None:
    if rc != LS_OK:
        raise LongStrawError(rc, lib().ls_last_error().decode(errors="replace"))
