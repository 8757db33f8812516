"""ctypes view of the C interface declared in include/streambp_head.h."""
from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libstreambp_head.so")

OK, ERR_INVALID_ARGUMENT, ERR_UNSUPPORTED, ERR_WORKSPACE_TOO_SMALL, ERR_HIP, ERR_LABEL_RANGE = range(6)
STATUS_NAMES = {0: "OK", 1: "INVALID_ARGUMENT", 2: "UNSUPPORTED", 3: "WORKSPACE_TOO_SMALL", 4: "HIP",
                5: "LABEL_RANGE"}
F32, BF16 = 0, 1
STATIC_SCRATCH_BYTES = 64 << 20  # STREAMBP_STATIC_SCRATCH_BYTES
IGNORE_INDEX = -100

_vp, _i64, _i32, _sz, _dbl = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t, ctypes.c_double
_int = ctypes.c_int

# name -> (restype, argtypes); the order of arguments follows the header.
SIGNATURES = {
    "streambp_head_create": (_int, [ctypes.POINTER(_vp), _i64, _i64, _i64, _int, _int]),
    "streambp_head_destroy": (_int, [_vp]),
    "streambp_head_workspace_bytes": (_sz, [_vp, _i64, _i32]),
    "streambp_head_last_error": (ctypes.c_char_p, [_vp]),
    "streambp_head_version": (ctypes.c_char_p, []),
    "streambp_head_sft": (_int, [_vp, _i64, _vp, _vp, _vp, _vp, _vp, _int, _vp, _vp, _vp, _vp, _sz, _vp]),
    "streambp_head_sft_noalloc": (_int, [_vp, _i64, _vp, _vp, _vp, _vp, _vp, _int, _vp, _vp, _vp, _vp]),
    "streambp_head_grpo": (_int, [_vp, _i64, _vp, _vp, _vp, _vp, _i32, _vp, _vp, _vp, _vp, _int, _vp, _vp, _vp,
                                  _sz, _vp]),
    "streambp_head_ppo": (_int, [_vp, _i64, _vp, _vp, _vp, _vp, _i32, _vp, _vp, _vp, _dbl, _dbl, _vp, _vp, _vp,
                                 _int, _vp, _vp, _vp, _sz, _vp]),
    "streambp_head_dpo_logp": (_int, [_vp, _i64, _vp, _vp, _vp, _vp, _i32, _vp, _vp, _vp, _vp, _sz, _vp]),
    "streambp_head_dpo_bwd": (_int, [_vp, _i64, _vp, _vp, _vp, _vp, _i32, _vp, _vp, _dbl, _vp, _vp, _vp, _int,
                                     _vp, _vp, _vp, _sz, _vp]),
    "streambp_head_suggest_chunk": (_int, [_i64, _i64, _i64, _i32, _int, _sz, ctypes.POINTER(_i64)]),
    "streambp_head_set_timing": (_int, [_vp, _int]),
    "streambp_head_set_row_compaction": (_int, [_vp, _int]),
    "streambp_head_set_tiled_logits": (_int, [_vp, _int]),
    "streambp_head_kernel_kinds": (_int, []),
    "streambp_head_kernel_name": (ctypes.c_char_p, [_int]),
    "streambp_head_kernel_times": (_int, [_vp, _int, ctypes.POINTER(_dbl), ctypes.POINTER(_i64)]),
    "streambp_head_mfma_probe": (_int, [_i64, _i32, _int, ctypes.POINTER(_dbl), _vp]),
}


class LibraryMissing(ImportError):
    pass


_lib = None


def load() -> ctypes.CDLL:
    """Load the HIP library (after torch, so that both share one HIP runtime).
    There is no fallback: without the built library every call fails here."""
    global _lib
    if _lib is not None:
        return _lib
    import torch  # noqa: F401  (loads torch's libamdhip64 first)
    if not os.path.exists(LIB_PATH):
        raise LibraryMissing(f"{LIB_PATH} is not built; run `python -m loss_head_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib
