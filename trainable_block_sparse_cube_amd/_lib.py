"""ctypes view of libvsa.so: one Python callable per C entry point of
include/vsa.h, with the same names and argument order.  Nothing here
computes; it only loads the library and declares the C signatures."""
from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libvsa.so")

VSA_OK, VSA_ERR_INVALID_ARG, VSA_ERR_UNSUPPORTED, VSA_ERR_WORKSPACE, VSA_ERR_HIP = range(5)
VSA_F32, VSA_BF16 = 0, 1

_p = ctypes.c_void_p
_i = ctypes.c_int
_i64 = ctypes.c_int64
_sz = ctypes.c_size_t
_f = ctypes.c_float

# name -> (restype, argtypes); mirrors include/vsa.h
SIGNATURES = {
    "vsa_status_string": (ctypes.c_char_p, [_i]),
    "vsa_forward_workspace_bytes": (_sz, [_i] * 7),
    "vsa_backward_workspace_bytes": (_sz, [_i] * 7 + [_i64]),
    "vsa_saved_bytes": (_sz, [_i] * 7),
    "vsa_forward": (_i, [_p] * 5 + [_i] * 8 + [_p, _p, _p, _p, _sz, _p]),
    "vsa_forward_noalloc": (_i, [_p] * 5 + [_i] * 8 + [_p, _p, _p, _p]),
    "block_sparse_attn_varlen": (_i, [_p] * 5 + [_i] * 6 + [_p, _p, _i64, _i, _p, _p, _p, _sz, _p]),
    "vsa_backward": (_i, [_p] * 8 + [_i] * 8 + [_p] * 5 + [_p, _sz, _p]),
    "block_sparse_attn_varlen_backward": (
        _i, [_p] * 8 + [_i64, _p] + [_i] * 7 + [_p] * 5 + [_p, _sz, _p]),
    "vsa_cube_permute_pool": (_i, [_p] * 3 + [_i] * 7 + [_p] * 6 + [_p]),
    "vsa_coarse_topk": (_i, [_p] * 3 + [_i] * 6 + [_p] * 3 + [_p]),
    "vsa_fine_forward": (_i, [_p] * 6 + [_i] * 6 + [_p, _p, _i64, _i, _i, _p, _p, _p, _p, _p]),
    "vsa_fine_order": (_i, [_p, _p, _i64, _i, _i, _i, _i, _p, _p]),
    "vsa_validate_lists": (_i, [_p, _p, _i64, _i, _i, _i, _p, _p]),
    "vsa_forward_mass_workspace_bytes": (_sz, [_i] * 8),
    "vsa_forward_mass": (_i, [_p] * 5 + [_i] * 6 + [_f, _i, _i, _i] + [_p] * 5 + [_sz, _p]),
    "vsa_coarse_select_mass": (_i, [_p] * 3 + [_i] * 4 + [_f, _i, _i, _i] + [_p] * 4 + [_p]),
    "vsa_pack_lists": (_i, [_p, _p, _i, _i, _p, _p, _p]),
    "vsa_cube_max_pool": (_i, [_p] * 3 + [_i] * 7 + [_p] * 3 + [_p]),
}

_lib = None


def load():
    """Load libvsa.so once; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build the HIP library first "
                "(python -m trainable_block_sparse_cube_amd.build)")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


class VSAError(RuntimeError):
    def __init__(self, fn, status):
        self.status = status
        msg = load().vsa_status_string(status).decode()
        super().__init__(f"{fn} failed with status {status} ({msg})")


def check(fn_name, status):
    if status != VSA_OK:
        raise VSAError(fn_name, status)
