"""ctypes loader of libvsa.so: declares the C ABI of include/vsa.h.

The library must have been built in-tree (``video_dit_block_amd/build.py``).
There is no fallback: a missing or unloadable library raises.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libvsa.so")

VSA_OK = 0
VSA_ERR_NULL = 1
VSA_ERR_SHAPE = 2
VSA_ERR_UNSUPPORTED = 3
VSA_ERR_RANGE = 4
VSA_ERR_WORKSPACE = 5
VSA_ERR_HIP = 6

VSA_ORDER_ROW_MAJOR = 0
VSA_ORDER_HILBERT = 1

_c_int = ctypes.c_int32
_vp = ctypes.c_void_p
_sz = ctypes.c_size_t

# name -> (restype, argtypes); mirrors include/vsa.h
SIGNATURES = {
    "vsa_abi_version": (_c_int, []),
    "vsa_status_string": (ctypes.c_char_p, [_c_int]),
    "vsa_last_error": (ctypes.c_char_p, []),
    "vsa_num_cubes": (_c_int, [_c_int, _c_int, _c_int]),
    "vsa_vbs_host": (_c_int, [_c_int, _c_int, _c_int, _vp, _c_int]),
    "vsa_tile": (_c_int, [_vp, _vp, _vp, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int, _vp]),
    "vsa_untile": (_c_int, [_vp, _vp, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int, _vp]),
    "vsa_cube_order_host": (_c_int, [_c_int, _c_int, _c_int, _c_int, _vp, _c_int]),
    "vsa_tile_ordered": (_c_int, [_vp, _vp, _vp, _vp, _c_int, _c_int, _c_int, _c_int, _c_int,
                                  _c_int, _vp]),
    "vsa_untile_ordered": (_c_int, [_vp, _vp, _vp, _c_int, _c_int, _c_int, _c_int, _c_int,
                                    _c_int, _vp]),
    "vsa_mask_to_lut": (_c_int, [_vp, _c_int, _c_int, _c_int, _c_int, _c_int, _vp, _vp, _vp,
                                 _vp]),
    "vsa_select_workspace_bytes": (_sz, [_c_int, _c_int, _c_int, _c_int]),
    "vsa_select": (_c_int, [_vp, _vp, _vp, _c_int, _c_int, _c_int, _c_int, _c_int, _vp, _vp,
                            _sz, _vp]),
    "vsa_select_noalloc_max_bytes": (_sz, []),
    "vsa_select_noalloc": (_c_int, [_vp, _vp, _vp, _c_int, _c_int, _c_int, _c_int, _c_int, _vp,
                                    _vp]),
    "vsa_select_cdf": (_c_int, [_vp, _vp, _vp, _c_int, _c_int, _c_int, _c_int, _c_int,
                                ctypes.c_float, ctypes.c_float, _vp, _vp, _vp, _sz, _vp]),
    "vsa_fwd_workspace_bytes": (_sz, [_c_int, _c_int, _c_int, _c_int, _c_int, _c_int]),
    "vsa_fwd_workspace_bytes_ex": (_sz, [_c_int, _c_int, _c_int, _c_int, _c_int, _c_int,
                                         _c_int]),
    "vsa_fwd_splits": (_c_int, [_c_int, _c_int, _c_int, _c_int]),
    "vsa_fwd": (_c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _c_int, _c_int, _c_int, _c_int, _c_int,
                         _c_int, ctypes.c_float, _vp, _sz, _vp]),
    "vsa_fwd_lut": (_c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _c_int, _c_int,
                             _c_int, _c_int, _c_int, _c_int, ctypes.c_float, _vp, _sz, _vp]),
    "vsa_fwd_lut_ex": (_c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _c_int, _c_int,
                                _c_int, _c_int, _c_int, _c_int, ctypes.c_float, _c_int, _vp, _sz,
                                _vp]),
    "vsa_coarse_workspace_bytes": (_sz, [_c_int, _c_int, _c_int, _c_int]),
    "vsa_coarse": (_c_int, [_vp, _vp, _vp, _vp, _c_int, _c_int, _c_int, _c_int, _c_int, _vp,
                            ctypes.c_float, _vp, _vp, _sz, _vp]),
    "vsa_gate_combine": (_c_int, [_vp, _vp, _vp, _vp, _vp, _c_int, _c_int, _c_int, _c_int, _vp]),
    "vsa_validate_topk": (_c_int, [_vp, _c_int, _c_int, _c_int, _c_int, _c_int, _vp, _vp]),
}

_lib = None


class VsaError(RuntimeError):
    def __init__(self, status: int, where: str, message: str):
        super().__init__(f"{where}: {status_name(status)} ({status}): {message}")
        self.status = status


def load() -> ctypes.CDLL:
    """Load libvsa.so once and declare its signatures."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with `python -m video_dit_block_amd.build`")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def status_name(status: int) -> str:
    return load().vsa_status_string(status).decode()


def check(status: int, where: str) -> None:
    if status != VSA_OK:
        raise VsaError(status, where, load().vsa_last_error().decode())
