"""ctypes loader for libswattn.so (the HIP kernels behind the C ABI of
include/swattn.h).  Loading fails loudly: there is no fallback path."""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libswattn.so")

ATTN_OK = 0
ATTN_ERR_INVALID_ARG = 1
ATTN_ERR_UNSUPPORTED = 2
ATTN_ERR_WORKSPACE = 3
ATTN_ERR_HIP = 4

# every symbol include/swattn.h declares
EXPORTS = (
    "attn_status_string", "attn_version", "attn_layer_windows", "attn_visible_pairs",
    "attn_band_tiles", "attn_fwd_workspace_bytes", "attn_fwd", "attn_bwd_workspace_bytes",
    "attn_bwd", "attn_fwd_gqa_workspace_bytes", "attn_fwd_gqa", "attn_bwd_gqa_workspace_bytes",
    "attn_bwd_gqa", "attn_fwd_rope_workspace_bytes", "attn_fwd_rope", "attn_bwd_rope_workspace_bytes",
    "attn_bwd_rope", "attn_fwd_ve_workspace_bytes", "attn_fwd_ve", "attn_bwd_ve_workspace_bytes",
    "attn_bwd_ve", "attn_bwd_gqa_reuse", "attn_bwd_rope_reuse", "attn_bwd_ve_reuse", "attn_profile_enable", "attn_profile_enable_mask", "attn_profile_read", "attn_kernel_name",
    "attn_device_info", "attn_fwd_noalloc_max_bytes", "attn_fwd_noalloc",
)


class SwattnError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} ({status})")


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with `python -m sliding_window_causal_qk_amd.build` "
            "(the HIP library is the only implementation; there is no fallback)")
    L = ctypes.CDLL(LIB_PATH)
    c_int, c_size, c_vp, c_float = ctypes.c_int, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_float
    P_int = ctypes.POINTER(ctypes.c_int)

    L.attn_status_string.argtypes = [c_int]
    L.attn_status_string.restype = ctypes.c_char_p
    L.attn_version.argtypes = []
    L.attn_version.restype = c_int
    L.attn_layer_windows.argtypes = [ctypes.c_char_p, c_int, c_int, P_int]
    L.attn_layer_windows.restype = c_int
    L.attn_visible_pairs.argtypes = [c_int, c_int]
    L.attn_visible_pairs.restype = ctypes.c_longlong
    L.attn_band_tiles.argtypes = [c_int, c_int, c_int, c_int, c_int, P_int, P_int, P_int, P_int]
    L.attn_band_tiles.restype = c_int
    for f in (L.attn_fwd_workspace_bytes, L.attn_bwd_workspace_bytes):
        f.argtypes = [c_int, c_int, c_int, c_int]
        f.restype = c_size
    L.attn_fwd.argtypes = [c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_size,
                           c_int, c_int, c_int, c_int, c_int, c_int, c_float, c_vp]
    L.attn_fwd.restype = c_int
    L.attn_bwd.argtypes = [c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_size,
                           c_int, c_int, c_int, c_int, c_int, c_int, c_float, c_vp]
    L.attn_bwd.restype = c_int
    for f in (L.attn_fwd_gqa_workspace_bytes, L.attn_bwd_gqa_workspace_bytes):
        f.argtypes = [c_int, c_int, c_int, c_int, c_int]
        f.restype = c_size
    L.attn_fwd_gqa.argtypes = [c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_size,
                               c_int, c_int, c_int, c_int, c_int, c_int, c_int, c_float, c_vp]
    L.attn_fwd_gqa.restype = c_int
    L.attn_bwd_gqa.argtypes = [c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_size,
                               c_int, c_int, c_int, c_int, c_int, c_int, c_int, c_float, c_vp]
    L.attn_bwd_gqa.restype = c_int
    for f in (L.attn_fwd_rope_workspace_bytes, L.attn_bwd_rope_workspace_bytes):
        f.argtypes = [c_int, c_int, c_int, c_int, c_int]
        f.restype = c_size
    L.attn_fwd_rope.argtypes = [c_vp] * 7 + [c_vp, c_size] + [c_int] * 7 + [c_float, c_vp]
    L.attn_fwd_rope.restype = c_int
    L.attn_bwd_rope.argtypes = [c_vp] * 11 + [c_vp, c_size] + [c_int] * 7 + [c_float, c_vp]
    L.attn_bwd_rope.restype = c_int
    for f in (L.attn_fwd_ve_workspace_bytes, L.attn_bwd_ve_workspace_bytes):
        f.argtypes = [c_int, c_int, c_int, c_int, c_int]
        f.restype = c_size
    L.attn_fwd_ve.argtypes = ([c_vp] * 5 + [c_int] + [c_vp] * 5 + [c_vp, c_size] + [c_int] * 7
                              + [c_float, c_vp])
    L.attn_fwd_ve.restype = c_int
    L.attn_bwd_ve.argtypes = ([c_vp] * 5 + [c_int] + [c_vp] * 12 + [c_vp, c_size] + [c_int] * 7
                              + [c_float, c_vp])
    L.attn_bwd_ve.restype = c_int
    L.attn_bwd_gqa_reuse.argtypes = [c_vp] * 10 + [c_size, c_vp, c_size] + [c_int] * 7 + [c_float, c_vp]
    L.attn_bwd_gqa_reuse.restype = c_int
    L.attn_bwd_rope_reuse.argtypes = [c_vp] * 12 + [c_size, c_vp, c_size] + [c_int] * 7 + [c_float, c_vp]
    L.attn_bwd_rope_reuse.restype = c_int
    L.attn_bwd_ve_reuse.argtypes = ([c_vp] * 5 + [c_int] + [c_vp] * 13 + [c_size, c_vp, c_size] + [c_int] * 7
                                    + [c_float, c_vp])
    L.attn_bwd_ve_reuse.restype = c_int
    L.attn_profile_enable.argtypes = [c_int]
    L.attn_profile_enable.restype = c_int
    L.attn_profile_enable_mask.argtypes = [ctypes.c_uint]
    L.attn_profile_enable_mask.restype = c_int
    L.attn_profile_read.argtypes = [c_int, ctypes.POINTER(ctypes.c_double),
                                    ctypes.POINTER(ctypes.c_longlong)]
    L.attn_profile_read.restype = c_int
    L.attn_kernel_name.argtypes = [c_int]
    L.attn_kernel_name.restype = ctypes.c_char_p
    L.attn_device_info.argtypes = [c_int, P_int, P_int]
    L.attn_device_info.restype = c_int
    L.attn_fwd_noalloc_max_bytes.argtypes = []
    L.attn_fwd_noalloc_max_bytes.restype = c_size
    L.attn_fwd_noalloc.argtypes = [c_vp] * 5 + [c_int] * 6 + [c_float, c_vp]
    L.attn_fwd_noalloc.restype = c_int
    _lib = L
    return L


def status_string(status: int) -> str:
    return lib().attn_status_string(int(status)).decode()


def check(status: int, where: str) -> None:
    if status != ATTN_OK:
        raise SwattnError(status, where)
