"""ctypes binding of libssd.so (the C ABI in include/ssd.h).

Argument marshalling only: every computation runs in the library's HIP
kernels. PyTorch supplies device memory and the current HIP stream. There is no
fallback: if the library is missing or cannot be loaded, importing this module
raises.
"""
from __future__ import annotations

import ctypes
import os

import torch  # loads the HIP runtime libssd.so binds to (same soname)

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libssd.so")

SSD_F32, SSD_BF16 = 0, 1
SSD_OK = 0
SSD_DISC_EULER, SSD_DISC_ZOH = 0, 1


class SsdOptions(ctypes.Structure):
    """ssd_options of include/ssd.h."""
    _fields_ = [("dt_bias", ctypes.c_void_p), ("dt_softplus", ctypes.c_int),
                ("dt_clamp", ctypes.c_int), ("dt_min", ctypes.c_float),
                ("dt_max", ctypes.c_float), ("discretization", ctypes.c_int)]


class SsdPlan(ctypes.Structure):
    """ssd_plan of include/ssd.h."""
    _fields_ = [("path", ctypes.c_int), ("segments", ctypes.c_int), ("pieces", ctypes.c_int),
                ("block_tokens", ctypes.c_int), ("segment_blocks", ctypes.c_int),
                ("piece_blocks", ctypes.c_int), ("kernel_dstate", ctypes.c_int),
                ("workspace_bytes", ctypes.c_size_t)]


_vp, _i, _sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
_op = ctypes.POINTER(SsdOptions)
_pp = ctypes.POINTER(SsdPlan)

# name -> (restype, argtypes); mirrors include/ssd.h
SIGNATURES = {
    "ssd_strerror": (ctypes.c_char_p, [_i]),
    "ssd_forward_workspace_size": (_sz, [_i] * 8),
    "ssd_forward_plan": (_i, [_i] * 8 + [_vp]),
    "ssd_forward_plan_info": (_i, [_i] * 8 + [_vp, _pp]),
    "ssd_chunk_cb_size": (_sz, [_i] * 5),
    "ssd_chunk_cb": (_i, [_vp, _vp] + [_i] * 6 + [_vp, _vp]),
    "ssd_forward": (_i, [_vp] * 6 + [_i] * 8 + [_vp, _vp, _vp, _vp, _sz, _vp]),
    "ssd_forward_timed": (_i, [_vp] * 6 + [_i] * 8 + [_vp, _vp, _vp, _vp, _sz, _vp, _vp]),
    "ssd_forward_ex": (_i, [_vp] * 6 + [_i] * 8 + [_vp, _vp, _vp, _vp, _sz, _op, _vp, _vp]),
    "ssd_forward_static": (_i, [_vp] * 6 + [_i] * 8 + [_vp, _vp, _vp, _op, _vp]),
    "ssd_backward_workspace_size": (_sz, [_i] * 7),
    "ssd_backward": (_i, [_vp] * 9 + [_i] * 7 + [_vp] * 9 + [_sz, _op, _vp]),
    "ssd_backward_timed": (_i, [_vp] * 9 + [_i] * 7 + [_vp] * 9 + [_sz, _op, _vp, _vp]),
    "ssd_forward_varlen_workspace_size": (_sz, [_i] * 7),
    "ssd_forward_varlen": (_i, [_vp] * 7 + [_i] * 8 + [_vp, _vp, _vp, _sz, _op, _vp]),
    "ssd_step": (_i, [_vp] * 7 + [_i] * 6 + [_vp, _vp]),
    "ssd_step_ex": (_i, [_vp] * 7 + [_i] * 6 + [_vp, _op, _vp]),
    "ssd_chunk_cumsum": (_i, [_vp, _vp] + [_i] * 5 + [_vp, _vp, _op, _vp]),
    "ssd_chunk_state": (_i, [_vp] * 4 + [_i] * 8 + [_vp, _vp]),
    "ssd_state_passing": (_i, [_vp] * 3 + [_i] * 7 + [_vp, _vp, _vp]),
    "ssd_chunk_scan": (_i, [_vp] * 8 + [_i] * 8 + [_vp, _vp]),
}


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is not built; run `python structured_state_space_ssd_amd/build.py` "
            "(there is no fallback implementation)")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


lib = _load()


class SSDError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {lib.ssd_strerror(status).decode()} (status {status})")


def check(status: int, where: str) -> None:
    if status != SSD_OK:
        raise SSDError(status, where)


def dtype_code(t: torch.dtype) -> int:
    if t == torch.float32:
        return SSD_F32
    if t == torch.bfloat16:
        return SSD_BF16
    raise TypeError(f"unsupported dtype {t}: use torch.float32 or torch.bfloat16")


def ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def stream_handle(device=None) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)
