"""ctypes loader for libqwha.so: the C-ABI declared in include/qwha.h.

The library is loaded after torch so that both share torch's HIP runtime
(same soname). There is no fallback: if the built library is missing the
import of this module raises.
"""
from __future__ import annotations

import ctypes
import os

import torch  # noqa: F401  (loads the HIP runtime the library links against)

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libqwha.so")

c_int32 = ctypes.c_int32
c_int64 = ctypes.c_int64
c_size_t = ctypes.c_size_t
c_void_p = ctypes.c_void_p
c_float = ctypes.c_float
c_double = ctypes.c_double
c_char_p = ctypes.c_char_p

# name -> (restype, argtypes); mirrors include/qwha.h
SIGNATURES = {
    "qwha_status_string": (c_char_p, [c_int32]),
    "qwha_last_error": (c_char_p, []),
    "qwha_version": (c_int32, []),
    "qwha_init_workspace_bytes": (c_size_t, [c_int32, c_int32]),
    "qwha_init_select": (c_int32, [c_void_p, c_int32, c_int32, c_int64, c_int32, c_double,
                                   c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                   c_void_p, c_size_t, c_void_p]),
    "qwha_init_global_workspace_bytes": (c_size_t, [c_int32, c_int32, c_int32]),
    "qwha_init_select_global": (c_int32, [c_void_p, c_int32, c_int32, c_int64, c_int32,
                                          ctypes.c_uint64, c_void_p, c_void_p, c_void_p,
                                          c_void_p, c_void_p, c_void_p, c_size_t, c_void_p]),
    "qwha_hessian": (c_int32, [c_void_p, c_int32, c_int64, c_int32, c_void_p, c_int32, c_void_p]),
    "qwha_init_calibrated_workspace_bytes": (c_size_t, [c_int32, c_int32]),
    "qwha_init_select_calibrated": (c_int32, [c_void_p, c_int32, c_int32, c_void_p, c_double,
                                              c_int64, c_int32, c_double, c_void_p, c_void_p,
                                              c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                              c_void_p, c_size_t, c_void_p]),
    "qwha_refine_workspace_bytes": (c_size_t, [c_void_p, c_int32]),
    "qwha_refine_values": (c_int32, [c_void_p, c_void_p, c_void_p, c_void_p, c_int32, c_int32,
                                     c_int64, c_void_p, c_void_p, c_void_p, c_size_t, c_void_p]),
    "qwha_merge": (c_int32, [c_void_p, c_void_p, c_void_p, c_int32, c_int32, c_int32, c_int32,
                             c_int64, c_void_p, c_void_p, c_void_p, c_float, c_int32, c_void_p,
                             c_void_p]),
    "qwha_layer_fwd_workspace_bytes": (c_size_t, [c_int64, c_int32, c_int32, c_int64]),
    "qwha_layer_fwd": (c_int32, [c_void_p, c_int32, c_int64, c_int32, c_int32, c_void_p,
                                 c_void_p, c_void_p, c_int32, c_int32, c_int64, c_void_p,
                                 c_void_p, c_void_p, c_float, c_void_p, c_void_p, c_size_t,
                                 c_void_p]),
    "qwha_materialize": (c_int32, [c_void_p, c_void_p, c_void_p, c_int32, c_int32, c_int64,
                                   c_float, c_int32, c_void_p, c_int32, c_void_p]),
    "qwha_fwd_workspace_bytes": (c_size_t, [c_int64, c_int32, c_int32, c_int64]),
    "qwha_fwd": (c_int32, [c_void_p, c_int32, c_int64, c_int32, c_int32, c_int64,
                           c_void_p, c_void_p, c_void_p, c_float, c_void_p, c_int32,
                           c_void_p, c_size_t, c_void_p]),
    "qwha_fwd_noalloc": (c_int32, [c_void_p, c_int32, c_int64, c_int32, c_int32, c_int64,
                                   c_void_p, c_void_p, c_void_p, c_float, c_void_p, c_int32,
                                   c_void_p]),
    "qwha_fwd_z": (c_int32, [c_void_p, c_int32, c_int64, c_int32, c_int32, c_int64,
                             c_void_p, c_void_p, c_void_p, c_float, c_void_p, c_int32,
                             c_void_p, c_size_t, c_void_p]),
    "qwha_bwd_dz": (c_int32, [c_void_p, c_void_p, c_int32, c_int64, c_int32, c_int32, c_int64,
                              c_void_p, c_void_p, c_void_p, c_void_p, c_float, c_void_p,
                              c_int32, c_void_p, c_void_p, c_size_t, c_void_p]),
    "qwha_plan_bytes": (c_size_t, [c_int32, c_int32, c_int64]),
    "qwha_plan_build": (c_int32, [c_void_p, c_void_p, c_void_p, c_void_p, c_int32, c_int32,
                                  c_int64, c_int32, c_void_p, c_size_t, c_void_p]),
    "qwha_fwd_plan": (c_int32, [c_void_p, c_void_p, c_int32, c_int64, c_int32, c_int32, c_int64,
                                c_void_p, c_void_p, c_float, c_void_p, c_int32, c_void_p,
                                c_void_p, c_size_t, c_void_p]),
    "qwha_bwd_plan": (c_int32, [c_void_p, c_void_p, c_int32, c_int64, c_int32, c_int32, c_int64,
                                c_void_p, c_void_p, c_float, c_void_p, c_int32, c_void_p,
                                c_int32, c_void_p, c_void_p, c_size_t, c_void_p]),
    "qwha_fwd_save": (c_int32, [c_void_p, c_int32, c_int64, c_int32, c_int32, c_int64,
                                c_void_p, c_void_p, c_void_p, c_float, c_void_p, c_int32,
                                c_void_p, c_void_p, c_size_t, c_void_p]),
    "qwha_bwd_saved": (c_int32, [c_void_p, c_void_p, c_int32, c_int64, c_int32, c_int32,
                                 c_int64, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                 c_float, c_void_p, c_int32, c_void_p, c_void_p, c_size_t,
                                 c_void_p]),
    "qwha_bwd_workspace_bytes": (c_size_t, [c_int64, c_int32, c_int32, c_int64]),
    "qwha_bwd": (c_int32, [c_void_p, c_void_p, c_int32, c_int64, c_int32, c_int32, c_int64,
                           c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_float,
                           c_void_p, c_int32, c_void_p, c_void_p, c_size_t, c_void_p]),
    "qwha_sign_update": (c_int32, [c_void_p, c_void_p, c_int64, c_float, c_void_p]),
    "qwha_fwht": (c_int32, [c_void_p, c_int32, c_void_p, c_int32, c_int64, c_int32, c_float,
                            c_void_p]),
    "qwha_profile_next": (c_int32, [c_int32, c_void_p, c_void_p]),
}


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is not built; run `python quantization_aware_sparse_amd/build.py` "
            "(there is no CPU fallback)")
    lib = ctypes.CDLL(LIB_PATH, mode=ctypes.RTLD_GLOBAL)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


lib = _load()


class QwhaError(RuntimeError):
    def __init__(self, status: int, where: str):
        msg = lib.qwha_last_error().decode()
        kind = lib.qwha_status_string(status).decode()
        super().__init__(f"{where}: {kind} ({status}): {msg}")
        self.status = status


def check(status: int, where: str) -> None:
    if status != 0:
        raise QwhaError(status, where)
