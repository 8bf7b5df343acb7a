"""ctypes declarations of libsgmv's C ABI (include/sgmv.h).  Loading fails loudly when
the library has not been built: there is no fallback implementation."""
from __future__ import annotations

import ctypes
import os

from .build import LIB_PATH, PHASES_LIB_PATH

F16 = 0
BF16 = 1

OK = 0
ERR_NULL = 1
ERR_SHAPE = 2
ERR_ALIGNMENT = 3
ERR_ADAPTER_ID = 4
ERR_UNSUPPORTED = 5
ERR_WORKSPACE = 6
ERR_ALIAS = 7
ERR_HIP = 8
ERR_DEVICE = 9

# flag bits of the workspace's first int32 (SGMV_FLAG_* in include/sgmv.h)
FLAG_WAIT_TIMEOUT = 1
FLAG_ADAPTER_ID = 2
FLAG_SEG_BOUNDS = 4

STATUS_NAMES = {
    OK: "SGMV_OK", ERR_NULL: "SGMV_ERR_NULL", ERR_SHAPE: "SGMV_ERR_SHAPE",
    ERR_ALIGNMENT: "SGMV_ERR_ALIGNMENT", ERR_ADAPTER_ID: "SGMV_ERR_ADAPTER_ID",
    ERR_UNSUPPORTED: "SGMV_ERR_UNSUPPORTED", ERR_WORKSPACE: "SGMV_ERR_WORKSPACE",
    ERR_ALIAS: "SGMV_ERR_ALIAS", ERR_HIP: "SGMV_ERR_HIP", ERR_DEVICE: "SGMV_ERR_DEVICE",
}

# every function the header declares, with its ctypes signature
_p = ctypes.c_void_p
_i32 = ctypes.c_int32
_i64 = ctypes.c_int64
_sz = ctypes.c_size_t
SIGNATURES = {
    "sgmv_abi_version": (ctypes.c_int, []),
    "sgmv_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "sgmv_build_segments": (ctypes.c_int, [_p, _i32, _i32, _p, _p, _p, _p, _p, _p]),
    "sgmv_build_ptr_table": (ctypes.c_int, [_p, _i32, _p, _i32, _p]),
    "sgmv_workspace_bytes": (_sz, [_i32, _i32, _i32]),
    "sgmv_check_workspace": (ctypes.c_int, [_p, _p, _p, _i32]),
    "sgmv_shrink": (ctypes.c_int, [_p, _i32, _p, _p, _i64, _p, _p, _p, _i32, _i32, _i32, _i32,
                                   _i32, _i32, _p, _sz]),
    "sgmv_expand": (ctypes.c_int, [_p, _i32, _p, _i64, _p, _p, _p, _p, _i32, _i32, _i32, _i32,
                                   _i32, _i32, ctypes.c_float]),
    "sgmv_lora_add": (ctypes.c_int, [_p, _i32, _p, _i64, _p, _i64, _p, _p, _p, _p, _i32, _i32,
                                     _i32, _i32, _i32, _i32, _i32, ctypes.c_float, _p, _sz]),
    "sgmv_build_segments_device": (ctypes.c_int, [_p, _p, _i32, _i32, _p, _p, _p, _p]),
    "sgmv_lora_add_pool": (ctypes.c_int, [_p, _i32, _p, _i64, _p, _i64, _p, _i32, _p, _i64, _p,
                                          _i64, _i32, _i32, _i32, _i32, ctypes.c_float, _p, _sz]),
    "sgmv_lora_add_host_ids": (ctypes.c_int, [_p, _i32, _p, _i64, _p, _i64, _p, _i32, _p, _i64,
                                              _p, _i64, _i32, _i32, _i32, _i32, ctypes.c_float,
                                              _p, _sz]),
    "sgmv_lora_add_host_ids_noalloc": (ctypes.c_int, [_p, _i32, _p, _i64, _p, _i64, _p, _i32,
                                                      _p, _i64, _p, _i64, _i32, _i32, _i32,
                                                      _i32, ctypes.c_float]),
}


class RankGroup(ctypes.Structure):
    """sgmv_rank_group (include/sgmv.h)."""
    _fields_ = [("r", _i32), ("row0", _i32), ("n", _i32), ("seg0", _i32), ("starts0", _i32),
                ("n_segments", _i32), ("min_seg_len", _i32), ("max_seg_len", _i32),
                ("scale", ctypes.c_float)]


SIGNATURES["sgmv_slot_cache_create"] = (ctypes.c_int, [_i32, _p])
SIGNATURES["sgmv_slot_cache_destroy"] = (None, [_p])
SIGNATURES["sgmv_slot_cache_map"] = (ctypes.c_int, [_p, _p, _i32, _p, _p, _p, _p])
SIGNATURES["sgmv_slot_cache_lookup"] = (ctypes.c_int, [_p, _i64, _p])
SIGNATURES["sgmv_slot_cache_evict"] = (ctypes.c_int, [_p, _i64])
SIGNATURES["sgmv_upload_adapter"] = (ctypes.c_int, [_p, _p, _i64, _p, _i64, _i32, _i32, _p, _p,
                                                    _i32, _i32, _i32])
SIGNATURES["sgmv_build_segments_ranked"] = (ctypes.c_int, [_p, _i32, _i32, _p, _p, _p, _p, _p, _p])
SIGNATURES["sgmv_lora_add_ranked"] = (ctypes.c_int, [_p, _i32, _p, _i64, _p, _i64, _p, _p, _p, _p,
                                                     _i32, _p, _i32, _i32, _i32, _p, _sz])

_LIB = None
_PATH = LIB_PATH


def use_phase_stamps() -> None:
    """Load the profiling variant (libsgmv_phases.so, built with build --phases) instead of
    libsgmv.so; must be called before the library is first used."""
    global _PATH
    if _LIB is not None and _PATH != PHASES_LIB_PATH:
        raise RuntimeError("libsgmv is already loaded")
    _PATH = PHASES_LIB_PATH


class SgmvError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {STATUS_NAMES.get(status, status)} ({status_string(status)})")


def lib() -> ctypes.CDLL:
    """The loaded libsgmv.so (raises if it was not built)."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(_PATH):
            raise RuntimeError(f"{_PATH} is missing; build it with "
                               "`python -m adapter_gemv_amd.build` (hipcc, gfx950)")
        L = ctypes.CDLL(_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        if _PATH == PHASES_LIB_PATH:
            L.sgmv_phase_stamps_attach.restype = ctypes.c_int64
            L.sgmv_phase_stamps_attach.argtypes = [ctypes.c_void_p, ctypes.c_int64]
        _LIB = L
    return _LIB


def status_string(status: int) -> str:
    return lib().sgmv_status_string(int(status)).decode()


def check(status: int, where: str) -> None:
    if status != OK:
        raise SgmvError(status, where)
