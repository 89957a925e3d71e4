"""ctypes view of the C ABI in include/lora.h (argument marshalling only).

Loads rank_specialized_amd/librank_specialized.so.  There is no fallback:
if the library is missing, every entry point raises.
"""
from __future__ import annotations

import ctypes as C
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "librank_specialized.so")

LORA_OK = 0
LORA_ERR_INVALID_ARG = 1
LORA_ERR_UNSUPPORTED = 2
LORA_ERR_HIP = 3
LORA_DTYPE_F32 = 0
LORA_DTYPE_BF16 = 1
LORA_MAX_RANK = 64
LORA_SEGMENT_MAX_T = 16384
LORA_SEGMENT_MAX_N = 16382


class lora_store(C.Structure):
    _fields_ = [
        ("n", C.c_int32), ("d_in", C.c_int32), ("d_out", C.c_int32), ("dtype", C.c_int32),
        ("r_max", C.c_int32), ("R", C.c_int32), ("pad_to", C.c_int32), ("reserved", C.c_int32),
        ("A_pack", C.c_void_p), ("B_pack", C.c_void_p), ("row_off", C.c_void_p),
        ("rank", C.c_void_p), ("scale", C.c_void_p),
    ]


class lora_jd_store(C.Structure):
    _fields_ = [
        ("basis", lora_store), ("n_adapters", C.c_int32), ("r", C.c_int32), ("diag", C.c_int32),
        ("reserved", C.c_int32), ("cluster_of", C.c_void_p), ("sigma", C.c_void_p), ("scale", C.c_void_p),
    ]


LORA_MAX_SLICES = 4
LORA_NOALLOC_SCRATCH_BYTES = 32 << 20


class lora_multi_store(C.Structure):
    _fields_ = [
        ("n_slices", C.c_int32), ("reserved", C.c_int32), ("stacked", lora_store),
        ("slice", lora_store * LORA_MAX_SLICES), ("hoff", C.c_void_p),
    ]


# name -> (restype, argtypes); mirrors include/lora.h
P = C.c_void_p
I = C.c_int
I64 = C.c_int64
SZ = C.c_size_t
SIGNATURES = {
    "lora_status_string": (C.c_char_p, [I]),
    "lora_last_hip_error": (I, []),
    "lora_abi_version": (I, []),
    "lora_store_bytes": (I, [I, I, I, I, P, I, C.POINTER(SZ), C.POINTER(SZ), C.POINTER(SZ)]),
    "lora_pack_retained": (I, [C.POINTER(lora_store), I, I, I, I, P, P, P, P, P, P, P, I, P]),
    "lora_segment": (I, [P, I, I, P, P, P, P]),
    "lora_plan_bytes": (SZ, [I, I]),
    "lora_group": (I, [P, I, I, P, P, P, SZ, P, P]),
    "lora_workspace_bytes": (SZ, [C.POINTER(lora_store), I]),
    "lora_shrink": (I, [C.POINTER(lora_store), P, I64, I, P, P, P, I64, P, SZ, P]),
    "lora_expand": (I, [C.POINTER(lora_store), P, I64, I, P, P, P, I64, P, SZ, P]),
    "lora_apply_batched": (I, [C.POINTER(lora_store), P, I64, P, I64, I, P, P, P, P, SZ, P]),
    "lora_apply_batched_phases": (I, [C.POINTER(lora_store), P, I64, P, I64, I, P, P, P, P, SZ, P, I]),
    "lora_apply_batched_noalloc": (I, [C.POINTER(lora_store), P, I64, P, I64, I, P, P, P, P]),
    "lora_apply_planned": (I, [C.POINTER(lora_store), P, I64, P, I64, I, P, SZ, P, SZ, P]),
    "lora_apply_planned_phases": (I, [C.POINTER(lora_store), P, I64, P, I64, I, P, SZ, P, SZ, P, I]),
    "lora_apply_launches": (I, [C.POINTER(lora_store), I, I]),
    "lora_apply_base_fused": (I, [C.POINTER(lora_store), P, I64, P, I64, P, I64, I, P, P, SZ, P]),
    "lora_jd_workspace_bytes": (SZ, [C.POINTER(lora_jd_store), I]),
    "lora_jd_apply": (I, [C.POINTER(lora_jd_store), P, I64, P, I64, I, P, P, SZ, P]),
    "lora_ranks_uniform": (I, [I, P, C.c_double, I, P]),
    "lora_ranks_spectral": (I, [I, P, P, P, I, I64, P]),
    "lora_rsvd_workspace_bytes": (SZ, [I, I, I]),
    "lora_rsvd_factor": (I, [I, I, I, I, I, P, P, P, P, P, SZ, P]),
    "lora_rsvd_write": (I, [C.POINTER(lora_store), I, P, P, P, SZ, P]),
    "lora_rsvd_factor_phases": (I, [I, I, I, I, I, P, P, P, P, P, SZ, P, I]),
    "lora_multi_bytes": (I, [I, P, C.POINTER(SZ), C.POINTER(SZ), C.POINTER(SZ)]),
    "lora_pack_multi": (I, [C.POINTER(lora_multi_store), I, P, P, P, P, P]),
    "lora_multi_workspace_bytes": (SZ, [C.POINTER(lora_multi_store), I]),
    "lora_apply_multi": (I, [C.POINTER(lora_multi_store), P, I64, P, P, I, P, P, P, P, SZ, P]),
    "lora_apply_multi_planned": (I, [C.POINTER(lora_multi_store), P, I64, P, P, I, P, SZ, P, SZ, P]),
}

_lib = None


class LoraError(RuntimeError):
    def __init__(self, fn: str, status: int, hip_error: int = 0):
        self.status = status
        self.hip_error = hip_error
        msg = f"{fn} failed: status {status}"
        if _lib is not None:
            msg += f" ({_lib.lora_status_string(status).decode()})"
        if status == LORA_ERR_HIP:
            msg += f", hipError_t {hip_error}"
        super().__init__(msg)


def lib():
    """The loaded library; raises ImportError if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with `python -m rank_specialized_amd.build`")
        L = C.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def check(fn: str, status: int) -> None:
    if status != LORA_OK:
        raise LoraError(fn, status, lib().lora_last_hip_error() if status == LORA_ERR_HIP else 0)
