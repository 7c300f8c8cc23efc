"""ctypes declarations for libdkv.so (the C ABI in include/dkv.h).

Loading fails loudly if the library has not been built: there is no fallback.
"""
from __future__ import annotations

import ctypes as C
import os

HERE = os.path.dirname(os.path.abspath(__file__))
# DKV_LIB names another build of the same library (e.g. the host-sanitizer
# build); the binding still raises if that file is missing.
LIB_PATH = os.environ.get("DKV_LIB") or os.path.join(HERE, "libdkv.so")

DKV_OK = 0
DKV_ERR_INVALID = 1
DKV_ERR_UNSUPPORTED = 2
DKV_ERR_NOMEM = 3
DKV_ERR_HIP = 4
DKV_HOST_COHERENT = 0
DKV_HOST_NONCOHERENT = 1

STATUS_NAMES = {0: "DKV_OK", 1: "DKV_ERR_INVALID", 2: "DKV_ERR_UNSUPPORTED", 3: "DKV_ERR_NOMEM",
                4: "DKV_ERR_HIP"}


class DkvError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


class KvDesc(C.Structure):
    _fields_ = [
        ("num_kv_heads", C.c_int32),
        ("head_dim", C.c_int32),
        ("page_size", C.c_int32),
        ("max_pages", C.c_int32),
        ("host_stride", C.c_int64),
        ("dev_stride", C.c_int64),
        ("host_rows", C.c_int64),
        ("dev_rows", C.c_int64),
        ("host_k", C.c_void_p),
        ("host_v", C.c_void_p),
        ("dev_k", C.c_void_p),
        ("dev_v", C.c_void_p),
        ("page_table", C.c_void_p),
        ("page_table_host", C.c_void_p),
    ]


class PlanInfo(C.Structure):
    _fields_ = [
        ("workspace_bytes", C.c_int64),
        ("num_splits", C.c_int32),
        ("host_items", C.c_int32),
        ("dev_items", C.c_int32),
        ("host_wgs", C.c_int32),
        ("dev_wgs", C.c_int32),
        ("host_chunk", C.c_int32),
        ("dev_chunk", C.c_int32),
        ("host_bytes", C.c_int64),
        ("dev_bytes", C.c_int64),
        ("staged_bytes", C.c_int64),
    ]

    def as_dict(self):
        return {k: getattr(self, k) for k, _ in self._fields_}


class Tuning(C.Structure):
    _fields_ = [
        ("num_cus", C.c_int32),
        ("host_wgs", C.c_int32),
        ("dev_wgs", C.c_int32),
        ("host_chunk", C.c_int32),
        ("dev_chunk", C.c_int32),
        ("stage_max_mib", C.c_int32),
        ("host_bw_gbs", C.c_double),
        ("dev_bw_gbs", C.c_double),
        ("writer_wgs", C.c_int32),
        ("reserved", C.c_int32),
    ]


class BwResult(C.Structure):
    _fields_ = [("read_gbs", C.c_double), ("read_ms", C.c_double), ("dma_gbs", C.c_double)]


class PagerStats(C.Structure):
    _fields_ = [
        ("free_host_pages", C.c_int32),
        ("free_dev_pages", C.c_int32),
        ("used_host_pages", C.c_int32),
        ("used_dev_pages", C.c_int32),
        ("spilled_pages", C.c_int32),
        ("reserved", C.c_int32),
    ]

    def as_dict(self):
        return {k: getattr(self, k) for k, _ in self._fields_ if k != "reserved"}


P = C.c_void_p
I32 = C.c_int32
I64 = C.c_int64
F32 = C.c_float
F64 = C.c_double
SZ = C.c_size_t
PI32 = C.POINTER(C.c_int32)

# name -> (restype, argtypes); the header is the source of truth and a CPU
# test checks that every function declared there is listed and exported.
SIGNATURES = {
    "dkv_last_error": (C.c_char_p, []),
    "dkv_version": (I32, []),
    "dkv_split_point": (I32, [F64, I64, C.POINTER(I64)]),
    "dkv_append_workspace_bytes": (SZ, [I32, I32, I32]),
    "dkv_project_rope_append": (I32, [C.POINTER(KvDesc), I32, P, F64, I32, P, P, P, I32, P, P, P, P,
                                      F64, P, SZ, P]),
    "dkv_decode_plan": (I32, [C.POINTER(KvDesc), I32, I32, P, F64, C.POINTER(PlanInfo)]),
    "dkv_plan_inspect": (I32, [C.POINTER(KvDesc), I32, I32, P, F64, I32, P, I32, P, I32, P,
                               C.POINTER(PlanInfo)]),
    "dkv_prefill_plan_inspect": (I32, [C.POINTER(KvDesc), I32, I32, P, P, P, F64, I32, I32, P, I32, P, I32, P,
                                       I32, P, I32, C.POINTER(PlanInfo)]),
    "dkv_prefill_fused_plan": (I32, [C.POINTER(KvDesc), I32, I32, P, P, P, F64, I32, C.POINTER(PlanInfo)]),
    "dkv_prefill_fused": (I32, [C.POINTER(KvDesc), I32, I32, P, P, P, P, F64, F32, F64, P, I32, P, P, P, P, P, SZ,
                                P, P, P]),
    "dkv_decode_attn_split": (I32, [C.POINTER(KvDesc), I32, I32, P, P, P, F64, F32, F64, P, SZ, P, P,
                                    P, I32, P]),
    "dkv_decode_step_plan": (I32, [C.POINTER(KvDesc), I32, I32, F64, I32, C.POINTER(PlanInfo)]),
    "dkv_decode_step": (I32, [C.POINTER(KvDesc), I32, I32, P, P, P, P, P, I32, P, P, P, P, F64, F32, F64, P, SZ,
                              P, P, P]),
    "dkv_decode_errors": (I32, [C.POINTER(KvDesc), P, I32, C.POINTER(I32)]),
    "dkv_decode_step_static": (I32, [C.POINTER(KvDesc), I32, I32, P, P, P, P, P, I32, P, P, P, P, F64, F32, F64,
                                     P, P, P]),
    "dkv_decode_staged_plan": (I32, [C.POINTER(KvDesc), I32, I64, F64, I32, C.POINTER(PlanInfo)]),
    "dkv_decode_staged": (I32, [C.POINTER(KvDesc), I32, P, P, I64, F64, F32, F64, I32, P, SZ, P, P, P]),
    "dkv_linear_plan": (I32, [I32, I32, I32, F64, C.POINTER(PlanInfo)]),
    "dkv_linear_split": (I32, [P, P, I32, I32, F64, P, I32, P, P, SZ, P]),
    "dkv_linear_plan_inspect": (I32, [I32, I32, F64, I32, P, I32, C.POINTER(PlanInfo)]),
    "dkv_merge_lse": (I32, [P, P, P, I32, I32, I32, P, P, P]),
    "dkv_pager_create": (I32, [I32, I32, I32, I32, I32, F64, C.POINTER(P)]),
    "dkv_pager_destroy": (I32, [P]),
    "dkv_pager_reserve": (I32, [P, I32, I64]),
    "dkv_pager_release": (I32, [P, I32]),
    "dkv_pager_table": (I32, [P, C.POINTER(PI32), C.POINTER(PI32)]),
    "dkv_pager_stats_get": (I32, [P, C.POINTER(PagerStats)]),
    "dkv_host_alloc": (I32, [SZ, C.c_uint32, C.POINTER(P), C.POINTER(P)]),
    "dkv_host_free": (I32, [P]),
    "dkv_set_tuning": (I32, [C.POINTER(Tuning)]),
    "dkv_get_tuning": (I32, [C.POINTER(Tuning)]),
    "dkv_probe_read": (I32, [P, P, SZ, I32, I32, I32, P, P, C.POINTER(BwResult), P]),
    "dkv_kernel_timing": (I32, [I32]),
    "dkv_kernel_timing_read": (I32, [I32, C.POINTER(I32), C.POINTER(F64)]),
    "dkv_attn_trace": (I32, [P, I32]),
    "dkv_prefill_plan": (I32, [C.POINTER(KvDesc), I32, I32, P, P, P, F64, C.POINTER(PlanInfo)]),
    "dkv_plan_cache_release_captured": (I32, []),
    "dkv_plan_cache_stats": (I32, [C.POINTER(I32), C.POINTER(I32), C.POINTER(I64)]),
    "dkv_prefill_attn_split": (I32, [C.POINTER(KvDesc), I32, I32, P, P, P, P, F64, F32, F64, P, SZ, P, P,
                                     P, I32, P]),
}

DKV_KERNEL_ATTN = 0
DKV_KERNEL_ROPE_Q = 1
DKV_KERNEL_MERGE = 2
DKV_KERNEL_APPEND = 3
DKV_KERNEL_PREFILL = 4
DKV_KERNEL_STAGE = 5
DKV_KERNEL_LINEAR = 6
DKV_KERNEL_TIERS = 7

_lib = None


def lib():
    """The loaded library (raises if libdkv.so is missing)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with `python -m decode_attention_host_amd.build` "
                "(the attention path has no fallback)")
        L = C.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def check(status: int):
    if status != DKV_OK:
        msg = lib().dkv_last_error()
        raise DkvError(status, msg.decode() if msg else "")
