"""ctypes declarations of libdak.so (include/dak.h).  Argument marshalling only."""
from __future__ import annotations

import ctypes as C
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libdak.so")

DAK_OK = 0
DAK_EINVAL = -1
DAK_EINFEASIBLE = -2
DAK_EHIP = -3
DAK_EUNSUPPORTED = -4
DAK_FLAG_COUNT_BYTES = 1
DAK_FLAG_STAGED_HOST = 2
DAK_FLAG_RECORD_XCC = 4
ABI_VERSION = 3


class OpDesc(C.Structure):
    _fields_ = [("units", C.c_uint64), ("unit_bytes", C.c_uint64), ("t_comp_s", C.c_double)]


class LaunchCfg(C.Structure):
    _fields_ = [("host_cus", C.c_int32), ("window", C.c_int32), ("flags", C.c_int32),
                ("reserved", C.c_int32), ("byte_counters", C.c_void_p)]


class SplitMatrixDesc(C.Structure):
    _fields_ = [("host", C.c_void_p), ("hbm", C.c_void_p), ("M", C.c_int64), ("K", C.c_int64),
                ("m", C.c_int32), ("reserved", C.c_int32), ("h", C.c_int64)]


class SplitMatrixFP8Desc(C.Structure):
    _fields_ = [("host", C.c_void_p), ("hbm", C.c_void_p), ("M", C.c_int64), ("K", C.c_int64),
                ("m", C.c_int32), ("reserved", C.c_int32), ("h", C.c_int64), ("row_scale", C.c_void_p)]


class SplitKVDesc(C.Structure):
    _fields_ = [("k_host", C.c_void_p), ("v_host", C.c_void_p), ("k_hbm", C.c_void_p), ("v_hbm", C.c_void_p),
                ("batch", C.c_int64), ("h", C.c_int64), ("n_kv_heads", C.c_int32), ("head_dim", C.c_int32),
                ("ctx", C.c_int64), ("unit", C.c_int32), ("reserved", C.c_int32), ("ctx_lens", C.c_void_p)]


class PagedKVDesc(C.Structure):
    _fields_ = [("k_host", C.c_void_p), ("v_host", C.c_void_p), ("k_hbm", C.c_void_p), ("v_hbm", C.c_void_p),
                ("host_pages", C.c_int64), ("hbm_pages", C.c_int64), ("batch", C.c_int64),
                ("n_kv_heads", C.c_int32), ("head_dim", C.c_int32), ("page", C.c_int32), ("max_pages", C.c_int32),
                ("page_table", C.c_void_p), ("ctx_lens", C.c_void_p), ("unit_order", C.c_void_p),
                ("n_host_units", C.c_int64)]


# (name, restype, argtypes) for every symbol include/dak.h declares.
SIGNATURES = [
    ("dak_last_error", C.c_char_p, []),
    ("dak_last_hip_error", C.c_int32, []),
    ("dak_abi_version", C.c_int32, []),
    ("dak_min_offload_ratio", C.c_double, [C.c_uint64, C.c_uint64]),
    ("dak_plan_offload", C.c_int32, [C.POINTER(OpDesc), C.c_size_t, C.c_double, C.c_double, C.c_double,
                                     C.POINTER(C.c_uint64), C.POINTER(C.c_double)]),
    ("dak_op_time", C.c_int32, [C.POINTER(OpDesc), C.c_uint64, C.c_double, C.c_double, C.POINTER(C.c_double)]),
    ("dak_plan_uniform", C.c_int32, [C.POINTER(OpDesc), C.c_size_t, C.c_double, C.c_double, C.c_double,
                                     C.POINTER(C.c_uint64), C.POINTER(C.c_double)]),
    ("dak_op_turning_points", C.c_int32, [C.POINTER(OpDesc), C.c_double, C.c_double, C.POINTER(C.c_uint64),
                                          C.POINTER(C.c_uint64), C.POINTER(C.c_int32)]),
    ("dak_host_workgroups", C.c_int64, [C.c_int64, C.c_int32]),
    ("dak_splitk_gemm", C.c_int32, [C.POINTER(SplitMatrixDesc), C.c_void_p, C.c_int64, C.c_void_p,
                                    C.POINTER(LaunchCfg), C.c_void_p]),
    ("dak_splitk_gemm_fp8", C.c_int32, [C.POINTER(SplitMatrixFP8Desc), C.c_void_p, C.c_int64, C.c_void_p,
                                        C.POINTER(LaunchCfg), C.c_void_p]),
    ("dak_splitk_gemm_workspace_bytes", C.c_uint64, [C.c_int64, C.c_int64, C.c_int64]),
    ("dak_splitk_gemm_ws", C.c_int32, [C.POINTER(SplitMatrixDesc), C.c_void_p, C.c_int64, C.c_void_p, C.c_void_p,
                                       C.c_uint64, C.POINTER(LaunchCfg), C.c_void_p]),
    ("dak_splitk_gemm_fp8_workspace_bytes", C.c_uint64, [C.c_int64, C.c_int64, C.c_int64]),
    ("dak_splitk_gemm_fp8_ws", C.c_int32, [C.POINTER(SplitMatrixFP8Desc), C.c_void_p, C.c_int64, C.c_void_p,
                                           C.c_void_p, C.c_uint64, C.POINTER(LaunchCfg), C.c_void_p]),
    ("dak_decode_attn_workspace_bytes", C.c_size_t, [C.POINTER(SplitKVDesc), C.c_int32]),
    ("dak_splitk_decode_attn", C.c_int32, [C.c_void_p, C.POINTER(SplitKVDesc), C.c_int32, C.c_float, C.c_void_p,
                                           C.c_void_p, C.c_size_t, C.POINTER(LaunchCfg), C.c_void_p]),
    ("dak_splitk_decode_attn_noalloc", C.c_int32, [C.c_void_p, C.POINTER(SplitKVDesc), C.c_int32, C.c_float,
                                                   C.c_void_p, C.POINTER(LaunchCfg), C.c_void_p]),
    ("dak_decode_attn_scratch_max_bytes", C.c_size_t, []),
    ("dak_paged_decode_attn_workspace_bytes", C.c_size_t, [C.POINTER(PagedKVDesc), C.c_int32]),
    ("dak_paged_decode_attn", C.c_int32, [C.c_void_p, C.POINTER(PagedKVDesc), C.c_int32, C.c_float, C.c_void_p,
                                          C.c_void_p, C.c_size_t, C.POINTER(LaunchCfg), C.c_void_p]),
    ("dak_probe_read", C.c_int32, [C.c_void_p, C.c_size_t, C.c_int32, C.c_int32, C.c_int32, C.c_void_p,
                                   C.POINTER(C.c_float)]),
    ("dak_probe_read_concurrent", C.c_int32, [C.c_void_p, C.c_size_t, C.c_int32, C.c_int32, C.c_void_p,
                                              C.c_size_t, C.c_int32, C.c_int32, C.c_void_p,
                                              C.POINTER(C.c_float), C.POINTER(C.c_float), C.POINTER(C.c_float)]),
    ("dak_probe_copy_interference", C.c_int32, [C.c_void_p, C.c_size_t, C.c_int32, C.c_int32, C.c_void_p,
                                                C.c_void_p, C.c_size_t, C.c_int32, C.c_void_p, C.c_void_p,
                                                C.POINTER(C.c_float), C.POINTER(C.c_float), C.POINTER(C.c_float),
                                                C.POINTER(C.c_int32)]),
    ("dak_probe_mfma", C.c_int32, [C.c_int32, C.c_int64, C.c_int32, C.c_void_p, C.POINTER(C.c_float),
                                   C.POINTER(C.c_double)]),
]

_lib = None


def load(path: str = LIB_PATH) -> C.CDLL:
    """Load libdak.so; raises if it has not been built (there is no fallback)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with "
                           "`python -m tiered_memory_offloading_amd.build` (no CPU fallback exists)")
    lib = C.CDLL(path)
    for name, res, args in SIGNATURES:
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    if lib.dak_abi_version() != ABI_VERSION:
        raise RuntimeError("libdak.so ABI version mismatch; rebuild it")
    _lib = lib
    return lib
